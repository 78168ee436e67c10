"""Helpers shared by the tests: oracle specs and library batches built from one
workload description, and the error metrics."""
from __future__ import annotations

import numpy as np

from oracle import oracle as o
from patch_merge_mlp_amd import vlbridge as v
from patch_merge_mlp_amd import workloads as wl


def oracle_spec(w: wl.Workload, act=o.GELU_ERF) -> o.Spec:
    return o.Spec(grids=w.grids, C=w.C, k=w.k, hidden=w.hidden, out_dim=w.out_dim,
                  views_per_image=w.views_per_image, has_ln=w.has_ln, ln_eps=w.ln_eps, act=act,
                  tiled=w.tiled, tiles=w.tiles, global_tail=w.global_tail)


def oracle_spans(w: wl.Workload):
    """Placeholder slots per image from the oracle's own assembly."""
    spec = oracle_spec(w)
    src = o.assemble(spec)
    out, v = [], 0
    for im, nv in enumerate(w.views_per_image):
        views = w.grids[v:v + nv]
        sub = o.Spec(grids=views, C=1, k=w.k, hidden=1, out_dim=1, views_per_image=[nv],
                     tiled=w.tiled, tiles=[w.tiles[im]] if w.tiled else (),
                     global_tail=w.global_tail)
        out.append(len(o.assemble(sub)))
        v += nv
    assert sum(out) == len(src)
    return out


def draw(w: wl.Workload) -> dict:
    """Seeded inputs of workload w (spans and merged width from the oracle)."""
    return wl.make(w, oracle_spans, lambda ww: ww.C * ww.k * ww.k)


def lib_projector(w: wl.Workload, act=v.GELU_ERF, has_ln=None, gather=False) -> v.vlb_projector:
    return v.projector(v.F32 if w.dtype == "f32" else v.BF16, w.C, w.k, w.hidden, w.out_dim,
                       has_ln=w.has_ln if has_ln is None else has_ln, ln_eps=w.ln_eps, act=act,
                       gather=gather)


def lib_batch(w: wl.Workload) -> v.Batch:
    return v.Batch(w.grids, w.views_per_image,
                   v.LAYOUT_TILED_2D if w.tiled else v.LAYOUT_PLAIN, w.tiles or None,
                   w.global_tail)


def image_row_ranges(w: wl.Workload):
    """Token-row range [r0, r1) of every image."""
    out, r, v = [], 0, 0
    for nv in w.views_per_image:
        n = sum(o.view_tokens(gh, gw, w.k) for gh, gw in w.grids[v:v + nv])
        out.append((r, r + n))
        r += n
        v += nv
    return out


def rel_frob(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))
