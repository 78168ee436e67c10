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


# ---- guard bands around device outputs -------------------------------------------

GUARD_BYTES = 4096   # canary bytes before and after every guarded buffer
CANARY = 0xA5


class Guards:
    """Device buffers with GUARD_BYTES of canary bytes on both sides.  check()
    asserts that every canary byte is intact: a kernel that writes past an
    output or past the workspace it was sized for changes them.  The buffers
    stay 256-byte aligned (the canaries are a multiple of 256 bytes)."""

    def __init__(self):
        self.bufs = []

    def empty(self, shape, dtype, label="buffer", device="cuda"):
        import torch
        shape = tuple(shape) if isinstance(shape, (tuple, list)) else (int(shape),)
        es = torch.empty(0, dtype=dtype).element_size()
        n = 1
        for d in shape:
            n *= int(d)
        g = GUARD_BYTES // es
        raw = torch.full(((n + 2 * g) * es,), CANARY, dtype=torch.uint8, device=device)
        inner = raw.view(dtype)[g:g + n].view(shape)
        self.bufs.append((raw, n * es, label))
        return inner

    def like(self, t, label="buffer"):
        x = self.empty(t.shape, t.dtype, label, device="cuda")
        x.copy_(t.to(x.device))
        return x

    def workspace(self, nbytes, label="workspace"):
        import torch
        return self.empty((max(int(nbytes), 16),), torch.uint8, label)

    def check(self):
        for raw, nb, label in self.bufs:
            head = raw[:GUARD_BYTES]
            tail = raw[GUARD_BYTES + nb:]
            assert bool((head == CANARY).all()), f"{label}: bytes before it were written"
            assert bool((tail == CANARY).all()), f"{label}: bytes after it were written"
