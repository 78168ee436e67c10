"""Seeded random shapes through the C ABI against the fp64 oracle.

The other GPU tests pick their shapes by hand; here each case draws its own
from a fixed seed: dtype, channels, merge factor, widths, LayerNorm, the
activation, plain or tiled layout (head or tail), grids with ragged edges,
images and views, and -- for the forward -- packed or unpacked weights and
the source of Linear1's operand.  Token counts stay small enough for the
oracle to finish in well under a second per case.

  * forward (vlb_bridge_fused): every projected row against the oracle (per
    image, per row and per element, the bounds of the full-size tests), every
    text row and every newline / separator row bit for bit;
  * backward (vlb_bridge_fused_train + vlb_bridge_backward): every gradient
    against the oracle's, with the bounds of the small backward tests.
"""
import random

import numpy as np
import pytest
import torch

import common
from oracle import oracle as o
from patch_merge_mlp_amd import vlbridge as v
from patch_merge_mlp_amd import workloads as wl
from test_gpu_backward import TOL_ACT, TOL_F32, TOL_SUM, _np, oracle_grads, run_train
from test_gpu_parity import ELEM_TOL, ROW_TOL, TOL, check_text_rows, run_fused, slot_positions

pytestmark = pytest.mark.gpu

N_FORWARD, N_BACKWARD = 24, 8
MAX_TOKENS = {False: 1500, True: 500}   # forward / backward


def random_workload(case: int, backward: bool) -> wl.Workload:
    """Shapes of one case, drawn from its own seed (the values come later, from
    the workload's seeded generator)."""
    r = random.Random((20000 if backward else 10000) + case)
    # the last backward case is fp32 whatever the draw
    dtype = "f32" if (r.random() < 0.15 or (backward and case == N_BACKWARD - 1)) else "bf16"
    k = r.choice([1, 2, 3])
    if dtype == "bf16":
        C = 64 * r.randint(1, 8 if backward else 16)
        hidden = 64 * r.randint(1, 6 if backward else 12)
        out_dim = 8 * r.randint(1, 40 if backward else 80)
    else:
        C, hidden, out_dim = (8 * r.randint(1, 16) for _ in range(3))
    has_ln = r.random() < 0.4
    tiled = r.random() < 0.3
    while True:
        if tiled:
            tiles = [(r.randint(1, 3), r.randint(1, 3)) for _ in range(r.randint(1, 3))]
            grids, vpi = [], []
            for tw, th in tiles:  # every view of an image has the image's grid
                g = r.randint(2, 16)
                grids += [(g, g)] * (1 + tw * th)
                vpi.append(1 + tw * th)
        else:
            tiles = []
            vpi = [r.randint(1, 3) for _ in range(r.randint(1, 4))]
            side = 40 if k > 1 else 20
            grids = [(r.randint(1, side), r.randint(1, side)) for _ in range(sum(vpi))]
        T = sum(o.view_tokens(gh, gw, k) for gh, gw in grids)
        if T <= MAX_TOKENS[backward]:
            break
    w = wl.Workload(f"{'bwd' if backward else 'fwd'}-{case}", 500 + case + (100 if backward else 0),
                    dtype, C=C, k=k, hidden=hidden, out_dim=out_dim, seq_len=0, grids=grids,
                    views_per_image=vpi, has_ln=has_ln, tiled=tiled, tiles=tiles,
                    global_tail=tiled and r.random() < 0.5)
    w.seq_len = sum(common.oracle_spans(w)) + r.randint(0, 300)
    return w


def describe(w):
    return (f"{w.name}: {w.dtype} C={w.C} k={w.k} {w.C * w.k * w.k}->{w.hidden}->{w.out_dim} "
            f"ln={w.has_ln} {'tiled ' + str(w.tiles) if w.tiled else 'plain'}"
            f"{' tail' if w.global_tail else ''} views={len(w.grids)} S={w.seq_len}")


@pytest.mark.parametrize("case", range(N_FORWARD))
def test_random_shapes_forward(case):
    w = random_workload(case, backward=False)
    r = random.Random(30000 + case)
    act = r.choice([v.GELU_ERF, v.GELU_TANH, v.ACT_NONE])
    bf16 = w.dtype == "bf16"
    pack = bf16 and r.random() < 0.7
    gather = r.choice([v.GATHER_AUTO, v.GATHER_ON, v.GATHER_OFF]) if bf16 and not w.has_ln \
        else v.GATHER_AUTO
    print(describe(w), "act", act, "pack", pack, "gather", gather, flush=True)
    t = common.draw(w)
    spec = common.oracle_spec(w, act)
    ref_rows = o.project_rows(spec, t["features"], t["ln_gamma"], t["ln_beta"], t["w1"], t["b1"],
                              t["w2"], t["b2"])
    st, out = run_fused(w, t, act=act, pack=pack, gather=gather)
    assert st == v.OK
    check_text_rows(t, out)
    src = o.assemble(spec)
    pos = slot_positions(t)
    tok = src >= 0
    got = out[torch.from_numpy(pos[tok])].double().numpy()
    rows = src[tok]
    ref = ref_rows[rows]
    assert len(np.unique(rows)) == len(ref_rows), "some projected row has no slot"
    rnorm = np.linalg.norm(ref, axis=1)
    per_row = np.linalg.norm(got - ref, axis=1) / np.where(rnorm > 0, rnorm, 1.0)
    rms = np.where(rnorm > 0, rnorm, 1.0) / np.sqrt(w.out_dim)
    per_elem = (np.abs(got - ref) / rms[:, None]).max(axis=1)
    worst_img = max(common.rel_frob(got[(rows >= r0) & (rows < r1)], ref[(rows >= r0) & (rows < r1)])
                    for r0, r1 in common.image_row_ranges(w))
    print(f"  max per-image {worst_img:.2e}, per-row {per_row.max():.2e}, "
          f"element / row rms {per_elem.max():.2e}")
    assert worst_img <= TOL[w.dtype], worst_img
    assert per_row.max() <= ROW_TOL[w.dtype], per_row.max()
    assert per_elem.max() <= ELEM_TOL[w.dtype], per_elem.max()
    if w.tiled:  # newline and separator rows are copies of the vectors
        extra = pos[~tok]
        want = np.where((src[~tok] == -1)[:, None], t["newline"].double().numpy()[None, :],
                        t["separator"].double().numpy()[None, :])
        assert np.array_equal(out[torch.from_numpy(extra)].double().numpy(), want)


@pytest.mark.parametrize("case", range(N_BACKWARD))
def test_random_shapes_backward(case):
    w = random_workload(case, backward=True)
    print(describe(w), flush=True)
    t = common.draw(w)
    dseq = wl.seq_grad(w)
    st, _, g, _ = run_train(w, t, dseq)
    assert st == v.OK
    ref = oracle_grads(w, t, dseq)
    errs = {
        "dw1": common.rel_frob(_np(g.d_w1), ref["dw1"]),
        "db1": common.rel_frob(_np(g.d_b1), ref["db1"]),
        "dw2": common.rel_frob(_np(g.d_w2), ref["dw2"]),
        "dx": common.rel_frob(_np(g.d_features), ref["dx"]),
        "db2": common.rel_frob(_np(g.d_b2), ref["db2"]),
    }
    if w.has_ln:
        errs["dgamma"] = common.rel_frob(_np(g.d_ln_gamma), ref["dgamma"])
        errs["dbeta"] = common.rel_frob(_np(g.d_ln_beta), ref["dbeta"])
    if w.tiled:
        errs["d_newline"] = common.rel_frob(_np(g.d_newline), ref["d_newline"])
        errs["d_separator"] = common.rel_frob(_np(g.d_separator), ref["d_separator"])
    print("  ", {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        if w.dtype == "f32":
            tol = TOL_F32
        else:
            tol = TOL_SUM if k in ("db2", "d_newline", "d_separator") else TOL_ACT
        assert e <= tol, (k, e)
