"""vlb_bridge_fused_noalloc: the fused call with the library's own device
scratch instead of a workspace argument, for callers that cannot allocate.

Each call's output must equal vlb_bridge_fused's (the same projector, the same
inputs) bit for bit -- that entry point is held against the oracle by the
parity tests.  Two calls in a row, the second on a smaller input, check that
the second does not depend on what the first left in the scratch; a
placeholder-count mismatch through the new entry point writes nothing and is
reported in its status words; a text-only batch writes zeros there.
"""
import numpy as np
import pytest
import torch

import common
from patch_merge_mlp_amd import vlbridge as v
from patch_merge_mlp_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev(x):
    return None if x is None else x.to(DEV)


def _inputs(w):
    t = common.draw(w)
    p, b = common.lib_projector(w), common.lib_batch(w)
    br = v.Bridge(p, v.Weights(*(_dev(t[n]) for n in ("w1", "b1", "w2", "b2", "ln_gamma",
                                                        "ln_beta"))))
    return t, br, b


def _fused(br, b, t):
    seq = _dev(t["seq"]).clone()
    ws = br.fused(b, _dev(t["features"]), _dev(t["newline"]), _dev(t["separator"]),
                  _dev(t["mask"]), seq)
    assert v.vlb_check(ws) == v.OK
    return seq.cpu()


def _noalloc(br, b, t, mask=None):
    g = common.Guards()  # guard bands around the outputs
    seq = g.like(t["seq"], "seq")
    status = g.empty((4,), torch.int32, "status")
    status.fill_(-7)
    v.vlb_bridge_fused_noalloc(br.p, b, _dev(t["features"]), br.w, _dev(t["newline"]),
                               _dev(t["separator"]), _dev(t["mask"] if mask is None else mask),
                               seq, status)
    st = v.vlb_check(status)
    g.check()
    return st, seq.cpu(), status.cpu()


def _same(a, c):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       c.view(torch.int16) if c.dtype == torch.bfloat16 else c.view(torch.int32))


def test_noalloc_two_calls_match_fused():
    """The 3x3 workload at full size (4 images of 96 x 96 x 1024), then the small
    LayerNorm workload: each call gives vlb_bridge_fused's bits."""
    big = wl.config(2)
    small = wl.Workload("small-2x2-ln", 11, "bf16", C=128, k=2, hidden=320, out_dim=192,
                        seq_len=800, grids=[(34, 34), (17, 20), (9, 31)],
                        views_per_image=[1, 1, 1], has_ln=True)
    for w in (big, small):
        t, br, b = _inputs(w)
        want = _fused(br, b, t)
        st, got, status = _noalloc(br, b, t)
        print(w.name, "status", status.tolist(), flush=True)
        assert st == v.OK
        assert status[1].item() == v.vlb_num_slots(br.p, b)
        assert _same(got, want), w.name


def test_noalloc_tiled_and_fp32():
    """A tiled batch (newline and separator rows) and the fp32 workload, after the
    calls above left other contents in the scratch."""
    tiled = wl.Workload("small-tiled", 13, "bf16", C=128, k=2, hidden=192, out_dim=128,
                        seq_len=700, grids=[(13, 13)] * 10, views_per_image=[7, 3], tiled=True,
                        tiles=[(2, 3), (1, 2)])
    for w in (tiled, wl.config(0)):
        t, br, b = _inputs(w)
        want = _fused(br, b, t)
        st, got, _ = _noalloc(br, b, t)
        assert st == v.OK
        assert _same(got, want), w.name


def test_noalloc_count_mismatch_and_text_only():
    w = wl.Workload("small-3x3", 12, "bf16", C=64, k=3, hidden=256, out_dim=320, seq_len=700,
                    grids=[(48, 48), (50, 47)], views_per_image=[1, 1])
    t, br, b = _inputs(w)
    mask = t["mask"].clone()
    mask[int(np.flatnonzero(mask.numpy())[-1])] = 0
    st, got, _ = _noalloc(br, b, t, mask=mask)
    assert st == v.ERR_MASK_COUNT
    assert _same(got, t["seq"])
    st, got, status = _noalloc(br, v.Batch([], []), t, mask=torch.zeros_like(t["mask"]))
    assert st == v.OK and status.tolist() == [0, 0, 0, 0]
    assert _same(got, t["seq"])
    st, got, _ = _noalloc(br, b, t)  # and a good call afterwards
    assert st == v.OK
    assert _same(got, _fused(br, b, t))
