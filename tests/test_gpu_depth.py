"""Projectors deeper than two Linears ([VL2] Projector 3: extra activation +
Linear(hidden -> hidden) pairs in the middle) against the oracle.

Small workloads: every projected row, per-image relative Frobenius error <= 1e-2
(bf16) / 1e-5 (fp32), packed and unpacked weights; workload 1 at full size with
depth 3: sampled rows; the unfused entry points give the fused call's bits.
"""
import numpy as np
import pytest
import torch

import common
from oracle import oracle as o
from patch_merge_mlp_amd import vlbridge as v
from patch_merge_mlp_amd import workloads as wl
from test_gpu_parity import (TOL, _dev, _sample_rows, check_text_rows, full, per_image_errors,
                             slot_positions, small_workloads)

pytestmark = pytest.mark.gpu


def deep_setup(w, t, depth, pack=True):
    mids = wl.mid_weights(w, depth)
    p = common.lib_projector(w)
    p.depth = depth
    weights = v.Weights(*(_dev(t[n]) for n in ("w1", "b1", "w2", "b2", "ln_gamma", "ln_beta")),
                        w_mid=[_dev(a) for a, _ in mids], b_mid=[_dev(b) for _, b in mids])
    return v.Bridge(p, weights, pack=pack), mids


def run_deep(w, t, depth, pack=True):
    br, mids = deep_setup(w, t, depth, pack)
    b = common.lib_batch(w)
    seq = _dev(t["seq"]).clone()
    ws = br.fused(b, _dev(t["features"]), _dev(t["newline"]), _dev(t["separator"]),
                  _dev(t["mask"]), seq)
    return v.vlb_check(ws), seq.cpu(), mids


def oracle_deep_rows(w, t, depth, mids, row_ids=None):
    spec = common.oracle_spec(w)
    spec.depth = depth
    return o.project_rows_deep(spec, t["features"], t["ln_gamma"], t["ln_beta"], t["w1"], t["b1"],
                               [a for a, _ in mids], [b for _, b in mids], t["w2"], t["b2"],
                               row_ids=row_ids)


CASES = [(0, 3), (0, 4), (1, 3), (2, 3), (5, 3), (5, 4)]


@pytest.mark.parametrize("wi,depth", CASES, ids=[f"{small_workloads()[i].name}-d{d}" for i, d in CASES])
def test_small_deep_vs_oracle(wi, depth):
    w = small_workloads()[wi]
    t = common.draw(w)
    for pack in (True, False) if w.dtype == "bf16" else (True,):
        st, out, mids = run_deep(w, t, depth, pack)
        assert st == v.OK
        check_text_rows(t, out)
        rows = oracle_deep_rows(w, t, depth, mids)
        st2, ref = o.scatter(o.assemble(common.oracle_spec(w)), rows, t["newline"], t["separator"],
                             t["mask"].numpy(), t["seq"])
        assert st2 == 0
        errs = per_image_errors(w, t, out.double().numpy(), ref)
        print(w.name, depth, "pack" if pack else "nopack", max(errs))
        assert max(errs) <= TOL[w.dtype], errs


def test_full_deep_sampled_rows():
    w, t = full(1)
    depth = 3
    st, out, mids = run_deep(w, t, depth)
    assert st == v.OK
    check_text_rows(t, out)
    rows = _sample_rows(w, per_image=2)
    ref = oracle_deep_rows(w, t, depth, mids, row_ids=rows)
    src = o.assemble(common.oracle_spec(w))
    slot_of_row = np.empty(len(src), dtype=np.int64)
    tok = src >= 0
    slot_of_row[src[tok]] = np.flatnonzero(tok)
    got = out.double().numpy()[slot_positions(t)[slot_of_row[rows]]]
    worst = 0.0
    for r0, r1 in common.image_row_ranges(w):
        sel = (rows >= r0) & (rows < r1)
        worst = max(worst, common.rel_frob(got[sel], ref[sel]))
    print(w.name, "depth", depth, "sampled rows", len(rows), "max per-image rel err", worst)
    assert worst <= TOL[w.dtype]


def test_deep_unfused_equals_fused():
    w = small_workloads()[2]
    t = common.draw(w)
    st, fused, _ = run_deep(w, t, 4)
    assert st == v.OK
    br, _ = deep_setup(w, t, 4)
    b = common.lib_batch(w)
    rows = br.project(b, _dev(t["features"]))
    seq = _dev(t["seq"]).clone()
    ws = v.workspace(br.p, b, seq.shape[0])
    v.vlb_scatter_tokens(br.p, b, rows, _dev(t["newline"]), _dev(t["separator"]),
                         _dev(t["mask"]), seq, ws)
    assert v.vlb_check(ws) == v.OK
    assert torch.equal(seq.cpu().view(torch.int16), fused.view(torch.int16))
