"""The projector backward (vlb_bridge_fused_train + vlb_bridge_backward) against
the fp64 oracle's gradients.

  * small workloads (LayerNorm / none, k = 1, 2, 3, plain and tiled head / tail):
    every gradient against the oracle -- relative Frobenius error <= 1e-2 for
    the gradients that pass through bf16-rounded activations (dW1, db1, dW2,
    dgamma, dbeta, the features), <= 1e-5 for the plain sums of bf16 gradient
    rows (db2, newline, separator);
  * the four bf16 workloads at full size, in the benchmark's launch configuration:
    db2, newline and separator gradients whole; sampled hidden units (row of
    dW1, db1 entry, column of dW2) and sampled pixels (feature gradient);
  * the training forward writes the same sequence as vlb_bridge_fused, and two
    backward runs give the same bits;
  * a placeholder-count mismatch writes no gradient; no images: zero gradients.
"""
import numpy as np
import pytest
import torch

import common
from oracle import oracle as o
from patch_merge_mlp_amd import vlbridge as v
from patch_merge_mlp_amd import workloads as wl
from test_gpu_parity import _dev, _weights, full, run_fused, small_workloads

pytestmark = pytest.mark.gpu
TOL_ACT = 1e-2   # through bf16 activations (Z1, act(Z1), dA1, dZ1, dXm rounded)
TOL_SUM = 1e-5   # fp32 sums of bf16 gradient rows


def run_train(w, t, dseq, features_grad=True, mask=None):
    """Training forward then backward on the device; returns (status, seq, grads, ws)."""
    p, b = common.lib_projector(w), common.lib_batch(w)
    wt = _weights(t)
    gd = common.Guards()  # guard bands around every output, workspace and saved buffer
    seq = gd.like(t["seq"], "seq")
    mask = _dev(t["mask"] if mask is None else mask)
    fws = gd.workspace(v.vlb_workspace_bytes(p, b, seq.shape[0]), "forward workspace")
    saved = gd.workspace(v.vlb_saved_bytes(p, b), "saved activations")
    v.vlb_bridge_fused_train(p, b, _dev(t["features"]), wt, _dev(t["newline"]),
                             _dev(t["separator"]), mask, seq, saved, fws)
    g = v.Grads.empty(p, b, features=features_grad)
    for name in ("d_w1", "d_b1", "d_w2", "d_b2", "d_features", "d_ln_gamma", "d_ln_beta",
                 "d_newline", "d_separator"):
        x = getattr(g, name)
        if x is not None:
            x = gd.empty(x.shape, x.dtype, name)
            if x.dtype == torch.float32:
                x.fill_(float("nan"))
            setattr(g, name, x)
    bws = gd.workspace(v.vlb_backward_workspace_bytes(p, b, seq.shape[0]), "backward workspace")
    v.vlb_bridge_backward(p, b, _dev(t["features"]), wt, mask, _dev(dseq), saved, g, bws)
    st = v.vlb_check(bws)
    gd.check()
    return st, seq.cpu(), g, bws


def oracle_grads(w, t, dseq):
    spec = common.oracle_spec(w)
    T = o.total_tokens(spec)
    st, drows, dnl, dsep = o.scatter_backward(o.assemble(spec), t["mask"].numpy(), dseq, T)
    assert st == 0
    ref = o.project_backward(spec, t["features"], t["ln_gamma"], t["ln_beta"], t["w1"], t["b1"],
                             t["w2"], drows)
    ref["d_newline"], ref["d_separator"], ref["drows"] = dnl, dsep, drows
    return ref


def _np(x):
    return x.detach().float().cpu().double().numpy()


BWD_SMALL = [small_workloads()[i] for i in (0, 1, 2, 3, 4)]
BWD_F32 = [small_workloads()[5], wl.config(0),
           wl.Workload("small-f32-ln-tiled", 17, "f32", C=32, k=2, hidden=48, out_dim=40,
                       seq_len=900, grids=[(9, 11)] * 7 + [(6, 6)] * 3, views_per_image=[7, 3],
                       has_ln=True, tiled=True, tiles=[(2, 3), (1, 2)])]
TOL_F32 = 1e-5   # fp32 throughout


@pytest.mark.parametrize("w", BWD_SMALL, ids=lambda w: w.name)
def test_small_backward_vs_oracle(w):
    t = common.draw(w)
    dseq = wl.seq_grad(w)
    st, seq, g, _ = run_train(w, t, dseq)
    assert st == v.OK
    st_f, seq_f = run_fused(w, t, pack=False)
    assert st_f == v.OK
    assert torch.equal(seq.view(torch.int16), seq_f.view(torch.int16)), "training forward differs"
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
    print(w.name, {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        tol = TOL_SUM if k in ("db2", "d_newline", "d_separator") else TOL_ACT
        assert e <= tol, (k, e)


@pytest.mark.parametrize("C", [768, 1152, 1280])
def test_layernorm_backward_channels(C):
    """The LayerNorm backward at the channel counts that take one dword per
    lane and step (6, 9 and 10 per lane), with a 9 x 10 grid whose last cells
    are padding: every gradient against the oracle."""
    w = wl.Workload(f"bwd-ln-{C}", 30 + C // 128, "bf16", C=C, k=2, hidden=256, out_dim=128,
                    seq_len=96, grids=[(9, 10), (4, 4)], views_per_image=[1, 1], has_ln=True)
    t = common.draw(w)
    dseq = wl.seq_grad(w)
    st, _, g, _ = run_train(w, t, dseq)
    assert st == v.OK
    ref = oracle_grads(w, t, dseq)
    errs = {"dx": common.rel_frob(_np(g.d_features), ref["dx"]),
            "dgamma": common.rel_frob(_np(g.d_ln_gamma), ref["dgamma"]),
            "dbeta": common.rel_frob(_np(g.d_ln_beta), ref["dbeta"]),
            "dw1": common.rel_frob(_np(g.d_w1), ref["dw1"])}
    print(w.name, {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        assert e <= TOL_ACT, (k, e)


@pytest.mark.parametrize("w", BWD_F32, ids=lambda w: w.name)
def test_small_backward_f32_vs_oracle(w):
    t = common.draw(w)
    dseq = wl.seq_grad(w)
    st, seq, g, _ = run_train(w, t, dseq)
    assert st == v.OK
    st_f, seq_f = run_fused(w, t)
    assert st_f == v.OK
    assert torch.equal(seq.view(torch.int32), seq_f.view(torch.int32)), "training forward differs"
    ref = oracle_grads(w, t, dseq)
    pairs = [("dw1", g.d_w1), ("db1", g.d_b1), ("dw2", g.d_w2), ("db2", g.d_b2),
             ("dx", g.d_features)]
    if w.has_ln:
        pairs += [("dgamma", g.d_ln_gamma), ("dbeta", g.d_ln_beta)]
    if w.tiled:
        pairs += [("d_newline", g.d_newline), ("d_separator", g.d_separator)]
    errs = {k: common.rel_frob(_np(x), ref[k]) for k, x in pairs}
    print(w.name, {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        assert e <= TOL_F32, (k, e)


@pytest.mark.parametrize("act", [v.GELU_TANH, v.ACT_NONE])
def test_small_backward_activations(act):
    w = small_workloads()[0]
    t = common.draw(w)
    dseq = wl.seq_grad(w)
    p, b = common.lib_projector(w, act), common.lib_batch(w)
    wt = _weights(t)
    seq = _dev(t["seq"]).clone()
    fws = torch.empty(v.vlb_workspace_bytes(p, b, seq.shape[0]), dtype=torch.uint8, device="cuda")
    saved = torch.empty(v.vlb_saved_bytes(p, b), dtype=torch.uint8, device="cuda")
    v.vlb_bridge_fused_train(p, b, _dev(t["features"]), wt, None, None, _dev(t["mask"]), seq,
                             saved, fws)
    g = v.Grads.empty(p, b)
    bws = torch.empty(v.vlb_backward_workspace_bytes(p, b, seq.shape[0]), dtype=torch.uint8,
                      device="cuda")
    v.vlb_bridge_backward(p, b, _dev(t["features"]), wt, _dev(t["mask"]), _dev(dseq), saved, g,
                          bws)
    assert v.vlb_check(bws) == v.OK
    spec = common.oracle_spec(w, act)
    T = o.total_tokens(spec)
    _, drows, _, _ = o.scatter_backward(o.assemble(spec), t["mask"].numpy(), dseq, T)
    ref = o.project_backward(spec, t["features"], t["ln_gamma"], t["ln_beta"], t["w1"], t["b1"],
                             t["w2"], drows)
    for name, got in (("dw1", g.d_w1), ("db1", g.d_b1), ("dw2", g.d_w2), ("dx", g.d_features),
                      ("dgamma", g.d_ln_gamma), ("dbeta", g.d_ln_beta)):
        e = common.rel_frob(_np(got), ref[name])
        assert e <= TOL_ACT, (act, name, e)


@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_full_backward_sampled(i):
    w, t = full(i)
    dseq = wl.seq_grad(w)
    st, _, g, _ = run_train(w, t, dseq)
    assert st == v.OK
    spec = common.oracle_spec(w)
    T = o.total_tokens(spec)
    st, drows, dnl, dsep = o.scatter_backward(o.assemble(spec), t["mask"].numpy(), dseq, T)
    assert st == 0
    assert common.rel_frob(_np(g.d_b2), drows.sum(axis=0)) <= TOL_SUM
    if w.tiled:
        assert common.rel_frob(_np(g.d_newline), dnl) <= TOL_SUM
        assert common.rel_frob(_np(g.d_separator), dsep) <= TOL_SUM
    # fp64 copies made once (each oracle call would otherwise widen them again)
    args = tuple(None if a is None else o._f64(a)
                 for a in (t["features"], t["ln_gamma"], t["ln_beta"], t["w1"], t["b1"], t["w2"]))
    args = args + (drows,)
    rng = np.random.default_rng(i)
    units = sorted({0, w.hidden - 1, *rng.integers(0, w.hidden, 3).tolist()})
    dw1, db1, dw2 = _np(g.d_w1), _np(g.d_b1), _np(g.d_w2)
    got_b1, want_b1 = [], []
    for h in units:
        r_w1, r_b1, r_w2 = o.hidden_unit_grads(spec, *args, int(h))
        e1, e2 = common.rel_frob(dw1[h], r_w1), common.rel_frob(dw2[:, h], r_w2)
        print(w.name, "unit", h, f"dw1 {e1:.2e} dw2 {e2:.2e}")
        assert e1 <= TOL_ACT and e2 <= TOL_ACT, (h, e1, e2)
        got_b1.append(db1[h])
        want_b1.append(r_b1)
    eb = common.rel_frob(np.array(got_b1), np.array(want_b1))
    print(w.name, "db1 at units", f"{eb:.2e}")
    assert eb <= TOL_ACT
    dx = g.d_features.float().cpu().double().numpy()
    pix0 = np.cumsum([0] + [gh * gw for gh, gw in w.grids])
    picks = [(0, 0, 0), (len(w.grids) - 1, w.grids[-1][0] - 1, w.grids[-1][1] - 1)]
    for _ in range(4):
        vv = int(rng.integers(0, len(w.grids)))
        picks.append((vv, int(rng.integers(0, w.grids[vv][0])), int(rng.integers(0, w.grids[vv][1]))))
    got, want = [], []
    for vv, y, xx in picks:
        want.append(o.pixel_grad(spec, *args, vv, y, xx))
        got.append(dx[pix0[vv] + y * w.grids[vv][1] + xx])
    e = common.rel_frob(np.array(got), np.array(want))
    print(w.name, "pixels", picks, f"dx {e:.2e}")
    assert e <= TOL_ACT


def test_full_backward_repeatable():
    """Workload 1's weight gradients split their tail tiles along K (dW2 into
    8 ranges, dW1 into 3) and add the partial tiles in range order: two runs
    give the same bits, as do the other gradients."""
    w, t = full(1)
    dseq = wl.seq_grad(w)
    st1, _, g1, _ = run_train(w, t, dseq)
    st2, _, g2, _ = run_train(w, t, dseq)
    assert st1 == v.OK and st2 == v.OK
    for name in ("d_w1", "d_w2", "d_b1", "d_b2", "d_ln_gamma", "d_ln_beta", "d_features"):
        a, b = getattr(g1, name), getattr(g2, name)
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)), name


@pytest.mark.parametrize("wi", [0, 2])
def test_backward_packed_equals_unpacked(wi):
    """With weights packed by vlb_pack_weights the backward gives the same bits."""
    w = small_workloads()[wi]
    t = common.draw(w)
    dseq = wl.seq_grad(w)
    _, _, g_ref, _ = run_train(w, t, dseq)
    p, b = common.lib_projector(w), common.lib_batch(w)
    br = v.Bridge(p, _weights(t))  # packs W1 and W2
    seq = _dev(t["seq"]).clone()
    mask = _dev(t["mask"])
    fws = torch.empty(v.vlb_workspace_bytes(br.p, b, seq.shape[0]), dtype=torch.uint8, device="cuda")
    saved = torch.empty(v.vlb_saved_bytes(br.p, b), dtype=torch.uint8, device="cuda")
    v.vlb_bridge_fused_train(br.p, b, _dev(t["features"]), br.w, _dev(t["newline"]),
                             _dev(t["separator"]), mask, seq, saved, fws)
    g = v.Grads.empty(br.p, b)
    bws = torch.empty(v.vlb_backward_workspace_bytes(br.p, b, seq.shape[0]), dtype=torch.uint8,
                      device="cuda")
    v.vlb_bridge_backward(br.p, b, _dev(t["features"]), br.w, mask, _dev(dseq), saved, g, bws)
    assert v.vlb_check(bws) == v.OK
    for name in ("d_w1", "d_b1", "d_w2", "d_b2", "d_features", "d_ln_gamma", "d_ln_beta",
                 "d_newline", "d_separator"):
        a_, b_ = getattr(g, name), getattr(g_ref, name)
        if b_ is None:
            continue
        view = torch.int16 if a_.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a_.view(view), b_.view(view)), name


DEEP_CASES = [(0, 3), (0, 4), (2, 3), (5, 3), (5, 4)]


@pytest.mark.parametrize("wi,depth", DEEP_CASES,
                         ids=[f"{small_workloads()[i].name}-d{d}" for i, d in DEEP_CASES])
def test_small_backward_deep_vs_oracle(wi, depth):
    """Depth 3 and 4: every gradient, the middle Linears' included, against the oracle."""
    w = small_workloads()[wi]
    t = common.draw(w)
    dseq = wl.seq_grad(w)
    mids = wl.mid_weights(w, depth)
    p, b = common.lib_projector(w), common.lib_batch(w)
    p.depth = depth
    wt = v.Weights(*(_dev(t[n]) for n in ("w1", "b1", "w2", "b2", "ln_gamma", "ln_beta")),
                   w_mid=[_dev(a) for a, _ in mids], b_mid=[_dev(c) for _, c in mids])
    seq = _dev(t["seq"]).clone()
    mask = _dev(t["mask"])
    fws = torch.empty(v.vlb_workspace_bytes(p, b, seq.shape[0]), dtype=torch.uint8, device="cuda")
    saved = torch.empty(v.vlb_saved_bytes(p, b), dtype=torch.uint8, device="cuda")
    v.vlb_bridge_fused_train(p, b, _dev(t["features"]), wt, _dev(t["newline"]),
                             _dev(t["separator"]), mask, seq, saved, fws)
    g = v.Grads.empty(p, b)
    bws = torch.empty(v.vlb_backward_workspace_bytes(p, b, seq.shape[0]), dtype=torch.uint8,
                      device="cuda")
    v.vlb_bridge_backward(p, b, _dev(t["features"]), wt, mask, _dev(dseq), saved, g, bws)
    assert v.vlb_check(bws) == v.OK
    spec = common.oracle_spec(w)
    spec.depth = depth
    T = o.total_tokens(spec)
    st, drows, dnl, dsep = o.scatter_backward(o.assemble(spec), t["mask"].numpy(), dseq, T)
    assert st == 0
    ref = o.project_backward_deep(spec, t["features"], t["ln_gamma"], t["ln_beta"], t["w1"],
                                  t["b1"], [a for a, _ in mids], [c for _, c in mids], t["w2"],
                                  drows)
    tol = TOL_F32 if w.dtype == "f32" else TOL_ACT
    pairs = [("dw1", g.d_w1), ("db1", g.d_b1), ("dw2", g.d_w2), ("dx", g.d_features)]
    if w.has_ln:
        pairs += [("dgamma", g.d_ln_gamma), ("dbeta", g.d_ln_beta)]
    errs = {k: common.rel_frob(_np(x_), ref[k]) for k, x_ in pairs}
    for q in range(depth - 2):
        errs[f"dw_mid{q}"] = common.rel_frob(_np(g.d_w_mid[q]), ref["dw_mid"][q])
        errs[f"db_mid{q}"] = common.rel_frob(_np(g.d_b_mid[q]), ref["db_mid"][q])
    print(w.name, depth, {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        assert e <= tol, (k, e)


def test_backward_deterministic():
    w = small_workloads()[2]
    t = common.draw(w)
    dseq = wl.seq_grad(w)
    _, _, g1, _ = run_train(w, t, dseq)
    _, _, g2, _ = run_train(w, t, dseq)
    for a, b in ((g1.d_w1, g2.d_w1), (g1.d_b1, g2.d_b1), (g1.d_w2, g2.d_w2), (g1.d_b2, g2.d_b2),
                 (g1.d_features, g2.d_features), (g1.d_newline, g2.d_newline)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("wi", [0, 2])
def test_backward_mask_mismatch_writes_nothing(wi):
    w = small_workloads()[wi]
    t = common.draw(w)
    mask = t["mask"].clone()
    mask[int(np.flatnonzero(mask.numpy())[-1])] = 0
    dseq = wl.seq_grad(w)
    p, b = common.lib_projector(w), common.lib_batch(w)
    wt = _weights(t)
    saved = torch.zeros(v.vlb_saved_bytes(p, b), dtype=torch.uint8, device="cuda")
    g = v.Grads.empty(p, b)
    for x in (g.d_w1, g.d_b1, g.d_w2, g.d_b2, g.d_ln_gamma, g.d_ln_beta, g.d_newline,
              g.d_separator):
        if x is not None:
            x.fill_(7.0)
    g.d_features.fill_(3.0)
    bws = torch.empty(v.vlb_backward_workspace_bytes(p, b, w.seq_len), dtype=torch.uint8,
                      device="cuda")
    v.vlb_bridge_backward(p, b, _dev(t["features"]), wt, _dev(mask), _dev(dseq), saved, g, bws)
    assert v.vlb_check(bws) == v.ERR_MASK_COUNT
    for x in (g.d_w1, g.d_b1, g.d_w2, g.d_b2, g.d_ln_gamma, g.d_ln_beta, g.d_newline,
              g.d_separator):
        if x is not None:
            assert bool((x == 7.0).all())
    assert bool((g.d_features.float() == 3.0).all())


def test_backward_no_images_zero():
    w = small_workloads()[0]
    p = common.lib_projector(w)
    b = v.Batch([], [])
    t = common.draw(w)
    g = v.Grads.empty(p, b)
    for x in (g.d_w1, g.d_b1, g.d_w2, g.d_b2, g.d_ln_gamma, g.d_ln_beta):
        x.fill_(5.0)
    saved = torch.empty(16, dtype=torch.uint8, device="cuda")
    bws = torch.empty(max(v.vlb_backward_workspace_bytes(p, b, w.seq_len), 16), dtype=torch.uint8,
                      device="cuda")
    mask = torch.zeros(w.seq_len, dtype=torch.uint8, device="cuda")
    v.vlb_bridge_backward(p, b, None, _weights(t), mask, _dev(wl.seq_grad(w)), saved, g, bws)
    torch.cuda.synchronize()
    for x in (g.d_w1, g.d_b1, g.d_w2, g.d_b2, g.d_ln_gamma, g.d_ln_beta):
        assert bool((x == 0).all())
