"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

  * small workloads that span several 256-row / 256-column tiles with ragged
    tails: every projected row against the oracle (max per-image relative
    Frobenius error <= 1e-2 in bf16, <= 1e-5 in fp32), every other row of the
    sequence bit for bit;
  * the five full-size workloads in the benchmark's launch configuration
    (packed weights, fused call): every projected row against the oracle (per
    image, per row and per element), every text row bit for bit, and -- with
    0/1 selection weights and no activation -- every placeholder slot bit for
    bit against the oracle's merge, assembly and scatter;
  * the standalone merge and scatter entry points bit for bit, the
    placeholder-count error path, text-only batches and degenerate grids.
"""
import numpy as np
import pytest
import torch

import common
from oracle import oracle as o
from patch_merge_mlp_amd import vlbridge as v
from patch_merge_mlp_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"bf16": 1e-2, "f32": 1e-5}


def _dev(t):
    return None if t is None else t.to(DEV)


def _weights(t):
    return v.Weights(*(_dev(t[n]) for n in ("w1", "b1", "w2", "b2", "ln_gamma", "ln_beta")))


def run_fused(w, t, act=v.GELU_ERF, pack=True, has_ln=None, weights=None, gather=v.GATHER_AUTO):
    """One fused call; the sequence and the workspace carry guard bands, checked
    after the call."""
    p = common.lib_projector(w, act, has_ln, gather)
    b = common.lib_batch(w)
    br = v.Bridge(p, weights or _weights(t), pack=pack)
    g = common.Guards()
    seq = g.like(t["seq"], "seq")
    ws = g.workspace(v.vlb_workspace_bytes(br.p, b, seq.shape[0]))
    v.vlb_bridge_fused(br.p, b, _dev(t["features"]), br.w, _dev(t["newline"]),
                       _dev(t["separator"]), _dev(t["mask"]), seq, ws)
    st = v.vlb_check(ws)
    g.check()
    return st, seq.cpu()


def slot_positions(t):
    return np.flatnonzero(t["mask"].numpy())


def check_text_rows(t, seq_out):
    text = t["mask"].numpy() == 0
    a = seq_out.float().numpy()[text]
    b = t["seq"].float().numpy()[text]
    assert np.array_equal(a, b), "text rows changed"


def expected_seq(w, t, rows64, act=o.GELU_ERF):
    spec = common.oracle_spec(w, act)
    st, ref = o.scatter(o.assemble(spec), rows64, t["newline"], t["separator"], t["mask"].numpy(),
                        t["seq"])
    assert st == 0
    return ref


def per_image_errors(w, t, got, ref):
    pos = slot_positions(t)
    errs, j = [], 0
    for n in t["spans"]:
        idx = pos[j:j + n]
        errs.append(common.rel_frob(got[idx], ref[idx]))
        j += n
    return errs


# ---- small workloads: the whole output against the oracle ---------------------

def small_workloads():
    return [
        wl.Workload("small-2x2-ln", 11, "bf16", C=128, k=2, hidden=320, out_dim=192, seq_len=800,
                    grids=[(34, 34), (17, 20), (9, 31)], views_per_image=[1, 1, 1], has_ln=True),
        wl.Workload("small-3x3", 12, "bf16", C=64, k=3, hidden=256, out_dim=320, seq_len=700,
                    grids=[(48, 48), (50, 47)], views_per_image=[1, 1]),
        wl.Workload("small-tiled", 13, "bf16", C=128, k=2, hidden=192, out_dim=128, seq_len=700,
                    grids=[(13, 13)] * 10, views_per_image=[7, 3], tiled=True,
                    tiles=[(2, 3), (1, 2)]),
        wl.Workload("small-tiled-tail", 14, "bf16", C=64, k=2, hidden=128, out_dim=64,
                    seq_len=1200, grids=[(27, 27)] * 5, views_per_image=[5], tiled=True,
                    tiles=[(2, 2)], global_tail=True),
        wl.Workload("small-k1", 15, "bf16", C=64, k=1, hidden=128, out_dim=64, seq_len=600,
                    grids=[(24, 24)], views_per_image=[1]),
        wl.Workload("small-f32-3x3", 16, "f32", C=24, k=3, hidden=72, out_dim=40, seq_len=300,
                    grids=[(20, 17), (6, 6)], views_per_image=[2]),
        wl.config(0),
        # a sequence longer than one pass of the placeholder scan (16K positions),
        # the first image's span straddling the boundary between two passes
        wl.Workload("small-2x2-long-seq", 17, "bf16", C=64, k=2, hidden=128, out_dim=64,
                    seq_len=40000, grids=[(34, 34), (20, 17)], views_per_image=[1, 1],
                    fixed_offset=16200),
    ]


@pytest.mark.parametrize("w", small_workloads(), ids=lambda w: w.name)
def test_small_fused_vs_oracle(w):
    t = common.draw(w)
    spec = common.oracle_spec(w)
    rows = o.project_rows(spec, t["features"], t["ln_gamma"], t["ln_beta"], t["w1"], t["b1"],
                          t["w2"], t["b2"])
    ref = expected_seq(w, t, rows)
    modes = [(True, v.GATHER_AUTO)]
    if w.dtype == "bf16":
        modes.append((False, v.GATHER_AUTO))
        if not w.has_ln:  # both sources of Linear1's operand
            modes += [(True, v.GATHER_ON), (True, v.GATHER_OFF)]
    for pack, gather in modes:
        st, out = run_fused(w, t, pack=pack, gather=gather)
        assert st == v.OK
        check_text_rows(t, out)
        errs = per_image_errors(w, t, out.double().numpy(), ref)
        print(w.name, "pack" if pack else "nopack", "gather", gather, "max rel err", max(errs))
        assert max(errs) <= TOL[w.dtype], errs
        if w.tiled:  # newline / separator rows are copies
            spec_src = o.assemble(spec)
            pos = slot_positions(t)[spec_src < 0]
            assert np.array_equal(out.float().numpy()[pos], torch.from_numpy(ref[pos]).float().numpy())


def test_many_views_plain():
    """70 views (more than the 64 of one merge launch), plain layout, LayerNorm: the
    merge runs as two launches and the placeholder scan rides in the first.  Whole
    output against the oracle, text rows untouched; then a count mismatch on the same
    batch writes nothing."""
    grids = [(4 + i % 3, 6 - i % 2) for i in range(70)]
    w = wl.Workload("many-views", 31, "bf16", C=64, k=2, hidden=128, out_dim=64, seq_len=900,
                    grids=grids, views_per_image=[1] * 70, has_ln=True)
    t = common.draw(w)
    rows = o.project_rows(common.oracle_spec(w), t["features"], t["ln_gamma"], t["ln_beta"],
                          t["w1"], t["b1"], t["w2"], t["b2"])
    ref = expected_seq(w, t, rows)
    st, out = run_fused(w, t)
    assert st == v.OK
    check_text_rows(t, out)
    errs = per_image_errors(w, t, out.double().numpy(), ref)
    assert max(errs) <= TOL["bf16"], errs
    mask = t["mask"].clone()
    mask[int(np.flatnonzero(mask.numpy())[-1])] = 0
    st, out = run_fused(w, dict(t, mask=mask))
    assert st == v.ERR_MASK_COUNT
    assert torch.equal(out.view(torch.int16), t["seq"].view(torch.int16))


@pytest.mark.parametrize("C", [768, 1280, 2048, 3072, 4096])
def test_wide_channel_layernorm(C):
    """LayerNorm + merge at other channel counts: 768 and 1280 take one dword
    per lane and step (6 and 10 per lane; 1152, the same form with 9, is the
    main workload's); 2048, 3072 and 4096 take 4, 6 and 8 16-byte chunks per
    lane, the last keeping gamma and beta in bf16 in LDS (fp32 would not fit
    beside the staged rows).  The 9 x 10 grid pads its last column and row of
    cells.  Whole output against the oracle."""
    w = wl.Workload(f"wide-ln-{C}", 20 + C // 1024, "bf16", C=C, k=2, hidden=256, out_dim=128,
                    seq_len=96, grids=[(9, 10), (4, 4)], views_per_image=[1, 1], has_ln=True)
    t = common.draw(w)
    rows = o.project_rows(common.oracle_spec(w), t["features"], t["ln_gamma"], t["ln_beta"],
                          t["w1"], t["b1"], t["w2"], t["b2"])
    ref = expected_seq(w, t, rows)
    st, out = run_fused(w, t)
    assert st == v.OK
    check_text_rows(t, out)
    errs = per_image_errors(w, t, out.double().numpy(), ref)
    print(w.name, "max rel err", max(errs))
    assert max(errs) <= TOL["bf16"], errs


@pytest.mark.parametrize("act", [v.GELU_TANH, v.ACT_NONE])
def test_small_activations(act):
    w = small_workloads()[0]
    t = common.draw(w)
    spec = common.oracle_spec(w, act)
    rows = o.project_rows(spec, t["features"], t["ln_gamma"], t["ln_beta"], t["w1"], t["b1"],
                          t["w2"], t["b2"])
    ref = expected_seq(w, t, rows, act)
    st, out = run_fused(w, t, act=act)
    assert st == v.OK
    check_text_rows(t, out)
    assert max(per_image_errors(w, t, out.double().numpy(), ref)) <= 1e-2


@pytest.mark.parametrize("w", small_workloads()[:3], ids=lambda w: w.name)
def test_unfused_equals_fused(w):
    """vlb_merge_project + vlb_scatter_tokens give the fused call's bits."""
    t = common.draw(w)
    st, fused = run_fused(w, t)
    assert st == v.OK
    p, b = common.lib_projector(w), common.lib_batch(w)
    br = v.Bridge(p, _weights(t))
    g = common.Guards()
    rows = g.empty((v.vlb_num_tokens(br.p, b), w.out_dim), w.torch_dtype, "rows")
    ws0 = g.workspace(v.vlb_workspace_bytes(br.p, b, 0))
    v.vlb_merge_project(br.p, b, _dev(t["features"]), br.w, rows, ws0)
    seq = g.like(t["seq"], "seq")
    ws = g.workspace(v.vlb_workspace_bytes(br.p, b, seq.shape[0]))
    v.vlb_scatter_tokens(br.p, b, rows, _dev(t["newline"]), _dev(t["separator"]),
                         _dev(t["mask"]), seq, ws)
    assert v.vlb_check(ws) == v.OK
    g.check()
    assert torch.equal(seq.cpu().view(torch.int16), fused.view(torch.int16))


# ---- full-size workloads ----------------------------------------------------------

_FULL = {}


def full(i):
    if i not in _FULL:
        w = wl.config(i)
        _FULL.clear()
        _FULL[i] = (w, common.draw(w))
    return _FULL[i]


def _sample_rows(w, per_image=3, seed=0):
    rng = np.random.default_rng(seed)
    out = []
    for r0, r1 in common.image_row_ranges(w):
        out += [r0, r1 - 1]
        out += list(rng.integers(r0, r1, per_image))
    return np.unique(np.array(out, dtype=np.int64))


# Per-row bound at full size, next to the per-image one: a row's relative
# error is the mean of its O elements' errors, so it concentrates near the
# per-image figure (about 3e-3 in bf16: rounding of the LayerNorm output, of
# the hidden activation and of the output row, each 2^-9 relative at most).
# One wrong 16 x 16 MFMA block puts 16 wrong columns into 16 rows, about 6%
# of each such row's norm at O = 4096: caught here, while it would move the
# per-image norm by well under 1e-2.
ROW_TOL = {"bf16": 1e-2, "f32": 1e-5}
# Every element: |got - ref| <= ELEM_TOL * rms(ref row).  A single wrong
# element of the size of its row's entries fails it.
ELEM_TOL = {"bf16": 0.05, "f32": 1e-4}


def check_all_rows(w, t, out, label):
    """Every projected row of a fused call's sequence against the fp64 oracle:
    per image (relative Frobenius), per row and per element."""
    spec = common.oracle_spec(w)
    ref_rows = o.project_rows(spec, t["features"], t["ln_gamma"], t["ln_beta"], t["w1"], t["b1"],
                              t["w2"], t["b2"])
    src = o.assemble(spec)
    tok = src >= 0
    pos = slot_positions(t)[tok]            # slot of each projected row, in assembly order
    rows = src[tok]                         # the row at each of those slots
    got = out[torch.from_numpy(pos)].double().numpy()
    ref = ref_rows[rows]
    rnorm = np.linalg.norm(ref, axis=1)
    per_row = np.linalg.norm(got - ref, axis=1) / rnorm
    rms = rnorm / np.sqrt(w.out_dim)
    per_elem = (np.abs(got - ref) / rms[:, None]).max(axis=1)
    worst_img = 0.0
    for r0, r1 in common.image_row_ranges(w):
        sel = (rows >= r0) & (rows < r1)
        worst_img = max(worst_img, common.rel_frob(got[sel], ref[sel]))
    print(f"{label}: {len(rows)} rows, max per-image rel err {worst_img:.3e}, max per-row "
          f"{per_row.max():.3e} (row {int(rows[per_row.argmax()])}), max element / row rms "
          f"{per_elem.max():.3e}", flush=True)
    assert len(np.unique(rows)) == len(ref_rows), "some projected row has no slot"
    assert worst_img <= TOL[w.dtype], worst_img
    assert per_row.max() <= ROW_TOL[w.dtype], (per_row.max(), int(rows[per_row.argmax()]))
    assert per_elem.max() <= ELEM_TOL[w.dtype], (per_elem.max(), int(rows[per_elem.argmax()]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("i", range(wl.N_CONFIGS))
def test_full_config_all_rows(i):
    """All five workloads at full size in the benchmark's launch configuration
    (packed weights, fused call): every projected row against the oracle, every
    text row bit for bit."""
    w, t = full(i)
    print(f"full-size parity: {w.name}", flush=True)
    st, out = run_fused(w, t)
    assert st == v.OK
    check_text_rows(t, out)
    check_all_rows(w, t, out, w.name)


def selection_weights(w, start, dt):
    """W1 picks merged coordinates start.. start+H-1, W2 passes the first min(H, O)
    hidden units through; biases zero."""
    K1 = w.C * w.k * w.k
    W1 = torch.zeros(w.hidden, K1, dtype=dt)
    h = torch.arange(w.hidden)
    keep = start + h < K1
    W1[h[keep], start + h[keep]] = 1
    W2 = torch.zeros(w.out_dim, w.hidden, dtype=dt)
    n = min(w.hidden, w.out_dim)
    W2[torch.arange(n), torch.arange(n)] = 1
    return W1, torch.zeros(w.hidden, dtype=dt), W2, torch.zeros(w.out_dim, dtype=dt)


@pytest.mark.parametrize("i", range(wl.N_CONFIGS))
def test_full_config_exact_placement(i):
    """Merge, assembly, scatter and newline / separator placement bit for bit."""
    w, t = full(i)
    K1 = w.C * w.k * w.k
    n = min(w.hidden, w.out_dim)
    starts = sorted({0, max(0, K1 - n)})
    spec = common.oracle_spec(w)
    merged, p = [], 0
    x = t["features"]
    for gh, gw in w.grids:
        merged.append(o.merge_view(x[p:p + gh * gw].reshape(gh, gw, w.C), w.k))
        p += gh * gw
    merged = np.concatenate(merged)
    src = o.assemble(spec)
    for s in starts:
        W1, b1, W2, b2 = selection_weights(w, s, w.torch_dtype)
        weights = v.Weights(_dev(W1), _dev(b1), _dev(W2), _dev(b2))
        st, out = run_fused(w, t, act=v.ACT_NONE, has_ln=False, weights=weights)
        assert st == v.OK
        rows = np.zeros((len(merged), w.out_dim))
        hi = min(n, K1 - s)
        rows[:, :hi] = merged[:, s:s + hi]
        st2, ref = o.scatter(src, rows, t["newline"], t["separator"], t["mask"].numpy(), t["seq"])
        assert st2 == 0
        want = torch.from_numpy(ref).to(w.torch_dtype)
        assert torch.equal(torch.from_numpy(ref).to(w.torch_dtype).double(), torch.from_numpy(ref)), \
            "expected values are not exact bf16 values"
        bad = (out.float() != want.float()).any(dim=1)
        assert not bad.any(), f"{int(bad.sum())} rows differ, first at {int(bad.nonzero()[0])}"


# ---- gather mode: Linear1 reads the merged tokens from the grid -------------------

def _gather_workloads():
    # bf16 without LayerNorm: 3x3 odd and rectangular grids, tiled head and tail,
    # k = 1, grids of one cell and one row
    ws = [w for w in small_workloads() if w.dtype == "bf16" and not w.has_ln]
    ws.append(wl.Workload("tiny-grids", 21, "bf16", C=64, k=3, hidden=64, out_dim=64, seq_len=64,
                          grids=[(1, 1), (1, 7), (4, 1)], views_per_image=[1, 1, 1]))
    return ws


@pytest.mark.parametrize("w", _gather_workloads(), ids=lambda w: w.name)
def test_gather_mode_small_vs_oracle(w):
    """Gather mode: the whole output against the oracle, and bit for bit the
    merging path's (the same bf16 operand values in the same K order and tiles)."""
    t = common.draw(w)
    rows = o.project_rows(common.oracle_spec(w), t["features"], None, None, t["w1"], t["b1"],
                          t["w2"], t["b2"])
    ref = expected_seq(w, t, rows)
    st, out = run_fused(w, t, gather=v.GATHER_ON)
    assert st == v.OK
    check_text_rows(t, out)
    errs = per_image_errors(w, t, out.double().numpy(), ref)
    assert max(errs) <= TOL["bf16"], errs
    st, base = run_fused(w, t, gather=v.GATHER_OFF)
    assert st == v.OK
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


@pytest.mark.parametrize("i", [2, 3, 4])
def test_gather_mode_full_config_bits(i):
    """Both operand sources at full size on the workloads without LayerNorm give
    the same bits in every slot (test_full_config_all_rows holds the automatic
    choice against the oracle row by row)."""
    w, t = full(i)
    st, out = run_fused(w, t, gather=v.GATHER_ON)
    assert st == v.OK
    st, base = run_fused(w, t, gather=v.GATHER_OFF)
    assert st == v.OK
    same = (out.view(torch.int16) == base.view(torch.int16)).all(dim=1)
    assert bool(same.all()), f"{int((~same).sum())} rows differ, first at {int((~same).nonzero()[0])}"


def test_gather_mode_count_mismatch_writes_nothing():
    w = _gather_workloads()[0]
    t = common.draw(w)
    mask = t["mask"].clone()
    mask[int(np.flatnonzero(mask.numpy())[-1])] = 0
    st, out = run_fused(w, dict(t, mask=mask), gather=v.GATHER_ON)
    assert st == v.ERR_MASK_COUNT
    assert torch.equal(out.view(torch.int16), t["seq"].view(torch.int16))


# ---- standalone merge and scatter ---------------------------------------------------

@pytest.mark.parametrize("w", small_workloads()[1:6] + [None], ids=lambda w: w.name if w else "cfg2")
def test_merge_tokens_exact(w):
    if w is None:
        w, t = full(2)
    else:
        t = common.draw(w)
    p, b = common.lib_projector(w, has_ln=False), common.lib_batch(w)
    T = v.vlb_num_tokens(p, b)
    g = common.Guards()
    merged = g.empty((T, w.C * w.k * w.k), w.torch_dtype, "merged")
    ws = g.workspace(v.vlb_workspace_bytes(p, b, 0))
    v.vlb_merge_tokens(p, b, _dev(t["features"]), None, None, merged, ws)
    torch.cuda.synchronize()
    g.check()
    got = merged.cpu().double().numpy()
    want, q = [], 0
    for gh, gw in w.grids:
        want.append(o.merge_view(t["features"][q:q + gh * gw].reshape(gh, gw, w.C), w.k))
        q += gh * gw
    assert np.array_equal(got, np.concatenate(want))


def test_merge_tokens_layernorm():
    """With the LayerNorm on, merged values are the oracle's to bf16 rounding."""
    w = small_workloads()[0]
    t = common.draw(w)
    p, b = common.lib_projector(w), common.lib_batch(w)
    T = v.vlb_num_tokens(p, b)
    merged = torch.empty(T, w.C * w.k * w.k, dtype=torch.bfloat16, device=DEV)
    ws = v.workspace(p, b, 0)
    v.vlb_merge_tokens(p, b, _dev(t["features"]), _dev(t["ln_gamma"]), _dev(t["ln_beta"]), merged,
                       ws)
    spec = common.oracle_spec(w)
    want = np.stack([o.merged_row(spec, t["features"], t["ln_gamma"], t["ln_beta"], r)
                     for r in range(T)])
    got = merged.cpu().double().numpy()
    assert np.all(np.abs(got - want) <= 2.0 ** -7 * np.abs(want) + 1e-6)


@pytest.mark.parametrize("w", small_workloads()[:4] + [None], ids=lambda w: w.name if w else "cfg3")
def test_scatter_tokens_exact(w):
    if w is None:
        w, t = full(3)
    else:
        t = common.draw(w)
    p, b = common.lib_projector(w), common.lib_batch(w)
    T = v.vlb_num_tokens(p, b)
    g = torch.Generator().manual_seed(7)
    rows = torch.randn(T, w.out_dim, generator=g).to(w.torch_dtype)
    gd = common.Guards()
    seq = gd.like(t["seq"], "seq")
    ws = gd.workspace(v.vlb_workspace_bytes(p, b, seq.shape[0]))
    v.vlb_scatter_tokens(p, b, _dev(rows), _dev(t["newline"]), _dev(t["separator"]),
                         _dev(t["mask"]), seq, ws)
    assert v.vlb_check(ws) == v.OK
    gd.check()
    st, ref = o.scatter(o.assemble(common.oracle_spec(w)), rows, t["newline"], t["separator"],
                        t["mask"].numpy(), t["seq"])
    assert st == 0
    assert np.array_equal(seq.cpu().double().numpy(), ref)


# ---- error path and degenerate cases -------------------------------------------------

@pytest.mark.parametrize("delta", [+1, -1])
@pytest.mark.parametrize("idx", [0, 2, 7])
def test_mask_count_mismatch_writes_nothing(delta, idx):
    w = small_workloads()[idx]
    t = common.draw(w)
    mask = t["mask"].clone()
    if delta > 0:
        mask[int(np.flatnonzero(mask.numpy() == 0)[0])] = 1
    else:
        mask[int(np.flatnonzero(mask.numpy())[-1])] = 0
    t2 = dict(t, mask=mask)
    st, out = run_fused(w, t2)
    assert st == v.ERR_MASK_COUNT
    assert torch.equal(out.view(torch.int16), t["seq"].view(torch.int16))
    st, _ = run_fused(w, t)  # the next good call on a fresh workspace reports ok
    assert st == v.OK


def test_text_only_is_noop():
    w = small_workloads()[0]
    t = common.draw(w)
    p = common.lib_projector(w)
    b = v.Batch([], [])
    seq = _dev(t["seq"]).clone()
    mask = torch.zeros(seq.shape[0], dtype=torch.uint8, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    v.vlb_bridge_fused(p, b, _dev(t["features"]), _weights(t), None, None, mask, seq, ws)
    torch.cuda.synchronize()
    assert torch.equal(seq.cpu().view(torch.int16), t["seq"].view(torch.int16))


def test_degenerate_grids():
    """1x1 grids (all but one cell of the 3x3 block is padding) and a grid of one row."""
    w = wl.Workload("tiny-grids", 21, "bf16", C=64, k=3, hidden=64, out_dim=64, seq_len=64,
                    grids=[(1, 1), (1, 7), (4, 1)], views_per_image=[1, 1, 1])
    t = common.draw(w)
    spec = common.oracle_spec(w)
    rows = o.project_rows(spec, t["features"], None, None, t["w1"], t["b1"], t["w2"], t["b2"])
    ref = expected_seq(w, t, rows)
    st, out = run_fused(w, t)
    assert st == v.OK
    check_text_rows(t, out)
    assert max(per_image_errors(w, t, out.double().numpy(), ref)) <= 1e-2


def test_repeated_calls_identical():
    w = small_workloads()[2]
    t = common.draw(w)
    st1, a = run_fused(w, t)
    st2, b = run_fused(w, t)
    assert st1 == st2 == v.OK
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
