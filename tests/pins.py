"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each pin_* function takes the oracle module and raises AssertionError when the
oracle disagrees with a value the pages print, a closed form, an invariant, or a
library routine that computes the same special case.  test_oracle_pins runs them
on the real oracle; test_oracle_mutants runs them on copies of the oracle with
one planted mistake each and requires that some pin fails.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            out.append(line.rstrip("\n").split("\t"))
    return out


def _tiled_spec(o, grid, k, tw, th, n_images=1, tail=False, D=1):
    views = 1 + tw * th
    return o.Spec(grids=[(grid, grid)] * (views * n_images), C=1, k=k, hidden=1, out_dim=D,
                  views_per_image=[views] * n_images, tiled=True, tiles=[(tw, th)] * n_images,
                  global_tail=tail)


# --- values the pages print -------------------------------------------------

def pin_page_counts(o):
    """Token and slot counts worked out on the pages (tests/golden/page_counts.tsv)."""
    for kind, px, patch, k, tw, th, expected, _src in _rows("page_counts.tsv"):
        px, patch, k, tw, th, expected = map(int, (px, patch, k, tw, th, expected))
        g = px // patch  # the tower's patch grid: floor(image_size / patch_size)
        if kind == "patches":
            assert g * g == expected
        elif kind == "tokens":
            assert o.view_tokens(g, g, k) == expected, (px, patch, k)
            spec = o.Spec(grids=[(g, g)], C=1, k=k, hidden=1, out_dim=1, views_per_image=[1])
            assert len(o.assemble(spec)) == expected
        elif kind == "slots":
            spec = _tiled_spec(o, g, k, tw, th)
            assert len(o.assemble(spec)) == expected, (px, patch, tw, th)
            hp = o.merged_side(g, k)
            assert o.tiled_placeholders(hp, hp, tw, th) == expected
        else:
            raise AssertionError(kind)


def pin_param_count(o):
    """40,119,040 = LN(1152) + Linear(4608->4608) + Linear(4608->4096); the other
    plausible layouts miss it."""
    for C, k, hidden, out, has_ln, expected in _rows("projector_params.tsv"):
        C, k, hidden, out, has_ln, expected = map(int, (C, k, hidden, out, has_ln, expected))
        assert o.param_count(C, k, hidden, out, bool(has_ln)) == expected
        assert o.param_count(C, k, hidden, out, not has_ln) != expected
        assert o.param_count(C * k * k, 1, hidden, out, bool(has_ln)) != expected  # LN over 4608


def pin_merged_width(o):
    """4 x 1152 = 4608 (2x2 PatchMerger) and 9 x 1024 = 9216 (3x3 pixel-unshuffle)."""
    assert o.merge_view(np.ones((2, 2, 1152)), 2).shape == (1, 4608)
    assert o.merge_view(np.ones((3, 3, 1024)), 3).shape == (1, 9216)


# --- the merge: bijection and the library pixel-unshuffle ------------------

_GRIDS = [(4, 4, 3, 2), (5, 7, 2, 2), (7, 5, 3, 3), (6, 6, 4, 3), (3, 3, 5, 1), (1, 1, 2, 2)]


def pin_merge_roundtrip(o):
    """The merge is lossless: unmerge(merge(x)) == x bit for bit; padded cells are 0."""
    rng = np.random.default_rng(1)
    for gh, gw, C, k in _GRIDS:
        x = rng.standard_normal((gh, gw, C)) + 3.0  # no zeros in the data
        m = o.merge_view(x, k)
        hp, wp = -(-gh // k), -(-gw // k)
        assert m.shape == (hp * wp, C * k * k)
        assert np.array_equal(o.unmerge_view(m, gh, gw, C, k), x)
        assert int((m == 0).sum()) == (hp * k * wp * k - gh * gw) * C


def _torch_merge(x, k):
    """The library pixel-unshuffle after high-end zero padding: (gh, gw, C) -> (tokens, C k^2)."""
    gh, gw, C = x.shape
    hp, wp = -(-gh // k), -(-gw // k)
    t = torch.from_numpy(x).permute(2, 0, 1).unsqueeze(0)
    t = F.pad(t, (0, wp * k - gw, 0, hp * k - gh))
    u = F.pixel_unshuffle(t, k)  # (1, C k^2, hp, wp), channel = c k^2 + dy k + dx
    return u[0].permute(1, 2, 0).reshape(hp * wp, C * k * k).numpy()


def pin_merge_pixel_unshuffle(o):
    """Feature order c*k*k + dy*k + dx equals torch's pixel_unshuffle channel order."""
    rng = np.random.default_rng(2)
    for gh, gw, C, k in _GRIDS:
        x = rng.standard_normal((gh, gw, C))
        assert np.array_equal(o.merge_view(x, k), _torch_merge(x, k)), (gh, gw, C, k)


# --- assembly: closed-form slot of every token, newline and separator --------

def _slot_map(hp, wp, tw, th, tail):
    """The assembled slots of one tiled image, built from the other direction than
    the oracle: each token (view v, merged row y, column x), newline and separator
    is placed at its slot index computed in closed form, then the slots are read
    out in order.  Token ids: v * hp * wp + y * wp + x; newline -1, separator -2.
    Layout ([VL2] Tile-sequence assembly): the global view as hp rows of wp tokens
    and a newline; the separator; the local views as one mosaic of th * hp rows
    by tw * wp columns (view 1 + i * tw + j covering rows i * hp .. and columns
    j * wp ..), a newline after each mosaic row.  Tail: mosaic, separator, global."""
    G = hp * (wp + 1)                # global block, newlines included
    W = tw * wp + 1                  # one mosaic row, its newline included
    L = th * hp * W                  # mosaic block
    n = G + 1 + L
    out = np.full(n, -99, dtype=np.int64)
    g0, s0, l0 = (L + 1, L, 0) if tail else (0, G, G + 1)
    for y in range(hp):
        for x in range(wp):
            out[g0 + y * (wp + 1) + x] = y * wp + x
        out[g0 + y * (wp + 1) + wp] = -1
    out[s0] = -2
    for v in range(1, 1 + tw * th):
        i, j = divmod(v - 1, tw)
        for y in range(hp):
            for x in range(wp):
                out[l0 + (i * hp + y) * W + j * wp + x] = v * hp * wp + y * wp + x
    for R in range(th * hp):
        out[l0 + R * W + tw * wp] = -1
    assert (out != -99).all(), "a slot was left unassigned"
    return out


def pin_assembly_slots(o):
    """The oracle's assembly equals the closed-form slot map, for several tile
    grids, head and tail; slot totals are h'(w'+1) + 1 + (th h')(tw w'+1)."""
    for hp, tw, th, tail in [(2, 2, 3, False), (3, 1, 1, False), (2, 3, 2, True), (14, 2, 1, False),
                             (4, 1, 3, False), (1, 2, 2, True)]:
        k = 2
        spec = _tiled_spec(o, hp * k - 1, k, tw, th, tail=tail)  # odd grid: padded to hp*k
        assert o.merged_side(hp * k - 1, k) == hp
        got = o.assemble(spec)
        want = _slot_map(hp, hp, tw, th, tail)
        assert np.array_equal(got, want), (hp, tw, th, tail)
        assert len(got) == hp * (hp + 1) + 1 + (th * hp) * (tw * hp + 1)
        assert (got == -1).sum() == hp + th * hp and (got == -2).sum() == 1


def pin_assembly_images(o):
    """Images are laid out one after another, each with its own token rows."""
    spec = _tiled_spec(o, 4, 2, 2, 1, n_images=3)
    got = o.assemble(spec)
    one = _slot_map(2, 2, 2, 1, False)
    per = 3 * 4  # three views of 2x2 tokens
    want = np.concatenate([np.where(one >= 0, one + i * per, one) for i in range(3)])
    assert np.array_equal(got, want)
    plain = o.Spec(grids=[(4, 6), (3, 3)], C=1, k=2, hidden=1, out_dim=1, views_per_image=[1, 1])
    assert np.array_equal(o.assemble(plain), np.arange(6 + 4))
    assert o.total_tokens(plain) == 10


# --- projector arithmetic against the library routines ----------------------

def pin_gelu_values(o):
    """GELU(x) = x Phi(x) at tabulated normal-CDF points, and GELU(x) - GELU(-x) = x."""
    for x, phi in _rows("normal_cdf.tsv"):
        x, phi = float(x), float(phi)
        got = o.gelu_erf(np.array([x, -x]))
        assert abs(got[0] - x * phi) < 1e-14
        assert abs(got[1] - (-x) * (1.0 - phi)) < 1e-14
    xs = np.linspace(-6, 6, 101)
    assert np.allclose(o.gelu_erf(xs) - o.gelu_erf(-xs), xs, rtol=0, atol=1e-14)
    assert o.gelu_erf(np.array([0.0]))[0] == 0.0


def pin_gelu_library(o):
    x = torch.linspace(-8, 8, 1001, dtype=torch.float64)
    assert np.allclose(o.gelu_erf(x.numpy()), F.gelu(x).numpy(), rtol=0, atol=1e-15)
    assert np.allclose(o.gelu_tanh(x.numpy()), F.gelu(x, approximate="tanh").numpy(), rtol=0,
                       atol=1e-15)


def pin_linear_library(o):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 13))
    W = rng.standard_normal((5, 13))
    b = rng.standard_normal(5)
    want = F.linear(torch.from_numpy(x), torch.from_numpy(W), torch.from_numpy(b)).numpy()
    for nt in (1, 3):
        assert np.allclose(o.linear(x, W, b, nt), want, rtol=1e-13, atol=1e-13)


def pin_layer_norm(o):
    rng = np.random.default_rng(4)
    C = 48
    x = rng.standard_normal((9, C)) * 3 + 1
    g = rng.standard_normal(C)
    b = rng.standard_normal(C)
    want = F.layer_norm(torch.from_numpy(x), (C,), torch.from_numpy(g), torch.from_numpy(b),
                        eps=1e-6).numpy()
    assert np.allclose(o.layer_norm(x, g, b, 1e-6), want, rtol=1e-12, atol=1e-12)
    # Invariants with gamma = 1, beta = 0: zero mean, variance var/(var+eps).
    eps = 0.5
    y = o.layer_norm(x, np.ones(C), np.zeros(C), eps)
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)


def pin_project_rows_library(o):
    """The whole projector row by row vs. library routines: layer_norm, pad,
    pixel_unshuffle, linear, gelu, linear; for both activations and with LN on/off,
    on views of different sizes (odd ones padded)."""
    rng = np.random.default_rng(5)
    C, k, H, O = 6, 2, 10, 7
    grids = [(3, 5), (4, 4), (5, 3)]
    x = rng.standard_normal((sum(a * b for a, b in grids), C))
    g = rng.standard_normal(C)
    bb = rng.standard_normal(C)
    W1 = rng.standard_normal((H, C * k * k))
    b1 = rng.standard_normal(H)
    W2 = rng.standard_normal((O, H))
    b2 = rng.standard_normal(O)
    for has_ln in (False, True):
        for act in (o.GELU_ERF, o.GELU_TANH, o.ACT_NONE):
            spec = o.Spec(grids=grids, C=C, k=k, hidden=H, out_dim=O, views_per_image=[1, 2],
                          has_ln=has_ln, ln_eps=1e-6, act=act)
            merged, p = [], 0
            for gh, gw in grids:
                v = torch.from_numpy(x[p:p + gh * gw].reshape(gh, gw, C))
                p += gh * gw
                if has_ln:
                    v = F.layer_norm(v, (C,), torch.from_numpy(g), torch.from_numpy(bb), eps=1e-6)
                merged.append(_torch_merge(v.numpy(), k))
            m = torch.from_numpy(np.concatenate(merged))
            h = F.linear(m, torch.from_numpy(W1), torch.from_numpy(b1))
            if act == o.GELU_ERF:
                h = F.gelu(h)
            elif act == o.GELU_TANH:
                h = F.gelu(h, approximate="tanh")
            want = F.linear(h, torch.from_numpy(W2), torch.from_numpy(b2)).numpy()
            got = o.project_rows(spec, x, g, bb, W1, b1, W2, b2, nthreads=2)
            assert got.shape == want.shape
            assert np.allclose(got, want, rtol=1e-12, atol=1e-12), (has_ln, act)
            sub = np.array([5, 0, len(want) - 1])
            got_sub = o.project_rows(spec, x, g, bb, W1, b1, W2, b2, row_ids=sub, nthreads=1)
            assert np.array_equal(got_sub, got[sub])


def pin_project_rows_deep_library(o):
    """Depth 3 and 4 ([VL2] Projector 3: extra activation + Linear(hidden -> hidden)
    pairs in the middle) vs library routines; depth 2 equals project_rows."""
    rng = np.random.default_rng(6)
    C, k, H, O = 4, 2, 9, 6
    grids = [(3, 3), (4, 2)]
    x = rng.standard_normal((sum(a * b for a, b in grids), C))
    g = rng.standard_normal(C)
    bb = rng.standard_normal(C)
    W1 = rng.standard_normal((H, C * k * k))
    b1 = rng.standard_normal(H)
    Wm = [rng.standard_normal((H, H)) / 3 for _ in range(2)]
    bm = [rng.standard_normal(H) for _ in range(2)]
    W2 = rng.standard_normal((O, H))
    b2 = rng.standard_normal(O)
    T = lambda a: torch.from_numpy(a)
    for has_ln in (False, True):
        for act in (o.GELU_ERF, o.GELU_TANH, o.ACT_NONE):
            merged, p = [], 0
            for gh, gw in grids:
                v = T(x[p:p + gh * gw].reshape(gh, gw, C))
                p += gh * gw
                if has_ln:
                    v = F.layer_norm(v, (C,), T(g), T(bb), eps=1e-6)
                merged.append(_torch_merge(v.numpy(), k))
            m = T(np.concatenate(merged))
            actf = {o.GELU_ERF: F.gelu, o.GELU_TANH: lambda z: F.gelu(z, approximate="tanh"),
                    o.ACT_NONE: lambda z: z}[act]
            for depth in (2, 3, 4):
                h = F.linear(m, T(W1), T(b1))
                for q in range(depth - 2):
                    h = F.linear(actf(h), T(Wm[q]), T(bm[q]))
                want = F.linear(actf(h), T(W2), T(b2)).numpy()
                spec = o.Spec(grids=grids, C=C, k=k, hidden=H, out_dim=O, views_per_image=[2],
                              has_ln=has_ln, ln_eps=1e-6, act=act, depth=depth)
                got = o.project_rows_deep(spec, x, g, bb, W1, b1, Wm[:depth - 2], bm[:depth - 2],
                                          W2, b2, nthreads=2)
                assert np.allclose(got, want, rtol=1e-12, atol=1e-12), (has_ln, act, depth)
                if depth == 2:
                    assert np.array_equal(got, o.project_rows(spec, x, g, bb, W1, b1, W2, b2,
                                                              nthreads=2))


# --- scatter -----------------------------------------------------------------

def pin_scatter(o):
    """Rows overwrite the placeholder positions in order; everything else is kept;
    a count mismatch writes nothing."""
    S, D = 12, 3
    seq = np.arange(S * D, dtype=np.float64).reshape(S, D) + 1000
    rows = np.array([[1, 1, 1], [2, 2, 2], [3, 3, 3]], dtype=np.float64)
    nl = np.full(D, -1.0)
    sp = np.full(D, -2.0)
    src = np.array([1, -1, 0, -2, 2])  # token 1, newline, token 0, separator, token 2
    mask = np.zeros(S, dtype=np.uint8)
    mask[[2, 3, 7, 8, 11]] = 1
    st, out = o.scatter(src, rows, nl, sp, mask, seq)
    assert st == 0
    want = seq.copy()
    want[2], want[3], want[7], want[8], want[11] = rows[1], nl, rows[0], sp, rows[2]
    assert np.array_equal(out, want)
    for bad in ([2, 3, 7, 8], [0, 2, 3, 7, 8, 11]):
        m = np.zeros(S, dtype=np.uint8)
        m[bad] = 1
        st, out = o.scatter(src, rows, nl, sp, m, seq)
        assert st == -1 and np.array_equal(out, seq)
    st, out = o.scatter(np.zeros(0, dtype=np.int64), rows, nl, sp, np.zeros(S, np.uint8), seq)
    assert st == 0 and np.array_equal(out, seq)


def pin_embed_scatter(o):
    """The embedded sequence equals torch's embedding lookup with the assembled rows
    placed by masked_scatter at the image-token positions (the page's "overwrite the
    token embeddings at exactly the positions holding image_token_index, in order");
    a placeholder-count mismatch or an out-of-range text id writes nothing."""
    g = torch.Generator().manual_seed(7)
    S, D, vocab, img = 20, 5, 11, 9
    E = torch.randn(vocab, D, generator=g, dtype=torch.float64)
    rows = torch.randn(4, D, generator=g, dtype=torch.float64)
    nl = torch.full((D,), -1.0, dtype=torch.float64)
    sp = torch.full((D,), -2.0, dtype=torch.float64)
    src = np.array([2, -1, 0, -2, 3, 1])  # assembled slots: token 2, newline, token 0, sep, 3, 1
    ids = torch.tensor([1, 0, img, img, 4, img, 10, 2, img, img, 3, 7, img, 5, 6, 8, 0, 10, 1, 2],
                       dtype=torch.int32)
    A = torch.stack([rows[s] if s >= 0 else (nl if s == -1 else sp) for s in src])
    mask = ids == img
    want = F.embedding(torch.where(mask, torch.zeros_like(ids), ids).long(), E)
    want = want.masked_scatter(mask[:, None].expand(S, D), A)
    st, got = o.embed_scatter(src, rows, nl, sp, ids, img, E, D)
    assert st == 0 and np.array_equal(got, want.numpy())
    # bf16 table: widened exactly
    Eb = E.to(torch.bfloat16)
    st, got = o.embed_scatter(src, rows, nl, sp, ids, img, Eb, D)
    want_b = F.embedding(torch.where(mask, torch.zeros_like(ids), ids).long(), Eb.double())
    want_b = want_b.masked_scatter(mask[:, None].expand(S, D), A)
    assert st == 0 and np.array_equal(got, want_b.numpy())
    # errors: one placeholder too many / too few, then a text id past the vocabulary
    for pos, val, code in ((0, img, -1), (2, 4, -1), (6, vocab, -2), (7, -3, -2)):
        bad = ids.clone()
        bad[pos] = val
        st, got = o.embed_scatter(src, rows, nl, sp, bad, img, E, D)
        assert st == code and not got.any(), (pos, val, st)
    # text only: every row comes from the table
    st, got = o.embed_scatter(np.zeros(0, np.int64), rows, nl, sp, ids[~mask], img, E, D)
    assert st == 0 and np.array_equal(got, F.embedding(ids[~mask].long(), E).numpy())



# --- backward ------------------------------------------------------------------

def _torch_projector(x, g, bb, W1, b1, W2, b2, grids, C, k, has_ln, act, eps):
    """The projector forward composed from library routines (differentiable)."""
    merged, p = [], 0
    for gh, gw in grids:
        v = x[p:p + gh * gw].reshape(gh, gw, C)
        p += gh * gw
        if has_ln:
            v = F.layer_norm(v, (C,), g, bb, eps=eps)
        hp, wp = -(-gh // k), -(-gw // k)
        t = F.pad(v.permute(2, 0, 1).unsqueeze(0), (0, wp * k - gw, 0, hp * k - gh))
        merged.append(F.pixel_unshuffle(t, k)[0].permute(1, 2, 0).reshape(hp * wp, C * k * k))
    h = F.linear(torch.cat(merged), W1, b1)
    if act == 0:
        h = F.gelu(h)
    elif act == 1:
        h = F.gelu(h, approximate="tanh")
    return F.linear(h, W2, b2)


def _bwd_problem(seed, C=5, k=2, H=9, O=7, grids=((3, 5), (4, 4), (5, 3))):
    rng = np.random.default_rng(seed)
    P = sum(a * b for a, b in grids)
    T = sum((-(-a // k)) * (-(-b // k)) for a, b in grids)
    d = dict(x=rng.standard_normal((P, C)) * 2 + 0.5, g=1 + 0.5 * rng.standard_normal(C),
             bb=rng.standard_normal(C), W1=rng.standard_normal((H, C * k * k)),
             b1=rng.standard_normal(H), W2=rng.standard_normal((O, H)), b2=rng.standard_normal(O),
             dY=rng.standard_normal((T, O)))
    return d, list(grids), C, k, H, O


def pin_project_backward_autograd(o):
    """Every projector gradient equals torch autograd (fp64) through the library
    forward, for each activation, with the LayerNorm on and off, on padded views."""
    d, grids, C, k, H, O = _bwd_problem(11)
    for has_ln in (False, True):
        for act in (o.GELU_ERF, o.GELU_TANH, o.ACT_NONE):
            eps = 0.3  # large enough that its place in the formula matters
            spec = o.Spec(grids=grids, C=C, k=k, hidden=H, out_dim=O, views_per_image=[3],
                          has_ln=has_ln, ln_eps=eps, act=act)
            ts = {n: torch.from_numpy(d[n]).requires_grad_(True)
                  for n in ("x", "g", "bb", "W1", "b1", "W2", "b2")}
            y = _torch_projector(ts["x"], ts["g"], ts["bb"], ts["W1"], ts["b1"], ts["W2"], ts["b2"],
                                 grids, C, k, has_ln, act, eps)
            (y * torch.from_numpy(d["dY"])).sum().backward()
            got = o.project_backward(spec, d["x"], d["g"], d["bb"], d["W1"], d["b1"], d["W2"],
                                     d["dY"])
            pairs = [("dx", "x"), ("dw1", "W1"), ("db1", "b1"), ("dw2", "W2"), ("db2", "b2")]
            if has_ln:
                pairs += [("dgamma", "g"), ("dbeta", "bb")]
            for mine, theirs in pairs:
                assert np.allclose(got[mine], ts[theirs].grad.numpy(), rtol=1e-10, atol=1e-11), \
                    (has_ln, act, mine)


def pin_project_backward_deep_autograd(o):
    """Depth 3 and 4: every gradient, the middle Linears' included, equals torch
    autograd through the library forward; depth 2 equals project_backward."""
    d, grids, C, k, H, O = _bwd_problem(14, C=4, H=7, O=5, grids=((3, 5), (4, 4)))
    rng = np.random.default_rng(15)
    Wm = [rng.standard_normal((H, H)) / 2 for _ in range(2)]
    bm = [rng.standard_normal(H) for _ in range(2)]
    for has_ln, act in ((True, o.GELU_ERF), (False, o.GELU_TANH), (True, o.ACT_NONE)):
        for depth in (2, 3, 4):
            n = depth - 2
            spec = o.Spec(grids=grids, C=C, k=k, hidden=H, out_dim=O, views_per_image=[2],
                          has_ln=has_ln, ln_eps=0.3, act=act, depth=depth)
            ts = {nm: torch.from_numpy(d[nm]).requires_grad_(True)
                  for nm in ("x", "g", "bb", "W1", "b1", "W2", "b2")}
            tm = [torch.from_numpy(w_).requires_grad_(True) for w_ in Wm[:n]]
            tb = [torch.from_numpy(b_).requires_grad_(True) for b_ in bm[:n]]
            actf = {o.GELU_ERF: F.gelu, o.GELU_TANH: lambda z: F.gelu(z, approximate="tanh"),
                    o.ACT_NONE: lambda z: z}[act]
            merged, p = [], 0
            for gh, gw in grids:
                v = ts["x"][p:p + gh * gw].reshape(gh, gw, C)
                p += gh * gw
                if has_ln:
                    v = F.layer_norm(v, (C,), ts["g"], ts["bb"], eps=0.3)
                hp, wp = -(-gh // k), -(-gw // k)
                tt = F.pad(v.permute(2, 0, 1).unsqueeze(0), (0, wp * k - gw, 0, hp * k - gh))
                merged.append(F.pixel_unshuffle(tt, k)[0].permute(1, 2, 0).reshape(hp * wp, C * k * k))
            h = F.linear(torch.cat(merged), ts["W1"], ts["b1"])
            for q in range(n):
                h = F.linear(actf(h), tm[q], tb[q])
            y = F.linear(actf(h), ts["W2"], ts["b2"])
            (y * torch.from_numpy(d["dY"])).sum().backward()
            got = o.project_backward_deep(spec, d["x"], d["g"], d["bb"], d["W1"], d["b1"], Wm[:n],
                                          bm[:n], d["W2"], d["dY"])
            pairs = [("dx", ts["x"]), ("dw1", ts["W1"]), ("db1", ts["b1"]), ("dw2", ts["W2"]),
                     ("db2", ts["b2"])]
            if has_ln:
                pairs += [("dgamma", ts["g"]), ("dbeta", ts["bb"])]
            for mine, t_ in pairs:
                assert np.allclose(got[mine], t_.grad.numpy(), rtol=1e-10, atol=1e-11), \
                    (depth, has_ln, act, mine)
            for q in range(n):
                assert np.allclose(got["dw_mid"][q], tm[q].grad.numpy(), rtol=1e-10, atol=1e-11)
                assert np.allclose(got["db_mid"][q], tb[q].grad.numpy(), rtol=1e-10, atol=1e-11)
            if depth == 2:
                ref = o.project_backward(spec, d["x"], d["g"], d["bb"], d["W1"], d["b1"], d["W2"],
                                         d["dY"])
                for nm in ref:
                    assert np.array_equal(ref[nm], got[nm]), nm


def pin_project_backward_fd(o):
    """Central finite differences of the (pinned) forward: L = sum(dY * Y)."""
    d, grids, C, k, H, O = _bwd_problem(12, C=3, H=5, O=4, grids=((3, 3), (2, 5)))
    spec = o.Spec(grids=grids, C=C, k=k, hidden=H, out_dim=O, views_per_image=[2], has_ln=True,
                  ln_eps=0.2, act=o.GELU_ERF)
    got = o.project_backward(spec, d["x"], d["g"], d["bb"], d["W1"], d["b1"], d["W2"], d["dY"])
    names = {"x": "dx", "g": "dgamma", "bb": "dbeta", "W1": "dw1", "b1": "db1", "W2": "dw2",
             "b2": "db2"}
    rng = np.random.default_rng(3)

    def loss(dd):
        y = o.project_rows(spec, dd["x"], dd["g"], dd["bb"], dd["W1"], dd["b1"], dd["W2"],
                           dd["b2"], nthreads=1)
        return float((y * d["dY"]).sum())

    h = 1e-5
    for n, gname in names.items():
        for _ in range(3):
            idx = tuple(int(rng.integers(0, s)) for s in d[n].shape)
            plus = {kk: v.copy() for kk, v in d.items()}
            minus = {kk: v.copy() for kk, v in d.items()}
            plus[n][idx] += h
            minus[n][idx] -= h
            fd = (loss(plus) - loss(minus)) / (2 * h)
            assert abs(fd - got[gname][idx]) <= 1e-6 * max(1.0, abs(fd)), (n, idx, fd,
                                                                             got[gname][idx])


def pin_backward_samples(o):
    """The sampled forms (one hidden unit; one pixel) equal the full gradients."""
    d, grids, C, k, H, O = _bwd_problem(13, C=4, k=3, H=6, O=5, grids=((4, 5), (3, 3)))
    for has_ln, act in ((True, o.GELU_ERF), (False, o.GELU_TANH)):
        spec = o.Spec(grids=grids, C=C, k=k, hidden=H, out_dim=O, views_per_image=[1, 1],
                      has_ln=has_ln, ln_eps=1e-6, act=act)
        args = (d["x"], d["g"], d["bb"], d["W1"], d["b1"], d["W2"], d["dY"])
        full = o.project_backward(spec, *args)
        for h in range(H):
            dw1, db1, dw2 = o.hidden_unit_grads(spec, *args, h)
            assert np.allclose(dw1, full["dw1"][h], rtol=1e-12, atol=1e-13)
            assert np.isclose(db1, full["db1"][h], rtol=1e-12, atol=1e-13)
            assert np.allclose(dw2, full["dw2"][:, h], rtol=1e-12, atol=1e-13)
        p = 0
        for v, (gh, gw) in enumerate(grids):
            for y in range(gh):
                for xx in range(gw):
                    got = o.pixel_grad(spec, *args, v, y, xx)
                    assert np.allclose(got, full["dx"][p + y * gw + xx], rtol=1e-12, atol=1e-13)
            p += gh * gw


def pin_scatter_backward(o):
    """The scatter's gradient equals autograd through masked_scatter of the
    assembled rows (newline and separator rows summed over their slots); a
    count mismatch is reported."""
    g = torch.Generator().manual_seed(5)
    S, D, T = 14, 3, 4
    src = np.array([2, -1, 0, -2, 3, -1, 1])
    mask = np.zeros(S, dtype=np.uint8)
    mask[[1, 2, 5, 6, 7, 10, 13]] = 1
    rows = torch.randn(T, D, generator=g, dtype=torch.float64, requires_grad=True)
    nl = torch.randn(D, generator=g, dtype=torch.float64, requires_grad=True)
    sp = torch.randn(D, generator=g, dtype=torch.float64, requires_grad=True)
    seq0 = torch.randn(S, D, generator=g, dtype=torch.float64)
    G = torch.randn(S, D, generator=g, dtype=torch.float64)
    A = torch.stack([rows[s] if s >= 0 else (nl if s == -1 else sp) for s in src])
    m = torch.from_numpy(mask).bool()[:, None].expand(S, D)
    (seq0.masked_scatter(m, A) * G).sum().backward()
    st, drows, dnl, dsp = o.scatter_backward(src, mask, G, T)
    assert st == 0
    assert np.allclose(drows, rows.grad.numpy(), rtol=1e-14, atol=0)
    assert np.allclose(dnl, nl.grad.numpy(), rtol=1e-14, atol=1e-15)
    assert np.allclose(dsp, sp.grad.numpy(), rtol=1e-14, atol=1e-15)
    for pos, val in ((0, 1), (5, 0)):  # one placeholder too many, one too few
        bad = mask.copy()
        bad[pos] = val
        assert o.scatter_backward(src, bad, G, T)[0] == -1


# --- processor (tile planning, placeholder expansion) -------------------------

def pin_processor_page_examples(o, pr=None):
    """[VL2] Processor step 7's worked counts through the planner: a 384 px tower
    with patch 14 gives 421 slots for a 1x1 grid and 617 for a 2x1 grid; patch
    16 gives 313 for 1x1.  Step 2 picks 1x1 for a square image (equal effective
    area, less waste) and the 2x1 candidate for a 2:1 image."""
    if pr is None:
        from oracle import processor as pr
    cands = [(384, 384), (768, 384), (384, 768)]
    plan = pr.plan_request([(384, 384), (800, 400)], cands, 14, 2)
    assert plan[0]["best"] == (384, 384) and plan[0]["tiles"] == (1, 1) and plan[0]["slots"] == 421
    assert plan[1]["best"] == (768, 384) and plan[1]["tiles"] == (2, 1) and plan[1]["slots"] == 617
    assert pr.plan_request([(640, 480)], [(384, 384)], 16, 2)[0]["slots"] == 313
    assert pr.merged_side(384, 14, 2) == 14 and pr.merged_side(384, 16, 2) == 12


def pin_processor_best_fit(o, pr=None):
    """Step 2 on hand-worked cases: the largest effective area wins even when it
    wastes more; the effective area is capped at the image's own area (no credit
    for upscaling); equal effective areas go to the smaller waste; full ties to
    the first candidate; floors are taken per side."""
    if pr is None:
        from oracle import processor as pr
    # 1000 x 500: (768, 384) fits 768 x 384 = 294912 (waste 0); (1152, 768) fits
    # 1152 x 576 = 663552 but is capped at 500000 (waste 384736); the larger area wins
    assert pr.best_resolution(1000, 500, [(768, 384), (1152, 768)]) == (1152, 768)
    # 300 x 200 upscales into both; both capped at 60000; (384, 384) wastes less
    assert pr.best_resolution(300, 200, [(768, 768), (384, 384)]) == (384, 384)
    # full tie: same size twice -> the first listed
    assert pr.best_resolution(500, 500, [(384, 768), (768, 384)]) == (384, 768)
    # 1000 x 300 into (384, 384): scale = min(0.384, 1.28) = 0.384;
    # floor(1000 * 0.384) = 384, floor(300 * 0.384) = floor(115.2) = 115
    sc = min(384 / 1000, 384 / 300)
    assert math.floor(1000 * sc) * math.floor(300 * sc) == 384 * 115
    assert pr.best_resolution(1000, 300, [(384, 384), (768, 384)]) == (768, 384)
    # fp64 as the page computes it: 737 x 738 into (384, 768) scales by 384/737, and
    # 737 * (384/737) evaluates to 383.99999999999994, so that side floors to 383:
    # 383 * floor(384.52...) = 147072; into (384, 384) (scale 384/738) the sides are
    # 383.47... and 384.00000000000006: 383 * 384 = 147072 as well.  Equal effective
    # areas, and (384, 384) wastes 384 against 147840.  (Flooring the product
    # instead would give 147656 against 147256 and pick (384, 768).)
    assert 737 * (384 / 737) == 383.99999999999994 and 738 * (384 / 738) == 384.00000000000006
    assert pr.best_resolution(737, 738, [(384, 768), (384, 384)]) == (384, 384)


def pin_processor_crop_rule(o, pr=None):
    """Step 1: at most two images are cropped; with three every image is 1x1."""
    if pr is None:
        from oracle import processor as pr
    cands = [(384, 384), (768, 384), (1152, 384)]
    two = pr.plan_request([(1200, 400), (1200, 400)], cands, 14, 2)
    assert [p["tiles"] for p in two] == [(3, 1), (3, 1)]
    three = pr.plan_request([(1200, 400)] * 3, cands, 14, 2)
    assert [p["tiles"] for p in three] == [(1, 1)] * 3 and [p["slots"] for p in three] == [421] * 3


def pin_processor_expand(o, pr=None):
    """Step 7: BOS first, each image token replaced by its image's count, in order;
    a prompt whose image tokens do not match the images is rejected."""
    if pr is None:
        from oracle import processor as pr
    img, bos = 9, 1
    got = pr.expand_prompt([5, img, 6, 7, img], img, [3, 2], bos)
    assert got == [1, 5, 9, 9, 9, 6, 7, 9, 9]
    for bad in ([5, 6], [img, img, img]):
        try:
            pr.expand_prompt(bad, img, [3, 2], bos)
        except ValueError:
            continue
        raise AssertionError("mismatched image tokens accepted")


PROCESSOR_PINS = [pin_processor_page_examples, pin_processor_best_fit, pin_processor_crop_rule,
                  pin_processor_expand]

ALL = [pin_page_counts, pin_param_count, pin_merged_width, pin_merge_roundtrip,
       pin_merge_pixel_unshuffle, pin_assembly_slots, pin_assembly_images, pin_gelu_values,
       pin_gelu_library, pin_linear_library, pin_layer_norm, pin_project_rows_library, pin_scatter,
       pin_embed_scatter, pin_project_rows_deep_library, pin_project_backward_autograd,
       pin_project_backward_deep_autograd, pin_project_backward_fd,
       pin_backward_samples, pin_scatter_backward] + PROCESSOR_PINS


def failing(o):
    """Names of the pins that fail (used by the mutation tests)."""
    bad = []
    for p in ALL:
        try:
            p(o)
        except Exception:  # noqa: BLE001 - any failure counts
            bad.append(p.__name__)
    return bad
