"""The C ABI without a GPU: the library loads and exports every entry point of
include/vlbridge.h; the host planner's sizes agree with the oracle; argument
validation returns its error codes before any HIP call is made."""
import ctypes as ct
import os
import re

import pytest

import common
from oracle import oracle as o
from patch_merge_mlp_amd import vlbridge as v
from patch_merge_mlp_amd import workloads as wl

HEADER = os.path.join(common.__file__.rsplit("/tests/", 1)[0], "include", "vlbridge.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vlb_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 13
    L = v.lib()
    for n in names:
        assert hasattr(L, n), n


def _batches():
    out = []
    for i in range(wl.N_CONFIGS):
        w = wl.config(i)
        wl.Generator(w)  # draws the ragged grids of the last workload
        out.append(w)
    # odd, rectangular, k=1 and tail variants
    out.append(wl.Workload("odd", 9, "bf16", 64, 3, 64, 64, 100, grids=[(5, 7), (1, 1), (9, 4)],
                           views_per_image=[2, 1]))
    out.append(wl.Workload("k1", 9, "bf16", 64, 1, 64, 64, 700, grids=[(24, 24)],
                           views_per_image=[1]))
    out.append(wl.Workload("tail", 9, "bf16", 64, 2, 64, 64, 4000, grids=[(27, 27)] * 7 + [(9, 9)] * 3,
                           views_per_image=[7, 3], tiled=True, tiles=[(3, 2), (1, 2)],
                           global_tail=True))
    return out


@pytest.mark.parametrize("w", _batches(), ids=lambda w: w.name)
def test_planner_sizes_match_oracle(w):
    p, b = common.lib_projector(w), common.lib_batch(w)
    spec = common.oracle_spec(w)
    assert v.vlb_num_tokens(p, b) == o.total_tokens(spec)
    assert v.vlb_num_slots(p, b) == len(o.assemble(spec))
    assert v.vlb_image_slots(p, b) == common.oracle_spans(w)
    ws = v.vlb_workspace_bytes(p, b, w.seq_len)
    assert ws > 0 and ws % 256 == 0


def test_config_slot_counts():
    """The tiled workload: 16 images of 210 + 1 + 42*29 slots; the text-only batch is empty."""
    w = wl.config(3)
    p, b = common.lib_projector(w), common.lib_batch(w)
    assert v.vlb_image_slots(p, b) == [1429] * 16
    assert v.vlb_num_slots(p, b) == 22864 <= w.seq_len
    empty = v.Batch([], [])
    assert v.vlb_num_tokens(p, empty) == 0 and v.vlb_num_slots(p, empty) == 0


# ---- validation: error codes, no HIP call --------------------------------------

FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def _proj(**kw):
    base = dict(dtype=v.BF16, C=64, k=2, hidden=128, out_dim=64)
    base.update(kw)
    return v.projector(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(k=4), v.ERR_UNSUPPORTED), (dict(k=0), v.ERR_UNSUPPORTED),
    (dict(dtype=7), v.ERR_DTYPE), (dict(C=0), v.ERR_SHAPE), (dict(C=12), v.ERR_UNSUPPORTED),
    (dict(C=72), v.ERR_UNSUPPORTED), (dict(hidden=100), v.ERR_UNSUPPORTED),
    (dict(C=4160), v.ERR_UNSUPPORTED), (dict(dtype=v.F32, C=2056, has_ln=True), v.ERR_UNSUPPORTED),
    (dict(act=5), v.ERR_UNSUPPORTED), (dict(has_ln=True, ln_eps=0.0), v.ERR_SHAPE),
    (dict(dtype=v.F32, packed=True), v.ERR_UNSUPPORTED),
    (dict(gather=v.GATHER_ON, dtype=v.F32), v.ERR_UNSUPPORTED),
    (dict(gather=v.GATHER_ON, has_ln=True), v.ERR_UNSUPPORTED),
    (dict(gather=3), v.ERR_UNSUPPORTED), (dict(gather=-1), v.ERR_UNSUPPORTED),
])
def test_bad_projector(kw, status):
    p = _proj(**kw)
    b = v.Batch([(4, 4)], [1])
    assert v.lib().vlb_num_tokens(ct.byref(p), ct.byref(b.c)) == -status


@pytest.mark.parametrize("batch,status", [
    (lambda: v.Batch([(0, 4)], [1]), v.ERR_SHAPE),
    (lambda: v.Batch([(4, 4)], [2]), v.ERR_SHAPE),
    (lambda: v.Batch([(4, 4), (4, 4)], [1]), v.ERR_SHAPE),
    (lambda: v.Batch([(4, 4)] * 3, [3], v.LAYOUT_TILED_2D, [(2, 2)]), v.ERR_SHAPE),
    (lambda: v.Batch([(4, 4), (4, 4), (6, 6)], [3], v.LAYOUT_TILED_2D, [(2, 1)]), v.ERR_SHAPE),
    (lambda: v.Batch([(4, 4)], [1], layout=5), v.ERR_UNSUPPORTED),
])
def test_bad_batch(batch, status):
    p = _proj()
    b = batch()
    assert v.lib().vlb_num_slots(ct.byref(p), ct.byref(b.c)) == -status


def test_entry_points_validate_before_launching():
    L = v.lib()
    p = _proj()
    b = v.Batch([(4, 4)], [1])
    need = v.vlb_workspace_bytes(p, b, 32)
    need0 = v.vlb_workspace_bytes(p, b, 0)
    assert 0 < need0 < need
    w = v.vlb_weights(None, None, FAKE, FAKE, FAKE, FAKE)
    # workspace too small
    assert L.vlb_merge_project(ct.byref(p), ct.byref(b.c), FAKE, ct.byref(w), FAKE, FAKE,
                               need0 - 1, None) == v.ERR_WORKSPACE
    assert L.vlb_bridge_fused(ct.byref(p), ct.byref(b.c), FAKE, ct.byref(w), None, None, FAKE, 32,
                              FAKE, FAKE, need - 1, None) == v.ERR_WORKSPACE
    # null and misaligned pointers
    assert L.vlb_merge_project(ct.byref(p), ct.byref(b.c), None, ct.byref(w), FAKE, FAKE, need,
                               None) == v.ERR_NULL
    assert L.vlb_merge_project(ct.byref(p), ct.byref(b.c), FAKE + 2, ct.byref(w), FAKE, FAKE, need,
                               None) == v.ERR_ALIGN
    wnull = v.vlb_weights(None, None, None, FAKE, FAKE, FAKE)
    assert L.vlb_merge_project(ct.byref(p), ct.byref(b.c), FAKE, ct.byref(wnull), FAKE, FAKE, need,
                               None) == v.ERR_NULL
    pln = _proj(has_ln=True)
    assert L.vlb_merge_project(ct.byref(pln), ct.byref(b.c), FAKE, ct.byref(w), FAKE, FAKE,
                               1 << 30, None) == v.ERR_NULL  # LN parameters missing
    assert L.vlb_scatter_tokens(ct.byref(p), ct.byref(b.c), FAKE, None, None, None, 32, FAKE, FAKE,
                                need, None) == v.ERR_NULL
    assert L.vlb_scatter_tokens(ct.byref(p), ct.byref(b.c), FAKE, None, None, FAKE + 1, 32, FAKE,
                                FAKE, need, None) == v.ERR_ALIGN
    bt = v.Batch([(4, 4)] * 2, [2], v.LAYOUT_TILED_2D, [(1, 1)])
    assert L.vlb_scatter_tokens(ct.byref(p), ct.byref(bt.c), FAKE, None, FAKE, FAKE, 64, FAKE, FAKE,
                                1 << 30, None) == v.ERR_NULL  # tiled needs the newline
    # pack: overlaps between any packed output and any input or the other output
    G = 1 << 24  # well apart
    for w1, w2, p1, p2 in [(FAKE, FAKE + G, FAKE, FAKE + 2 * G),          # w1_packed on w1
                           (FAKE, FAKE + G, FAKE + 2 * G, FAKE + G + 4096),  # w2_packed in w2
                           (FAKE, FAKE + G, FAKE + G - 4096, FAKE + 2 * G),  # w1_packed runs into w2
                           (FAKE, FAKE + G, FAKE + 2 * G, FAKE + 2 * G + 16)]:  # outputs overlap
        assert L.vlb_pack_weights(ct.byref(p), w1, w2, p1, p2, None) == v.ERR_UNSUPPORTED
    assert L.vlb_pack_weights(ct.byref(p), FAKE, None, FAKE + G, FAKE + 2 * G, None) == v.ERR_NULL
    assert L.vlb_pack_weights(ct.byref(p), FAKE, FAKE + G, FAKE + 2 * G + 8, FAKE + 3 * G,
                              None) == v.ERR_ALIGN
    pf = _proj(dtype=v.F32)
    assert L.vlb_pack_weights(ct.byref(pf), FAKE, FAKE + G, FAKE + 2 * G, FAKE + 3 * G,
                              None) == v.ERR_UNSUPPORTED
    assert L.vlb_merge_project(None, ct.byref(b.c), FAKE, ct.byref(w), FAKE, FAKE, need,
                               None) == v.ERR_NULL
    # text only: a successful no-op
    e = v.Batch([], [])
    assert L.vlb_bridge_fused(ct.byref(p), ct.byref(e.c), None, None, None, None, None, 0, None,
                              None, 0, None) == v.OK


def test_embed_validates_before_launching():
    """vlb_bridge_embed: the same checks as the fused call plus the token ids and the
    embedding table; text-only batches need no projector inputs."""
    L = v.lib()
    p = _proj()
    b = v.Batch([(4, 4)], [1])
    need = v.vlb_workspace_bytes(p, b, 32)
    w = v.vlb_weights(None, None, FAKE, FAKE, FAKE, FAKE)
    V = 1000

    def call(b=b, feats=FAKE, w=w, ids=FAKE, embed=FAKE, vocab=V, S=32, seq=FAKE, ws=FAKE,
             ws_bytes=need):
        return L.vlb_bridge_embed(ct.byref(p), ct.byref(b.c), feats, ct.byref(w) if w else None,
                                  None, None, ids, 5, embed, vocab, S, seq, ws, ws_bytes, None)

    assert call(ids=None) == v.ERR_NULL
    assert call(embed=None) == v.ERR_NULL
    assert call(ids=FAKE + 4) == v.ERR_ALIGN
    assert call(embed=FAKE + 8) == v.ERR_ALIGN
    assert call(vocab=0) == v.ERR_SHAPE
    assert call(vocab=1 << 31) == v.ERR_SHAPE
    assert call(S=0) == v.ERR_SHAPE
    assert call(feats=None) == v.ERR_NULL
    assert call(w=v.vlb_weights(None, None, None, FAKE, FAKE, FAKE)) == v.ERR_NULL
    assert call(ws_bytes=need - 1) == v.ERR_WORKSPACE
    # text only: features and weights may be null, the workspace still holds the status
    e = v.Batch([], [])
    need_e = v.vlb_workspace_bytes(p, e, 32)
    assert need_e > 0
    assert call(b=e, feats=None, w=None, ws_bytes=need_e - 1) == v.ERR_WORKSPACE


def test_training_entry_points_validate():
    """vlb_saved_bytes / vlb_backward_workspace_bytes sizes; the training forward and
    the backward reject fp32, packed weights (backward), missing or misaligned
    pointers and small buffers before launching anything."""
    L = v.lib()
    p = _proj(has_ln=True)
    b = v.Batch([(4, 4)], [1])
    T = v.vlb_num_tokens(p, b)
    K1 = p.C * p.k * p.k
    # bf16: blocked merged rows, then Z1 and act(Z1), 256-row blocks each
    assert v.vlb_saved_bytes(p, b) == 256 * K1 * 2 + 2 * 256 * p.hidden * 2
    # fp32: row-major merged rows (4 x 256) and Z1 (4 x 128), 256-byte aligned
    assert v.vlb_saved_bytes(_proj(dtype=v.F32), b) == 4 * K1 * 4 + 4 * p.hidden * 4
    need = v.vlb_backward_workspace_bytes(p, b, 32)
    assert need > 0
    assert v.vlb_backward_workspace_bytes(_proj(dtype=v.F32), b, 32) > 0
    assert v.vlb_backward_workspace_bytes(_proj(packed=True), b, 32) > 0
    # unpacked weights are packed into the backward workspace
    assert v.vlb_backward_workspace_bytes(_proj(), b, 32) > v.vlb_backward_workspace_bytes(
        _proj(packed=True), b, 32)
    assert v.vlb_backward_workspace_bytes(_proj(has_ln=True, C=2112), b, 32) == 0
    w = v.vlb_weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    fneed = v.vlb_workspace_bytes(p, b, 32)
    sneed = v.vlb_saved_bytes(p, b)
    G = 1 << 26

    def train(saved=FAKE + 2 * G, saved_bytes=sneed, proj=p, ws_bytes=fneed):
        return L.vlb_bridge_fused_train(ct.byref(proj), ct.byref(b.c), FAKE, ct.byref(w), None,
                                        None, FAKE, 32, FAKE + G, saved, saved_bytes, FAKE + 3 * G,
                                        ws_bytes, None)
    assert train(saved=None) == v.ERR_NULL
    assert train(saved=FAKE + 2 * G + 8) == v.ERR_ALIGN
    assert train(saved_bytes=sneed - 1) == v.ERR_WORKSPACE
    assert train(ws_bytes=fneed - 1) == v.ERR_WORKSPACE
    assert train(saved=FAKE + G) == v.ERR_UNSUPPORTED  # saved overlaps the sequence

    grads = v.vlb_grads(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)

    def bwd(proj=p, g=grads, wts=w, feats=FAKE, ws_bytes=need, saved_bytes=sneed, S=32):
        return L.vlb_bridge_backward(ct.byref(proj), ct.byref(b.c), feats, ct.byref(wts), FAKE, S,
                                     FAKE, FAKE, saved_bytes, ct.byref(g) if g else None, FAKE,
                                     ws_bytes, None)
    assert bwd(g=None) == v.ERR_NULL
    assert bwd(g=v.vlb_grads(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)) == v.ERR_NULL
    assert bwd(g=v.vlb_grads(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None)) == v.ERR_NULL
    assert bwd(g=v.vlb_grads(FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)) == v.ERR_ALIGN
    assert bwd(wts=v.vlb_weights(None, FAKE, FAKE, FAKE, FAKE, FAKE)) == v.ERR_NULL  # LN gamma
    assert bwd(feats=None) == v.ERR_NULL  # the LayerNorm backward reads the features
    assert bwd(ws_bytes=need - 1) == v.ERR_WORKSPACE
    assert bwd(saved_bytes=sneed - 1) == v.ERR_WORKSPACE
    assert bwd(S=0) == v.ERR_SHAPE
    bt = v.Batch([(4, 4)] * 2, [2], v.LAYOUT_TILED_2D, [(1, 1)])
    assert L.vlb_bridge_backward(ct.byref(p), ct.byref(bt.c), FAKE, ct.byref(w), FAKE, 64, FAKE,
                                 FAKE, 1 << 30, ct.byref(grads), FAKE, 1 << 30,
                                 None) == v.ERR_NULL  # tiled: newline / separator gradients


def test_depth_validation():
    """depth: 0 reads as 2, 1 is a shape error, above 16 unsupported; depth > 2 needs
    the middle weights, a larger workspace, and has no training entry points."""
    L = v.lib()
    b = v.Batch([(4, 4)], [1])
    assert v.vlb_num_tokens(_proj(depth=0), b) == v.vlb_num_tokens(_proj(), b) == 4
    assert v.lib().vlb_num_tokens(ct.byref(_proj(depth=1)), ct.byref(b.c)) == -v.ERR_SHAPE
    assert v.lib().vlb_num_tokens(ct.byref(_proj(depth=17)), ct.byref(b.c)) == -v.ERR_UNSUPPORTED
    assert v.vlb_num_tokens(_proj(depth=16), b) == 4
    p3 = _proj(depth=3)
    n2, n3 = v.vlb_workspace_bytes(_proj(), b, 32), v.vlb_workspace_bytes(p3, b, 32)
    # a second hidden buffer (256 x 128 bf16) and one packed middle weight (256 x 128)
    assert n3 - n2 == 2 * 256 * 128 * 2
    # saved: merged tokens, then the pre-activations and the activations of
    # Linear1 and the middle Linear
    assert v.vlb_saved_bytes(p3, b) == 256 * 256 * 2 + 4 * 256 * 128 * 2
    assert v.vlb_backward_workspace_bytes(p3, b, 32) > v.vlb_backward_workspace_bytes(_proj(), b, 32)

    def fused(w, proj=p3):
        return L.vlb_bridge_fused(ct.byref(proj), ct.byref(b.c), FAKE, ct.byref(w), None, None,
                                  FAKE, 32, FAKE + (1 << 26), FAKE + (2 << 26), n3, None)
    arr = lambda *xs: ct.cast((ct.c_void_p * len(xs))(*xs), ct.POINTER(ct.c_void_p))
    w_none = v.vlb_weights(None, None, FAKE, FAKE, FAKE, FAKE, None, None)
    assert fused(w_none) == v.ERR_NULL
    assert fused(v.vlb_weights(None, None, FAKE, FAKE, FAKE, FAKE, arr(None), arr(FAKE))) == v.ERR_NULL
    assert fused(v.vlb_weights(None, None, FAKE, FAKE, FAKE, FAKE, arr(FAKE + 2), arr(FAKE))) == v.ERR_ALIGN
    assert L.vlb_bridge_fused_train(ct.byref(p3), ct.byref(b.c), FAKE, ct.byref(w_none), None,
                                    None, FAKE, 32, FAKE, FAKE, 1 << 30, FAKE, 1 << 30,
                                    None) == v.ERR_NULL  # the middle weights are missing
    g_no_mid = v.vlb_grads(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None, None, None)
    w_mid = v.vlb_weights(None, None, FAKE, FAKE, FAKE, FAKE, arr(FAKE), arr(FAKE))
    assert L.vlb_bridge_backward(ct.byref(p3), ct.byref(b.c), FAKE, ct.byref(w_mid), FAKE, 32,
                                 FAKE, FAKE, 1 << 30, ct.byref(g_no_mid), FAKE, 1 << 30,
                                 None) == v.ERR_NULL  # the middle gradients are missing
    assert L.vlb_pack_mid(ct.byref(p3), FAKE, FAKE + 1024, None) == v.ERR_UNSUPPORTED  # overlap
    assert L.vlb_pack_mid(ct.byref(_proj(dtype=v.F32)), FAKE, FAKE + (1 << 26), None) == v.ERR_UNSUPPORTED
    assert L.vlb_pack_mid(ct.byref(p3), None, FAKE, None) == v.ERR_NULL


def test_packed_bytes():
    """Tile-blocked weights: rows padded to a multiple of 256, K unchanged."""
    p = _proj()  # C=64, k=2 -> K1=256; hidden=128; out_dim=64
    assert v.vlb_packed_bytes(p, 1) == 256 * 256 * 2
    assert v.vlb_packed_bytes(p, 2) == 256 * 128 * 2
    big = _proj(C=1152, hidden=4608, out_dim=4096)
    assert v.vlb_packed_bytes(big, 1) == 4608 * 4608 * 2
    assert v.vlb_packed_bytes(big, 2) == 4096 * 4608 * 2
    assert v.vlb_packed_bytes(p, 3) == 256 * 128 * 2  # a middle weight [hidden][hidden]
    assert v.vlb_packed_bytes(p, 0) == 0 and v.vlb_packed_bytes(p, 4) == 0
    assert v.vlb_packed_bytes(_proj(dtype=v.F32), 1) == 0
    assert v.vlb_packed_bytes(_proj(k=9), 1) == 0


def test_status_strings():
    for s in range(10):
        assert v.status_str(s)
    assert "placeholder" in v.status_str(v.ERR_MASK_COUNT)


def test_operand_size_limits():
    """Every GEMM operand is addressed with 32-bit byte offsets (buffer loads), so each must
    stay under 2 GiB: the features, the packed W1, the hidden activation and the sequence.
    One past each limit is rejected before any launch, the largest size inside is accepted."""
    L = v.lib()

    def tokens(p, b):
        return L.vlb_num_tokens(ct.byref(p), ct.byref(b.c))

    # features: 1024 x 910 x 1152 bf16 = 2,146,959,360 B; one more column passes 2^31 - 1
    p = v.projector(v.BF16, 1152, 2, 4608, 4096)
    assert tokens(p, v.Batch([(1024, 910)], [1])) == 512 * 455
    assert tokens(p, v.Batch([(1024, 911)], [1])) == -v.ERR_SHAPE
    # packed W1 (256-row blocks): 58112 x 18432 bf16 fits, 58368 x 18432 does not
    small = v.Batch([(6, 6)], [1])
    assert tokens(v.projector(v.BF16, 2048, 3, 58112, 64), small) == 4
    assert tokens(v.projector(v.BF16, 2048, 3, 58368, 64), small) == -v.ERR_SHAPE
    # hidden activation, tile-blocked in 256-row blocks: 32512 x 32768 bf16 fits; 32513 rows
    # round up to 32768 rows = 2^31 bytes
    ph = v.projector(v.BF16, 64, 1, 32768, 64)
    assert tokens(ph, v.Batch([(32512, 1)], [1])) == 32512
    assert tokens(ph, v.Batch([(32513, 1)], [1])) == -v.ERR_SHAPE
    # sequence: seq_len x out_dim elements
    ps = v.projector(v.BF16, 64, 2, 128, 4096)
    b = v.Batch([(4, 4)], [1])
    assert L.vlb_workspace_bytes(ct.byref(ps), ct.byref(b.c), (1 << 19) - 1) > 0
    assert L.vlb_workspace_bytes(ct.byref(ps), ct.byref(b.c), 1 << 19) == 0


def test_gather_mode_workspace():
    """Gathering drops the merged tokens from the workspace (T rounded up to 256
    rows of C*k*k bf16).  The automatic choice gathers for bf16 without
    LayerNorm up to hidden 4096; fp32 and the LayerNorm keep their own layout.
    The training sizes do not depend on the flag."""
    b = v.Batch([(9, 7), (4, 4)], [1, 1])
    T = v.vlb_num_tokens(_proj(), b)
    assert T == 5 * 4 + 4
    merged = 256 * 64 * 4 * 2
    off = v.vlb_workspace_bytes(_proj(gather=v.GATHER_OFF), b, 32)
    on = v.vlb_workspace_bytes(_proj(gather=v.GATHER_ON), b, 32)
    assert off - on == merged
    assert v.vlb_workspace_bytes(_proj(), b, 32) == on                      # auto, hidden 128
    big = dict(hidden=4160, out_dim=64)
    assert (v.vlb_workspace_bytes(_proj(**big), b, 32)
            - v.vlb_workspace_bytes(_proj(gather=v.GATHER_ON, **big), b, 32)) == merged
    assert (v.vlb_workspace_bytes(_proj(has_ln=True), b, 32)
            == v.vlb_workspace_bytes(_proj(has_ln=True, gather=v.GATHER_OFF), b, 32))
    assert v.vlb_workspace_bytes(_proj(dtype=v.F32), b, 32) == \
        v.vlb_workspace_bytes(_proj(dtype=v.F32, gather=v.GATHER_OFF), b, 32)
    assert v.vlb_saved_bytes(_proj(gather=v.GATHER_ON), b) == v.vlb_saved_bytes(_proj(), b)


def test_noalloc_validates_before_launching():
    """vlb_bridge_fused_noalloc: argument errors and the scratch limit are found on
    the host, before any HIP call (no GPU here).  A LayerNorm batch keeps its
    merged tokens, so 16 MoonViT-size images need 151 + 151 MB > 256 MiB."""
    L = v.lib()
    p = _proj(C=1152, hidden=4608, out_dim=4096, has_ln=True)
    b = v.Batch([(64, 64)] * 16, [1] * 16)
    S = 16 * 1024 + 8
    need = v.vlb_workspace_bytes(p, b, S)
    assert need > v.NOALLOC_SCRATCH_BYTES
    w = v.vlb_weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    call = lambda pp, bb, status: L.vlb_bridge_fused_noalloc(
        ct.byref(pp), ct.byref(bb.c), FAKE, ct.byref(w), FAKE, FAKE, FAKE, S, FAKE, status, None)
    assert call(p, b, FAKE) == v.ERR_SCRATCH
    assert call(p, b, None) == v.ERR_NULL
    assert call(p, b, FAKE + 4) == v.ERR_ALIGN
    bad = _proj(C=1152, hidden=4608, out_dim=4096, has_ln=True, gather=v.GATHER_ON)
    assert call(bad, b, FAKE) == v.ERR_UNSUPPORTED
    # the same images without the LayerNorm fit: the merged tokens are gathered
    p2 = _proj(C=1152, hidden=4608, out_dim=4096)
    assert v.vlb_workspace_bytes(_proj(C=1152, hidden=4608, out_dim=4096,
                                       gather=v.GATHER_ON), b, S) <= v.NOALLOC_SCRATCH_BYTES
    assert v.vlb_workspace_bytes(_proj(C=1152, hidden=4608, out_dim=4096,
                                       gather=v.GATHER_OFF), b, S) > v.NOALLOC_SCRATCH_BYTES
    assert v.status_str(v.ERR_SCRATCH) == "problem too large for the no-allocation scratch"
    del p2
