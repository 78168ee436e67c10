"""Python binding of the vlbridge C ABI (include/vlbridge.h).

Argument marshalling only: every step of the bridge runs in the HIP kernels of
libvlbridge.so.  Tensors supply device pointers, torch's current stream
supplies the HIP stream.  The functions keep the C names; each raises VlbError
(with .status) when the library returns an error.  Sizes of the tensors handed
in are checked here against what the library will read or write.
"""
from __future__ import annotations

import ctypes as ct
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; VLBRIDGE_LIB names another build of the same sources (the
# CPU tests' sanitizer build of the host code).
LIB_PATH = os.environ.get("VLBRIDGE_LIB") or os.path.join(_HERE, "libvlbridge.so")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_WORKSPACE, ERR_MASK_COUNT, \
    ERR_UNSUPPORTED, ERR_HIP, ERR_TOKEN_ID, ERR_SCRATCH = range(11)
NOALLOC_SCRATCH_BYTES = 256 << 20  # VLB_NOALLOC_SCRATCH_BYTES
F32, BF16 = 0, 1
GELU_ERF, GELU_TANH, ACT_NONE = 0, 1, 2
LAYOUT_PLAIN, LAYOUT_TILED_2D = 0, 1
GATHER_AUTO, GATHER_ON, GATHER_OFF = 0, 1, 2
K_PLAN, K_SCAN, K_PLACE, K_LN, K_GEMM1, K_GEMM2, K_SCATTER, K_MERGE, K_PACK, K_EMBED, \
    K_BWD_PACK, K_BWD_DW2, K_BWD_DA1, K_BWD_DW1, K_BWD_DX, K_BWD_UNMERGE, K_BWD_SUM, \
    K_GEMM_MID = range(18)
KERNEL_NAMES = ["plan", "scan", "place", "layernorm", "gemm1", "gemm2", "scatter", "merge", "pack",
                "embed", "bwd_pack", "bwd_dw2", "bwd_da1", "bwd_dw1", "bwd_dx", "bwd_unmerge",
                "bwd_sum", "gemm_mid"]


class VlbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class vlb_projector(ct.Structure):
    _fields_ = [("dtype", ct.c_int32), ("C", ct.c_int32), ("k", ct.c_int32),
                ("hidden", ct.c_int32), ("out_dim", ct.c_int32), ("has_ln", ct.c_int32),
                ("ln_eps", ct.c_float), ("act", ct.c_int32), ("packed", ct.c_int32),
                ("depth", ct.c_int32), ("gather", ct.c_int32)]


class vlb_weights(ct.Structure):
    _fields_ = [("ln_gamma", ct.c_void_p), ("ln_beta", ct.c_void_p), ("w1", ct.c_void_p),
                ("b1", ct.c_void_p), ("w2", ct.c_void_p), ("b2", ct.c_void_p),
                ("w_mid", ct.POINTER(ct.c_void_p)), ("b_mid", ct.POINTER(ct.c_void_p))]


_P32 = ct.POINTER(ct.c_int32)


class vlb_grads(ct.Structure):
    _fields_ = [("d_features", ct.c_void_p), ("d_w1", ct.c_void_p), ("d_b1", ct.c_void_p),
                ("d_w2", ct.c_void_p), ("d_b2", ct.c_void_p), ("d_ln_gamma", ct.c_void_p),
                ("d_ln_beta", ct.c_void_p), ("d_newline", ct.c_void_p),
                ("d_separator", ct.c_void_p), ("d_w_mid", ct.POINTER(ct.c_void_p)),
                ("d_b_mid", ct.POINTER(ct.c_void_p))]


class vlb_batch(ct.Structure):
    _fields_ = [("n_views", ct.c_int32), ("grid_h", _P32), ("grid_w", _P32),
                ("n_images", ct.c_int32), ("views_per_image", _P32), ("layout", ct.c_int32),
                ("tile_w", _P32), ("tile_h", _P32), ("global_view_tail", ct.c_int32)]


class vlb_processor(ct.Structure):
    _fields_ = [("candidates", _P32), ("n_candidates", ct.c_int32), ("patch_size", ct.c_int32),
                ("downsample", ct.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"vlbridge HIP library missing at {LIB_PATH}: build it first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ct.CDLL(LIB_PATH)
        pp, pb, vp, i64, sz = (ct.POINTER(vlb_projector), ct.POINTER(vlb_batch), ct.c_void_p,
                               ct.c_int64, ct.c_size_t)
        st = ct.c_int
        sigs = {
            "vlb_num_tokens": (i64, [pp, pb]),
            "vlb_num_slots": (i64, [pp, pb]),
            "vlb_image_slots": (i64, [pp, pb, ct.POINTER(ct.c_int64)]),
            "vlb_workspace_bytes": (sz, [pp, pb, i64]),
            "vlb_packed_bytes": (sz, [pp, ct.c_int32]),
            "vlb_pack_weights": (st, [pp, vp, vp, vp, vp, vp]),
            "vlb_pack_mid": (st, [pp, vp, vp, vp]),
            "vlb_merge_tokens": (st, [pp, pb, vp, vp, vp, vp, vp, sz, vp]),
            "vlb_merge_project": (st, [pp, pb, vp, ct.POINTER(vlb_weights), vp, vp, sz, vp]),
            "vlb_scatter_tokens": (st, [pp, pb, vp, vp, vp, vp, i64, vp, vp, sz, vp]),
            "vlb_bridge_fused": (st, [pp, pb, vp, ct.POINTER(vlb_weights), vp, vp, vp, i64, vp,
                                      vp, sz, vp]),
            "vlb_bridge_fused_noalloc": (st, [pp, pb, vp, ct.POINTER(vlb_weights), vp, vp, vp,
                                              i64, vp, vp, vp]),
            "vlb_bridge_embed": (st, [pp, pb, vp, ct.POINTER(vlb_weights), vp, vp, vp, ct.c_int32,
                                      vp, i64, i64, vp, vp, sz, vp]),
            "vlb_saved_bytes": (sz, [pp, pb]),
            "vlb_backward_workspace_bytes": (sz, [pp, pb, i64]),
            "vlb_bridge_fused_train": (st, [pp, pb, vp, ct.POINTER(vlb_weights), vp, vp, vp, i64,
                                            vp, vp, sz, vp, sz, vp]),
            "vlb_bridge_backward": (st, [pp, pb, vp, ct.POINTER(vlb_weights), vp, i64, vp, vp, sz,
                                         ct.POINTER(vlb_grads), vp, sz, vp]),
            "vlb_select_resolution": (st, [ct.POINTER(vlb_processor), ct.c_int32, ct.c_int32,
                                           _P32]),
            "vlb_plan_request": (st, [ct.POINTER(vlb_processor), ct.c_int32, _P32, _P32,
                                      ct.POINTER(ct.c_int64)]),
            "vlb_expand_prompt": (i64, [_P32, i64, ct.c_int32, ct.c_int32, ct.POINTER(ct.c_int64),
                                        ct.c_int32, _P32, i64]),
            "vlb_check": (st, [vp, vp]),
            "vlb_status_str": (ct.c_char_p, [st]),
            "vlb_prof_enable": (st, [ct.c_int32]),
            "vlb_prof_resume": (st, [ct.c_int32]),
            "vlb_prof_read": (st, [ct.c_int32, ct.POINTER(ct.c_int64), ct.POINTER(ct.c_double)]),
        }
        for name, (res, args) in sigs.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().vlb_status_str(s).decode()


def _check(status: int, where: str):
    if status != OK:
        raise VlbError(status, where)


def projector(dtype: int, C: int, k: int, hidden: int, out_dim: int, has_ln: bool = False,
              ln_eps: float = 1e-6, act: int = GELU_ERF, packed: bool = False,
              depth: int = 2, gather: int = 0) -> vlb_projector:
    return vlb_projector(dtype, C, k, hidden, out_dim, int(has_ln), ln_eps, act, int(packed),
                         depth, int(gather))


def _depth(p: vlb_projector) -> int:
    return 2 if p.depth == 0 else p.depth


class Batch:
    """Host-side batch description (keeps its int32 arrays alive for the C struct)."""

    def __init__(self, grids: Sequence[tuple], views_per_image: Sequence[int],
                 layout: int = LAYOUT_PLAIN, tiles: Optional[Sequence[tuple]] = None,
                 global_view_tail: bool = False):
        self.grids = [tuple(g) for g in grids]
        self.views_per_image = list(views_per_image)
        self.layout = layout
        self.tiles = list(tiles or [])
        arr = lambda xs: (ct.c_int32 * max(len(xs), 1))(*xs)
        self._gh = arr([g[0] for g in self.grids])
        self._gw = arr([g[1] for g in self.grids])
        self._vpi = arr(self.views_per_image)
        self._tw = arr([t[0] for t in self.tiles])
        self._th = arr([t[1] for t in self.tiles])
        self.c = vlb_batch(len(self.grids), self._gh, self._gw, len(self.views_per_image),
                           self._vpi, layout, self._tw, self._th, int(global_view_tail))


@dataclass
class Weights:
    w1: torch.Tensor
    b1: torch.Tensor
    w2: torch.Tensor
    b2: torch.Tensor
    ln_gamma: Optional[torch.Tensor] = None
    ln_beta: Optional[torch.Tensor] = None
    w_mid: Sequence[torch.Tensor] = ()   # depth > 2: [hidden][hidden] each (or packed forms)
    b_mid: Sequence[torch.Tensor] = ()   # [hidden] each

    def c(self) -> vlb_weights:
        # the pointer arrays live on the returned struct (kept with it)
        wm = (ct.c_void_p * max(len(self.w_mid), 1))(*[_ptr(t) for t in self.w_mid])
        bm = (ct.c_void_p * max(len(self.b_mid), 1))(*[_ptr(t) for t in self.b_mid])
        c = vlb_weights(_ptr(self.ln_gamma), _ptr(self.ln_beta), _ptr(self.w1), _ptr(self.b1),
                        _ptr(self.w2), _ptr(self.b2),
                        ct.cast(wm, ct.POINTER(ct.c_void_p)) if self.w_mid else None,
                        ct.cast(bm, ct.POINTER(ct.c_void_p)) if self.b_mid else None)
        c._keep = (wm, bm)
        return c


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("vlbridge takes device tensors")
    if not t.is_contiguous():
        raise ValueError("vlbridge takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _tdtype(p: vlb_projector):
    return torch.float32 if p.dtype == F32 else torch.bfloat16


def _need(t: Optional[torch.Tensor], n: int, dtype, what: str):
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if t.numel() < n:
        raise ValueError(f"{what}: {t.numel()} elements, need {n}")


def _pixels(b: Batch) -> int:
    return sum(gh * gw for gh, gw in b.grids)


# ---- sizing ------------------------------------------------------------------

def vlb_num_tokens(p: vlb_projector, b: Batch) -> int:
    n = lib().vlb_num_tokens(ct.byref(p), ct.byref(b.c))
    if n < 0:
        raise VlbError(-n, "vlb_num_tokens")
    return n


def vlb_num_slots(p: vlb_projector, b: Batch) -> int:
    n = lib().vlb_num_slots(ct.byref(p), ct.byref(b.c))
    if n < 0:
        raise VlbError(-n, "vlb_num_slots")
    return n


def vlb_image_slots(p: vlb_projector, b: Batch) -> list:
    out = (ct.c_int64 * max(len(b.views_per_image), 1))()
    n = lib().vlb_image_slots(ct.byref(p), ct.byref(b.c), out)
    if n < 0:
        raise VlbError(-n, "vlb_image_slots")
    return [int(out[i]) for i in range(len(b.views_per_image))]


def vlb_workspace_bytes(p: vlb_projector, b: Batch, seq_len: int) -> int:
    return int(lib().vlb_workspace_bytes(ct.byref(p), ct.byref(b.c), seq_len))


def workspace(p: vlb_projector, b: Batch, seq_len: int, device="cuda") -> torch.Tensor:
    n = vlb_workspace_bytes(p, b, seq_len)
    if n == 0:
        raise VlbError(ERR_SHAPE, "vlb_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


# ---- entry points -----------------------------------------------------------

def vlb_packed_bytes(p: vlb_projector, which: int) -> int:
    return int(lib().vlb_packed_bytes(ct.byref(p), which))


def vlb_pack_weights(p: vlb_projector, w1: torch.Tensor, w2: torch.Tensor,
                     w1_packed: torch.Tensor, w2_packed: torch.Tensor, stream=None):
    dt = _tdtype(p)
    _need(w1, p.hidden * p.C * p.k * p.k, dt, "w1")
    _need(w2, p.out_dim * p.hidden, dt, "w2")
    for t, which, what in ((w1_packed, 1, "w1_packed"), (w2_packed, 2, "w2_packed")):
        n = vlb_packed_bytes(p, which)
        if n == 0:
            raise VlbError(ERR_UNSUPPORTED, "vlb_packed_bytes")
        _need(t, n // 2, dt, what)
    _check(lib().vlb_pack_weights(ct.byref(p), _ptr(w1), _ptr(w2), _ptr(w1_packed),
                                  _ptr(w2_packed), _stream(stream)), "vlb_pack_weights")


def vlb_pack_mid(p: vlb_projector, w: torch.Tensor, w_packed: torch.Tensor, stream=None):
    dt = _tdtype(p)
    _need(w, p.hidden * p.hidden, dt, "w_mid")
    _need(w_packed, vlb_packed_bytes(p, 3) // 2, dt, "w_mid_packed")
    _check(lib().vlb_pack_mid(ct.byref(p), _ptr(w), _ptr(w_packed), _stream(stream)),
           "vlb_pack_mid")


def _check_weights(p, w: Weights):
    dt = _tdtype(p)
    if p.packed:
        _need(w.w1, vlb_packed_bytes(p, 1) // 2, dt, "w1 (packed)")
        _need(w.w2, vlb_packed_bytes(p, 2) // 2, dt, "w2 (packed)")
    else:
        _need(w.w1, p.hidden * p.C * p.k * p.k, dt, "w1")
        _need(w.w2, p.out_dim * p.hidden, dt, "w2")
    _need(w.b1, p.hidden, dt, "b1")
    _need(w.b2, p.out_dim, dt, "b2")
    _need(w.ln_gamma, p.C, dt, "ln_gamma")
    _need(w.ln_beta, p.C, dt, "ln_beta")
    n_mid = _depth(p) - 2
    if len(w.w_mid) != n_mid or len(w.b_mid) != n_mid:
        raise ValueError(f"depth {_depth(p)} needs {n_mid} middle weights and biases")
    for q in range(n_mid):
        _need(w.w_mid[q], vlb_packed_bytes(p, 3) // 2 if p.packed else p.hidden * p.hidden, dt,
              f"w_mid[{q}]")
        _need(w.b_mid[q], p.hidden, dt, f"b_mid[{q}]")


def vlb_merge_tokens(p, b: Batch, features, ln_gamma, ln_beta, merged, ws, stream=None):
    dt = _tdtype(p)
    _need(features, _pixels(b) * p.C, dt, "features")
    _need(merged, vlb_num_tokens(p, b) * p.C * p.k * p.k, dt, "merged")
    _need(ln_gamma, p.C, dt, "ln_gamma")
    _need(ln_beta, p.C, dt, "ln_beta")
    _check(lib().vlb_merge_tokens(ct.byref(p), ct.byref(b.c), _ptr(features), _ptr(ln_gamma),
                                  _ptr(ln_beta), _ptr(merged), _ptr(ws), ws.numel(),
                                  _stream(stream)), "vlb_merge_tokens")


def vlb_merge_project(p, b: Batch, features, w: Weights, rows, ws, stream=None):
    dt = _tdtype(p)
    _need(features, _pixels(b) * p.C, dt, "features")
    _check_weights(p, w)
    _need(rows, vlb_num_tokens(p, b) * p.out_dim, dt, "rows")
    wc = w.c()
    _check(lib().vlb_merge_project(ct.byref(p), ct.byref(b.c), _ptr(features), ct.byref(wc),
                                   _ptr(rows), _ptr(ws), ws.numel(), _stream(stream)),
           "vlb_merge_project")


def _check_seq(p, mask, seq):
    if mask.dtype != torch.uint8:
        raise ValueError("mask must be uint8")
    if seq.dim() != 2 or seq.shape[1] != p.out_dim or mask.numel() != seq.shape[0]:
        raise ValueError("seq must be [seq_len, out_dim] and mask [seq_len]")
    if seq.dtype != _tdtype(p):
        raise ValueError(f"seq dtype {seq.dtype}")


def vlb_scatter_tokens(p, b: Batch, rows, newline, separator, mask, seq, ws, stream=None):
    dt = _tdtype(p)
    _check_seq(p, mask, seq)
    _need(rows, vlb_num_tokens(p, b) * p.out_dim, dt, "rows")
    _need(newline, p.out_dim, dt, "newline")
    _need(separator, p.out_dim, dt, "separator")
    _check(lib().vlb_scatter_tokens(ct.byref(p), ct.byref(b.c), _ptr(rows), _ptr(newline),
                                    _ptr(separator), _ptr(mask), seq.shape[0], _ptr(seq),
                                    _ptr(ws), ws.numel(), _stream(stream)), "vlb_scatter_tokens")


def vlb_bridge_fused(p, b: Batch, features, w: Weights, newline, separator, mask, seq, ws,
                     stream=None):
    dt = _tdtype(p)
    _check_seq(p, mask, seq)
    _need(features, _pixels(b) * p.C, dt, "features")
    _check_weights(p, w)
    _need(newline, p.out_dim, dt, "newline")
    _need(separator, p.out_dim, dt, "separator")
    wc = w.c()
    _check(lib().vlb_bridge_fused(ct.byref(p), ct.byref(b.c), _ptr(features), ct.byref(wc),
                                  _ptr(newline), _ptr(separator), _ptr(mask), seq.shape[0],
                                  _ptr(seq), _ptr(ws), ws.numel(), _stream(stream)),
           "vlb_bridge_fused")


def vlb_bridge_fused_noalloc(p, b: Batch, features, w: Weights, newline, separator, mask, seq,
                             status, stream=None):
    """vlb_bridge_fused with the library's own device scratch instead of a
    workspace; status: int32 [4] on the device, the call's status words (read
    them with vlb_check(status))."""
    dt = _tdtype(p)
    _check_seq(p, mask, seq)
    _need(features, _pixels(b) * p.C, dt, "features")
    _check_weights(p, w)
    _need(newline, p.out_dim, dt, "newline")
    _need(separator, p.out_dim, dt, "separator")
    _need(status, 4, torch.int32, "status")
    wc = w.c()
    _check(lib().vlb_bridge_fused_noalloc(ct.byref(p), ct.byref(b.c), _ptr(features), ct.byref(wc),
                                          _ptr(newline), _ptr(separator), _ptr(mask), seq.shape[0],
                                          _ptr(seq), _ptr(status), _stream(stream)),
           "vlb_bridge_fused_noalloc")


def vlb_bridge_embed(p, b: Batch, features, w: Weights, newline, separator, ids, image_token_id,
                     embed, seq, ws, stream=None):
    """Every row of seq: text positions from the embedding table, image-token
    positions from the bridge (see vlb_bridge_embed in the header)."""
    dt = _tdtype(p)
    if ids.dtype != torch.int32 or ids.dim() != 1:
        raise ValueError("ids must be int32 [seq_len]")
    if seq.dim() != 2 or seq.shape[1] != p.out_dim or seq.shape[0] != ids.numel():
        raise ValueError("seq must be [seq_len, out_dim]")
    if seq.dtype != dt or embed.dtype != dt or embed.dim() != 2 or embed.shape[1] != p.out_dim:
        raise ValueError("seq / embed dtype or shape")
    T = vlb_num_tokens(p, b)
    if T > 0:
        _need(features, _pixels(b) * p.C, dt, "features")
        _check_weights(p, w)
        _need(newline, p.out_dim, dt, "newline")
        _need(separator, p.out_dim, dt, "separator")
    wc = w.c() if w is not None else vlb_weights()
    _check(lib().vlb_bridge_embed(ct.byref(p), ct.byref(b.c), _ptr(features), ct.byref(wc),
                                  _ptr(newline), _ptr(separator), _ptr(ids), int(image_token_id),
                                  _ptr(embed), embed.shape[0], seq.shape[0], _ptr(seq), _ptr(ws),
                                  ws.numel(), _stream(stream)), "vlb_bridge_embed")


# ---- training --------------------------------------------------------------

def vlb_saved_bytes(p: vlb_projector, b: Batch) -> int:
    return int(lib().vlb_saved_bytes(ct.byref(p), ct.byref(b.c)))


def vlb_backward_workspace_bytes(p: vlb_projector, b: Batch, seq_len: int) -> int:
    return int(lib().vlb_backward_workspace_bytes(ct.byref(p), ct.byref(b.c), seq_len))


def vlb_bridge_fused_train(p, b: Batch, features, w: Weights, newline, separator, mask, seq,
                           saved, ws, stream=None):
    dt = _tdtype(p)
    _check_seq(p, mask, seq)
    _need(features, _pixels(b) * p.C, dt, "features")
    _check_weights(p, w)
    _need(newline, p.out_dim, dt, "newline")
    _need(separator, p.out_dim, dt, "separator")
    if saved.dtype != torch.uint8:
        raise ValueError("saved must be a uint8 buffer")
    wc = w.c()
    _check(lib().vlb_bridge_fused_train(ct.byref(p), ct.byref(b.c), _ptr(features), ct.byref(wc),
                                        _ptr(newline), _ptr(separator), _ptr(mask), seq.shape[0],
                                        _ptr(seq), _ptr(saved), saved.numel(), _ptr(ws),
                                        ws.numel(), _stream(stream)), "vlb_bridge_fused_train")


@dataclass
class Grads:
    """Gradient outputs (fp32 except d_features, in the projector dtype)."""
    d_w1: torch.Tensor
    d_b1: torch.Tensor
    d_w2: torch.Tensor
    d_b2: torch.Tensor
    d_features: Optional[torch.Tensor] = None
    d_ln_gamma: Optional[torch.Tensor] = None
    d_ln_beta: Optional[torch.Tensor] = None
    d_newline: Optional[torch.Tensor] = None
    d_separator: Optional[torch.Tensor] = None
    d_w_mid: Sequence[torch.Tensor] = ()   # depth > 2: [hidden][hidden] each
    d_b_mid: Sequence[torch.Tensor] = ()   # [hidden] each

    @staticmethod
    def empty(p: vlb_projector, b: Batch, features=True, device="cuda") -> "Grads":
        f32 = dict(dtype=torch.float32, device=device)
        K1 = p.C * p.k * p.k
        g = Grads(torch.empty(p.hidden, K1, **f32), torch.empty(p.hidden, **f32),
                  torch.empty(p.out_dim, p.hidden, **f32), torch.empty(p.out_dim, **f32))
        if features:
            g.d_features = torch.empty(_pixels(b), p.C, dtype=_tdtype(p), device=device)
        if p.has_ln:
            g.d_ln_gamma = torch.empty(p.C, **f32)
            g.d_ln_beta = torch.empty(p.C, **f32)
        if b.layout == LAYOUT_TILED_2D:
            g.d_newline = torch.empty(p.out_dim, **f32)
            g.d_separator = torch.empty(p.out_dim, **f32)
        n_mid = _depth(p) - 2
        g.d_w_mid = [torch.empty(p.hidden, p.hidden, **f32) for _ in range(n_mid)]
        g.d_b_mid = [torch.empty(p.hidden, **f32) for _ in range(n_mid)]
        return g

    def c(self) -> vlb_grads:
        wm = (ct.c_void_p * max(len(self.d_w_mid), 1))(*[_ptr(t) for t in self.d_w_mid])
        bm = (ct.c_void_p * max(len(self.d_b_mid), 1))(*[_ptr(t) for t in self.d_b_mid])
        c = vlb_grads(_ptr(self.d_features), _ptr(self.d_w1), _ptr(self.d_b1), _ptr(self.d_w2),
                      _ptr(self.d_b2), _ptr(self.d_ln_gamma), _ptr(self.d_ln_beta),
                      _ptr(self.d_newline), _ptr(self.d_separator),
                      ct.cast(wm, ct.POINTER(ct.c_void_p)) if self.d_w_mid else None,
                      ct.cast(bm, ct.POINTER(ct.c_void_p)) if self.d_b_mid else None)
        c._keep = (wm, bm)
        return c


def vlb_bridge_backward(p, b: Batch, features, w: Weights, mask, dseq, saved, g: Grads, ws,
                        stream=None):
    dt = _tdtype(p)
    _check_seq(p, mask, dseq)
    _need(features, _pixels(b) * p.C, dt, "features")
    _need(w.w1, vlb_packed_bytes(p, 1) // 2 if p.packed else p.hidden * p.C * p.k * p.k, dt, "w1")
    _need(w.w2, vlb_packed_bytes(p, 2) // 2 if p.packed else p.out_dim * p.hidden, dt, "w2")
    _need(w.ln_gamma, p.C, dt, "ln_gamma")
    f32 = torch.float32
    _need(g.d_w1, p.hidden * p.C * p.k * p.k, f32, "d_w1")
    _need(g.d_b1, p.hidden, f32, "d_b1")
    _need(g.d_w2, p.out_dim * p.hidden, f32, "d_w2")
    _need(g.d_b2, p.out_dim, f32, "d_b2")
    _need(g.d_features, _pixels(b) * p.C, dt, "d_features")
    for t, n, what in ((g.d_ln_gamma, p.C, "d_ln_gamma"), (g.d_ln_beta, p.C, "d_ln_beta"),
                       (g.d_newline, p.out_dim, "d_newline"),
                       (g.d_separator, p.out_dim, "d_separator")):
        _need(t, n, f32, what)
    n_mid = _depth(p) - 2
    if len(g.d_w_mid) != n_mid or len(g.d_b_mid) != n_mid or len(w.w_mid) != n_mid:
        raise ValueError(f"depth {_depth(p)}: {n_mid} middle weights and gradients needed")
    for q in range(n_mid):
        _need(g.d_w_mid[q], p.hidden * p.hidden, f32, f"d_w_mid[{q}]")
        _need(g.d_b_mid[q], p.hidden, f32, f"d_b_mid[{q}]")
    wc = w.c()
    gc = g.c()
    _check(lib().vlb_bridge_backward(ct.byref(p), ct.byref(b.c), _ptr(features), ct.byref(wc),
                                     _ptr(mask), dseq.shape[0], _ptr(dseq), _ptr(saved),
                                     saved.numel(), ct.byref(gc), _ptr(ws), ws.numel(),
                                     _stream(stream)), "vlb_bridge_backward")


# ---- request planning (host) ---------------------------------------------------

class Processor:
    """Candidate resolutions [(W, H)], patch size and merge factor of a tiled
    (VL2-style) processor; keeps the C arrays alive."""

    def __init__(self, candidates: Sequence[tuple], patch_size: int, downsample: int):
        self.candidates = [tuple(c) for c in candidates]
        flat = [x for c in self.candidates for x in c]
        self._arr = (ct.c_int32 * max(len(flat), 1))(*flat)
        self.c = vlb_processor(self._arr, len(self.candidates), patch_size, downsample)
        self.image_size = self.candidates[0][0] if self.candidates else 0
        self.patch_size = patch_size

    @property
    def grid(self) -> int:
        """Patches per side of every view."""
        return self.image_size // self.patch_size


def vlb_select_resolution(pc: Processor, w0: int, h0: int) -> tuple:
    best = (ct.c_int32 * 2)()
    _check(lib().vlb_select_resolution(ct.byref(pc.c), w0, h0, best), "vlb_select_resolution")
    return int(best[0]), int(best[1])


def vlb_plan_request(pc: Processor, sizes: Sequence[tuple]):
    """[(tw, th)] and [slots] for the images (w0, h0) of one request."""
    n = len(sizes)
    flat = (ct.c_int32 * max(2 * n, 1))(*[x for s_ in sizes for x in s_])
    tiles = (ct.c_int32 * max(2 * n, 1))()
    slots = (ct.c_int64 * max(n, 1))()
    _check(lib().vlb_plan_request(ct.byref(pc.c), n, flat, tiles, slots), "vlb_plan_request")
    return [(int(tiles[2 * i]), int(tiles[2 * i + 1])) for i in range(n)], \
        [int(slots[i]) for i in range(n)]


def vlb_expand_prompt(ids: Sequence[int], image_token_id: int, bos_id: int,
                      slots: Sequence[int]) -> list:
    n = len(ids)
    a = (ct.c_int32 * max(n, 1))(*ids)
    sl = (ct.c_int64 * max(len(slots), 1))(*slots)
    m = int(lib().vlb_expand_prompt(a, n, image_token_id, bos_id, sl, len(slots), None, 0))
    if m < 0:
        raise VlbError(-m, "vlb_expand_prompt")
    out = (ct.c_int32 * m)()
    got = int(lib().vlb_expand_prompt(a, n, image_token_id, bos_id, sl, len(slots), out, m))
    if got != m:
        raise VlbError(-got if got < 0 else ERR_SHAPE, "vlb_expand_prompt")
    return list(out)


def batch_for_request(pc: Processor, tiles: Sequence[tuple], global_view_tail: bool = False) -> Batch:
    """The 2D-tiled batch of planned images: image i has 1 + tw*th views of
    grid x grid patches, the global view first."""
    g = pc.grid
    grids, vpi = [], []
    for tw, th in tiles:
        vpi.append(1 + tw * th)
        grids += [(g, g)] * (1 + tw * th)
    return Batch(grids, vpi, LAYOUT_TILED_2D, list(tiles), global_view_tail)


def vlb_check(ws, stream=None) -> int:
    """Device-recorded status of the last scatter / fused call on this workspace."""
    return int(lib().vlb_check(_ptr(ws), _stream(stream)))


def vlb_prof_enable(mask):
    """True / -1: time every kernel; an int: bit kid times kernel id kid (K_*);
    False / 0: stop recording."""
    if mask is True:
        mask = -1
    elif mask is False:
        mask = 0
    _check(lib().vlb_prof_enable(int(mask)), "vlb_prof_enable")


def vlb_prof_resume(mask: int):
    """Like vlb_prof_enable(mask) but keeps the records taken so far."""
    _check(lib().vlb_prof_resume(int(mask)), "vlb_prof_resume")


def vlb_prof_read(kid: int):
    n = ct.c_int64(0)
    ms = ct.c_double(0.0)
    _check(lib().vlb_prof_read(kid, ct.byref(n), ct.byref(ms)), "vlb_prof_read")
    return int(n.value), float(ms.value)


class Bridge:
    """A projector with its weights resident on the device (bf16: both weights packed
    once into the GEMMs' tile-blocked form), plus a cached workspace."""

    def __init__(self, p: vlb_projector, w: Weights, pack: bool = True):
        self.w = w
        if p.dtype == BF16 and pack and not p.packed:
            dev = w.w1.device
            w1p = torch.empty(vlb_packed_bytes(p, 1) // 2, dtype=w.w1.dtype, device=dev)
            w2p = torch.empty(vlb_packed_bytes(p, 2) // 2, dtype=w.w2.dtype, device=dev)
            vlb_pack_weights(p, w.w1, w.w2, w1p, w2p)
            mids = []
            for wm in w.w_mid:
                t = torch.empty(vlb_packed_bytes(p, 3) // 2, dtype=wm.dtype, device=dev)
                vlb_pack_mid(p, wm, t)
                mids.append(t)
            self.w = Weights(w1p, w.b1, w2p, w.b2, w.ln_gamma, w.ln_beta, mids, list(w.b_mid))
            p = vlb_projector.from_buffer_copy(p)
            p.packed = 1
        self.p = p
        self._ws = None

    def workspace(self, b: Batch, seq_len: int = 0) -> torch.Tensor:
        n = vlb_workspace_bytes(self.p, b, seq_len)
        if n == 0:
            raise VlbError(ERR_SHAPE, "vlb_workspace_bytes")
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.w.w2.device)
        return self._ws

    def project(self, b: Batch, features, rows=None):
        if rows is None:
            rows = torch.empty(vlb_num_tokens(self.p, b), self.p.out_dim, dtype=_tdtype(self.p),
                               device=features.device)
        vlb_merge_project(self.p, b, features, self.w, rows, self.workspace(b))
        return rows

    def fused(self, b: Batch, features, newline, separator, mask, seq):
        ws = self.workspace(b, seq.shape[0])
        vlb_bridge_fused(self.p, b, features, self.w, newline, separator, mask, seq, ws)
        return ws
