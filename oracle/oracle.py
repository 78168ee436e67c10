"""ctypes wrapper of the fp64 CPU oracle (vlb_oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only tests/, the smoke check in
__graft_entry__ and the CPU-baseline leg of bench.py import this module.  The
oracle shares no code with the HIP path; it reads the same seeded host inputs,
widened exactly to float64.

Page citations for each step live in vlb_oracle.c and vlb_oracle.h.
"""
from __future__ import annotations

import ctypes as ct
import os
import subprocess
from dataclasses import dataclass, field
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vlb_oracle.c")
_LIB = os.path.join(_HERE, "libvlb_oracle.so")

GELU_ERF, GELU_TANH, ACT_NONE = 0, 1, 2
SRC_NEWLINE, SRC_SEPARATOR = -1, -2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "vlb_oracle.h"))
    ):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-std=c11", "-D_GNU_SOURCE", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """The oracle library: the -O2 build, or the build that VLB_ORACLE_LIB names
    (the CPU tests' sanitizer build)."""
    global _lib
    if _lib is None:
        _lib = ct.CDLL(os.environ.get("VLB_ORACLE_LIB") or build())
        _declare(_lib)
    return _lib


def build_sanitized(out_dir: str) -> str:
    """The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
    (ROCm's clang, the sanitizer runtime shared, so that one runtime serves it and
    the library's sanitized host code in one process)."""
    so = os.path.join(out_dir, "libvlb_oracle_san.so")
    subprocess.check_call(
        ["/opt/rocm/lib/llvm/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared-libsan",
         "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", "-D_GNU_SOURCE", "-o", so, _SRC,
         "-lm", "-lpthread"])
    return so


class use_library:
    """Context manager: route every call of this module to another build of the
    oracle (the mutation tests load copies with a planted mistake)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = lib()
        L = ct.CDLL(self.path)
        _declare(L)
        _lib = L
        return L

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def build_variant(src_text: str, out_dir: str, name: str) -> str:
    """Compile a modified copy of the oracle source (used only by mutation tests)."""
    import shutil
    c = os.path.join(out_dir, name + ".c")
    with open(c, "w") as f:
        f.write(src_text)
    shutil.copy(os.path.join(_HERE, "vlb_oracle.h"), os.path.join(out_dir, "vlb_oracle.h"))
    so = os.path.join(out_dir, "lib" + name + ".so")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
                           "-D_GNU_SOURCE", "-o", so, c, "-lm", "-lpthread"])
    return so


class _Spec(ct.Structure):
    _fields_ = [
        ("n_views", ct.c_int32),
        ("grid_h", ct.POINTER(ct.c_int32)),
        ("grid_w", ct.POINTER(ct.c_int32)),
        ("C", ct.c_int32), ("k", ct.c_int32), ("hidden", ct.c_int32), ("out_dim", ct.c_int32),
        ("has_ln", ct.c_int32),
        ("ln_eps", ct.c_double),
        ("act", ct.c_int32),
        ("n_images", ct.c_int32),
        ("views_per_image", ct.POINTER(ct.c_int32)),
        ("tiled", ct.c_int32),
        ("tile_w", ct.POINTER(ct.c_int32)),
        ("tile_h", ct.POINTER(ct.c_int32)),
        ("global_tail", ct.c_int32),
        ("n_mid", ct.c_int32),
    ]


_D = ct.POINTER(ct.c_double)
_I64 = ct.POINTER(ct.c_int64)
_U8 = ct.POINTER(ct.c_uint8)


def _declare(L):
    i64 = ct.c_int64
    L.orc_merged_side.restype = i64
    L.orc_merged_side.argtypes = [i64, i64]
    L.orc_view_tokens.restype = i64
    L.orc_view_tokens.argtypes = [i64, i64, i64]
    L.orc_total_tokens.restype = i64
    L.orc_total_tokens.argtypes = [ct.POINTER(_Spec)]
    L.orc_tiled_placeholders.restype = i64
    L.orc_tiled_placeholders.argtypes = [i64, i64, i64, i64]
    L.orc_param_count.restype = i64
    L.orc_param_count.argtypes = [i64, i64, i64, i64, ct.c_int32]
    L.orc_layer_norm.restype = None
    L.orc_layer_norm.argtypes = [_D, i64, ct.c_int32, _D, _D, ct.c_double, _D]
    L.orc_merge_view.restype = None
    L.orc_merge_view.argtypes = [_D, ct.c_int32, ct.c_int32, ct.c_int32, ct.c_int32, _D]
    L.orc_unmerge_view.restype = None
    L.orc_unmerge_view.argtypes = [_D, ct.c_int32, ct.c_int32, ct.c_int32, ct.c_int32, _D]
    L.orc_linear.restype = None
    L.orc_linear.argtypes = [_D, i64, ct.c_int32, _D, _D, ct.c_int32, _D, ct.c_int32]
    L.orc_gelu_erf.restype = None
    L.orc_gelu_erf.argtypes = [_D, i64]
    L.orc_gelu_tanh.restype = None
    L.orc_gelu_tanh.argtypes = [_D, i64]
    L.orc_merged_row.restype = None
    L.orc_merged_row.argtypes = [ct.POINTER(_Spec), _D, _D, _D, i64, _D]
    L.orc_project_rows.restype = None
    L.orc_project_rows.argtypes = [ct.POINTER(_Spec), _D, _D, _D, _D, _D, _D, _D, _I64, i64, _D,
                                   ct.c_int32]
    L.orc_project_rows_deep.restype = None
    L.orc_project_rows_deep.argtypes = [ct.POINTER(_Spec), _D, _D, _D, _D, _D, _D, _D, _D, _D,
                                        _I64, i64, _D, ct.c_int32]
    L.orc_assemble.restype = i64
    L.orc_assemble.argtypes = [ct.POINTER(_Spec), _I64, i64]
    L.orc_scatter.restype = ct.c_int32
    L.orc_scatter.argtypes = [_I64, i64, _D, _D, _D, _U8, i64, ct.c_int32, _D]
    L.orc_embed_scatter.restype = ct.c_int32
    L.orc_embed_scatter.argtypes = [_I64, i64, _D, _D, _D, ct.POINTER(ct.c_int32), i64,
                                    ct.c_int32, ct.POINTER(ct.c_uint16), _D, i64, ct.c_int32, _D]
    L.orc_scatter_backward.restype = ct.c_int32
    L.orc_scatter_backward.argtypes = [_I64, i64, _U8, i64, ct.c_int32, _D, i64, _D, _D, _D]
    L.orc_project_backward.restype = None
    L.orc_project_backward.argtypes = [ct.POINTER(_Spec)] + [_D] * 14
    L.orc_project_backward_deep.restype = None
    L.orc_project_backward_deep.argtypes = [ct.POINTER(_Spec)] + [_D] * 18
    L.orc_hidden_unit_grads.restype = None
    L.orc_hidden_unit_grads.argtypes = [ct.POINTER(_Spec)] + [_D] * 7 + [ct.c_int32, _D, _D, _D]
    L.orc_pixel_grad.restype = None
    L.orc_pixel_grad.argtypes = [ct.POINTER(_Spec)] + [_D] * 7 + [ct.c_int32] * 3 + [_D]


def _f64(a) -> np.ndarray:
    """Exact widening of a host array (numpy or torch CPU, any float dtype) to float64."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen in torch (bf16 has no numpy dtype)
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _dp(a):
    return None if a is None else a.ctypes.data_as(_D)


@dataclass
class Spec:
    """A bridge problem as the oracle sees it (same meaning as orc_spec)."""

    grids: Sequence[tuple]          # (gh, gw) per view, in storage order
    C: int
    k: int
    hidden: int
    out_dim: int
    views_per_image: Sequence[int]
    has_ln: bool = False
    ln_eps: float = 1e-6
    act: int = GELU_ERF
    tiled: bool = False
    tiles: Sequence[tuple] = ()     # (tw, th) per image when tiled
    global_tail: bool = False
    depth: int = 2                  # Linears in the projector (>= 2)
    _keep: list = field(default_factory=list, repr=False)

    def c(self) -> _Spec:
        gh = np.ascontiguousarray([g[0] for g in self.grids], dtype=np.int32)
        gw = np.ascontiguousarray([g[1] for g in self.grids], dtype=np.int32)
        vpi = np.ascontiguousarray(self.views_per_image, dtype=np.int32)
        tw = np.ascontiguousarray([t[0] for t in self.tiles] or [0], dtype=np.int32)
        th = np.ascontiguousarray([t[1] for t in self.tiles] or [0], dtype=np.int32)
        self._keep = [gh, gw, vpi, tw, th]
        p32 = lambda a: a.ctypes.data_as(ct.POINTER(ct.c_int32))
        return _Spec(len(self.grids), p32(gh), p32(gw), self.C, self.k, self.hidden,
                     self.out_dim, int(self.has_ln), float(self.ln_eps), int(self.act),
                     len(self.views_per_image), p32(vpi), int(self.tiled), p32(tw), p32(th),
                     int(self.global_tail), int(self.depth) - 2)


def merged_side(g: int, k: int) -> int:
    return int(lib().orc_merged_side(g, k))


def view_tokens(gh: int, gw: int, k: int) -> int:
    return int(lib().orc_view_tokens(gh, gw, k))


def total_tokens(spec: Spec) -> int:
    s = spec.c()
    return int(lib().orc_total_tokens(ct.byref(s)))


def tiled_placeholders(hp: int, wp: int, tw: int, th: int) -> int:
    return int(lib().orc_tiled_placeholders(hp, wp, tw, th))


def param_count(C: int, k: int, hidden: int, out_dim: int, has_ln: bool) -> int:
    return int(lib().orc_param_count(C, k, hidden, out_dim, int(has_ln)))


def layer_norm(x, gamma, beta, eps: float) -> np.ndarray:
    x = _f64(x)
    C = x.shape[-1]
    out = np.empty_like(x)
    lib().orc_layer_norm(_dp(x), x.size // C, C, _dp(_f64(gamma)), _dp(_f64(beta)), eps, _dp(out))
    return out


def merge_view(x, k: int) -> np.ndarray:
    """x: (gh, gw, C) -> (tokens, C*k*k) in the pages' feature order."""
    x = _f64(x)
    gh, gw, C = x.shape
    out = np.empty((view_tokens(gh, gw, k), C * k * k), dtype=np.float64)
    lib().orc_merge_view(_dp(x), gh, gw, C, k, _dp(out))
    return out


def unmerge_view(m, gh: int, gw: int, C: int, k: int) -> np.ndarray:
    m = _f64(m)
    out = np.empty((gh, gw, C), dtype=np.float64)
    lib().orc_unmerge_view(_dp(m), gh, gw, C, k, _dp(out))
    return out


def linear(x, W, b, nthreads: int = 1) -> np.ndarray:
    x = _f64(x)
    W = _f64(W)
    rows, in_dim = x.shape
    out_dim = W.shape[0]
    out = np.empty((rows, out_dim), dtype=np.float64)
    lib().orc_linear(_dp(x), rows, in_dim, _dp(W), _dp(_f64(b)), out_dim, _dp(out), nthreads)
    return out


def gelu_erf(x) -> np.ndarray:
    x = _f64(x).copy()
    lib().orc_gelu_erf(_dp(x), x.size)
    return x


def gelu_tanh(x) -> np.ndarray:
    x = _f64(x).copy()
    lib().orc_gelu_tanh(_dp(x), x.size)
    return x


def merged_row(spec: Spec, x, gamma, beta, r: int) -> np.ndarray:
    s = spec.c()
    out = np.empty(spec.C * spec.k * spec.k, dtype=np.float64)
    lib().orc_merged_row(ct.byref(s), _dp(_f64(x)), _dp(_f64(gamma)), _dp(_f64(beta)), r, _dp(out))
    return out


def project_rows(spec: Spec, x, gamma, beta, W1, b1, W2, b2, row_ids=None,
                 nthreads: int = 0) -> np.ndarray:
    """fp64 projected rows for the listed token rows (all rows when None)."""
    s = spec.c()
    if row_ids is None:
        row_ids = np.arange(total_tokens(spec), dtype=np.int64)
    row_ids = np.ascontiguousarray(row_ids, dtype=np.int64)
    if nthreads <= 0:
        nthreads = min(os.cpu_count() or 1, 16)
    out = np.empty((len(row_ids), spec.out_dim), dtype=np.float64)
    xs = [_f64(a) for a in (x, gamma, beta, W1, b1, W2, b2)]
    lib().orc_project_rows(ct.byref(s), *[_dp(a) for a in xs], row_ids.ctypes.data_as(_I64),
                           len(row_ids), _dp(out), nthreads)
    return out


def project_rows_deep(spec: Spec, x, gamma, beta, W1, b1, W_mid, b_mid, W2, b2, row_ids=None,
                      nthreads: int = 0) -> np.ndarray:
    """project_rows for depth = spec.depth: W_mid [depth-2][hidden][hidden], b_mid
    [depth-2][hidden] (sequences of per-layer arrays are stacked)."""
    s = spec.c()
    n_mid = spec.depth - 2
    H = spec.hidden
    wm = np.ascontiguousarray(np.stack([_f64(a) for a in W_mid]) if n_mid else np.zeros((1, H, H)))
    bm = np.ascontiguousarray(np.stack([_f64(a) for a in b_mid]) if n_mid else np.zeros((1, H)))
    assert wm.shape[1:] == (H, H) and (n_mid == 0 or len(wm) == n_mid)
    if row_ids is None:
        row_ids = np.arange(total_tokens(spec), dtype=np.int64)
    row_ids = np.ascontiguousarray(row_ids, dtype=np.int64)
    if nthreads <= 0:
        nthreads = min(os.cpu_count() or 1, 16)
    out = np.empty((len(row_ids), spec.out_dim), dtype=np.float64)
    xs = [_f64(a) for a in (x, gamma, beta, W1, b1)]
    ys = [_f64(a) for a in (W2, b2)]
    lib().orc_project_rows_deep(ct.byref(s), *[_dp(a) for a in xs], _dp(wm), _dp(bm),
                                *[_dp(a) for a in ys], row_ids.ctypes.data_as(_I64), len(row_ids),
                                _dp(out), nthreads)
    return out


def assemble(spec: Spec) -> np.ndarray:
    s = spec.c()
    n = int(lib().orc_assemble(ct.byref(s), None, 0))
    src = np.empty(max(n, 1), dtype=np.int64)
    got = int(lib().orc_assemble(ct.byref(s), src.ctypes.data_as(_I64), n))
    assert got == n
    return src[:n]


def scatter(src, rows, newline, separator, mask, seq):
    """Returns (status, new_seq); status -1 = placeholder-count mismatch (seq untouched)."""
    src = np.ascontiguousarray(src, dtype=np.int64)
    rows = _f64(rows)
    seq = _f64(seq).copy()
    S, D = seq.shape
    mask = np.ascontiguousarray(np.asarray(mask), dtype=np.uint8)
    nl = _f64(newline) if newline is not None else np.zeros(D)
    sp = _f64(separator) if separator is not None else np.zeros(D)
    st = int(lib().orc_scatter(src.ctypes.data_as(_I64), len(src), _dp(rows), _dp(nl), _dp(sp),
                               mask.ctypes.data_as(_U8), S, D, _dp(seq)))
    return st, seq


def embed_scatter(src, rows, newline, separator, ids, image_id, embed, D):
    """Whole embedded sequence: text positions from the table, image_id positions
    from the assembled rows in order.  embed: torch bf16 / fp32 / fp64 or numpy
    [vocab][D] (bf16 is passed as its bit patterns and widened exactly in C).
    Returns (status, seq [S][D] fp64); status -1 = placeholder-count mismatch,
    -2 = text id out of range (seq is then all zero, i.e. untouched)."""
    src = np.ascontiguousarray(src, dtype=np.int64)
    rows = _f64(rows)
    ids = np.ascontiguousarray(np.asarray(ids), dtype=np.int32)
    S = len(ids)
    nl = _f64(newline) if newline is not None else np.zeros(D)
    sp = _f64(separator) if separator is not None else np.zeros(D)
    bits = None
    e64 = None
    if hasattr(embed, "detach") and str(embed.dtype) == "torch.bfloat16":
        import torch
        bits = np.ascontiguousarray(embed.detach().cpu().contiguous().view(torch.int16).numpy()).view(np.uint16)
        vocab = bits.shape[0]
    else:
        e64 = _f64(embed)
        vocab = e64.shape[0]
    seq = np.zeros((S, D), dtype=np.float64)
    st = int(lib().orc_embed_scatter(
        src.ctypes.data_as(_I64), len(src), _dp(rows), _dp(nl), _dp(sp),
        ids.ctypes.data_as(ct.POINTER(ct.c_int32)), S, int(image_id),
        bits.ctypes.data_as(ct.POINTER(ct.c_uint16)) if bits is not None else None,
        _dp(e64) if e64 is not None else None, vocab, D, _dp(seq)))
    return st, seq


# ---- backward --------------------------------------------------------------

def scatter_backward(src, mask, dseq, T):
    """Gradient of scatter: (status, drows [T][D], dnewline [D], dseparator [D]);
    status -1 = placeholder-count mismatch (outputs zero)."""
    src = np.ascontiguousarray(src, dtype=np.int64)
    dseq = _f64(dseq)
    S, D = dseq.shape
    mask = np.ascontiguousarray(np.asarray(mask), dtype=np.uint8)
    drows = np.zeros((T, D))
    dnl = np.zeros(D)
    dsp = np.zeros(D)
    st = int(lib().orc_scatter_backward(src.ctypes.data_as(_I64), len(src),
                                        mask.ctypes.data_as(_U8), S, D, _dp(dseq), T,
                                        _dp(drows), _dp(dnl), _dp(dsp)))
    return st, drows, dnl, dsp


def project_backward(spec: Spec, x, gamma, beta, W1, b1, W2, dY) -> dict:
    """All projector gradients for the output-row gradient dY [T][out_dim]:
    dict with dx [n_pixels][C], dw1, db1, dw2, db2 and (LayerNorm) dgamma, dbeta."""
    s = spec.c()
    x = _f64(x)
    K1 = spec.C * spec.k * spec.k
    out = {"dx": np.zeros_like(x), "dw1": np.zeros((spec.hidden, K1)),
           "db1": np.zeros(spec.hidden), "dw2": np.zeros((spec.out_dim, spec.hidden)),
           "db2": np.zeros(spec.out_dim), "dgamma": np.zeros(spec.C), "dbeta": np.zeros(spec.C)}
    ins = [x] + [_f64(a) for a in (gamma, beta, W1, b1, W2, dY)]
    lib().orc_project_backward(ct.byref(s), *[_dp(a) for a in ins],
                               *[_dp(out[n]) for n in ("dx", "dw1", "db1", "dw2", "db2",
                                                       "dgamma", "dbeta")])
    if not spec.has_ln:
        del out["dgamma"], out["dbeta"]
    return out


def project_backward_deep(spec: Spec, x, gamma, beta, W1, b1, W_mid, b_mid, W2, dY) -> dict:
    """project_backward for depth = spec.depth, with "dw_mid" [depth-2][H][H] and
    "db_mid" [depth-2][H] as well."""
    s = spec.c()
    x = _f64(x)
    n_mid, H = spec.depth - 2, spec.hidden
    K1 = spec.C * spec.k * spec.k
    wm = np.ascontiguousarray(np.stack([_f64(a) for a in W_mid]) if n_mid else np.zeros((1, H, H)))
    bm = np.ascontiguousarray(np.stack([_f64(a) for a in b_mid]) if n_mid else np.zeros((1, H)))
    out = {"dx": np.zeros_like(x), "dw1": np.zeros((H, K1)), "db1": np.zeros(H),
           "dw_mid": np.zeros((max(n_mid, 1), H, H)), "db_mid": np.zeros((max(n_mid, 1), H)),
           "dw2": np.zeros((spec.out_dim, H)), "db2": np.zeros(spec.out_dim),
           "dgamma": np.zeros(spec.C), "dbeta": np.zeros(spec.C)}
    ins = [x] + [_f64(a) for a in (gamma, beta, W1, b1)]
    lib().orc_project_backward_deep(ct.byref(s), *[_dp(a) for a in ins], _dp(wm), _dp(bm),
                                    _dp(_f64(W2)), _dp(_f64(dY)),
                                    *[_dp(out[n]) for n in ("dx", "dw1", "db1", "dw_mid", "db_mid",
                                                            "dw2", "db2", "dgamma", "dbeta")])
    out["dw_mid"], out["db_mid"] = out["dw_mid"][:n_mid], out["db_mid"][:n_mid]
    if not spec.has_ln:
        del out["dgamma"], out["dbeta"]
    return out


def hidden_unit_grads(spec: Spec, x, gamma, beta, W1, b1, W2, dY, h: int):
    """(row h of dW1, db1[h], column h of dW2)."""
    s = spec.c()
    K1 = spec.C * spec.k * spec.k
    dw1 = np.zeros(K1)
    db1 = np.zeros(1)
    dw2 = np.zeros(spec.out_dim)
    ins = [_f64(a) for a in (x, gamma, beta, W1, b1, W2, dY)]
    lib().orc_hidden_unit_grads(ct.byref(s), *[_dp(a) for a in ins], int(h), _dp(dw1), _dp(db1),
                                _dp(dw2))
    return dw1, float(db1[0]), dw2


def pixel_grad(spec: Spec, x, gamma, beta, W1, b1, W2, dY, view: int, y: int, xx: int):
    """Feature gradient [C] of pixel (y, xx) of view `view`."""
    s = spec.c()
    out = np.zeros(spec.C)
    ins = [_f64(a) for a in (x, gamma, beta, W1, b1, W2, dY)]
    lib().orc_pixel_grad(ct.byref(s), *[_dp(a) for a in ins], int(view), int(y), int(xx),
                         _dp(out))
    return out
