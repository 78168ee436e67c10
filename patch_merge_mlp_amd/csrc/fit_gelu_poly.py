"""Fits the polynomial behind the bf16 GEMM epilogue's GELU (act_fn<0> in vlb_common.h).

For a >= 0 the Gaussian tail Phi(-a) = erfc(a / sqrt 2) / 2 is written as
2^(-h(a)); h is smooth on [0, 6] (it grows like a^2 / (2 ln 2)), so a degree-7
polynomial fitted by iteratively reweighted least squares on Chebyshev nodes
(a minimax approximation in practice) holds h to ~5e-6, i.e. Phi(-a) to a
relative ~3e-6, tails included.  GELU(x) = x Phi(x) = max(x, 0) - |x| Phi(-|x|).
Past |x| = 6 the argument is clamped (Phi(-6) ~ 1e-9).

Run: python fit_gelu_poly.py  -> prints the float32 coefficients c0..c7 and the
fp32-evaluated GELU error over [-10, 10].
"""
import numpy as np
from scipy.special import erfc, ndtr

CLAMP = 6.0
DEG = 7


def h_exact(a):
    return -np.log2(0.5 * erfc(a / np.sqrt(2.0)))


def fit():
    n = 4000
    a = (np.cos(np.pi * (np.arange(n) + 0.5) / n)[::-1] + 1.0) * CLAMP / 2.0
    w = np.ones_like(a)
    for _ in range(60):
        c = np.polynomial.polynomial.polyfit(a, h_exact(a), DEG, w=np.sqrt(w))
        err = np.abs(np.polynomial.polynomial.polyval(a, c) - h_exact(a))
        w = w * (err / err.max() + 1e-3)
        w /= w.mean()
    return c.astype(np.float32)


def gelu_fp32(x, c):
    """The epilogue's arithmetic, step for step, in float32."""
    x = x.astype(np.float32)
    a = np.minimum(np.abs(x), np.float32(CLAMP))
    h = np.full_like(a, c[-1])
    for k in range(len(c) - 2, -1, -1):
        h = (h * a + c[k]).astype(np.float32)
    e = np.exp2(-h).astype(np.float32)
    return (np.maximum(x, np.float32(0)) - np.abs(x) * e).astype(np.float32)


if __name__ == "__main__":
    c = fit()
    x = np.linspace(-10, 10, 2000001)
    y = gelu_fp32(x, c).astype(np.float64)
    ref = x * ndtr(x)
    big = np.abs(ref) > 1e-3
    print("coefficients c0..c7:", ", ".join(f"{v:.9g}f" for v in c))
    print("max abs err", np.abs(y - ref).max(), "max rel err (|y| > 1e-3)",
          (np.abs(y - ref)[big] / np.abs(ref[big])).max())
