"""Fits the polynomial behind the bf16 GEMM epilogue's GELU (act_fn<0> in vlb_common.h).

For a >= 0 the Gaussian tail Phi(-a) = erfc(a / sqrt 2) / 2 is written as
2^(-h(a)); GELU(x) = x Phi(x) = max(x, 0) - |x| Phi(-|x|).  A relative error
dh in h is a relative error ln2 * dh in the tail, which is the relative error
of GELU(-a) and bounds that of GELU(a) (Phi(-a) <= Phi(a)).  The output is
rounded to bf16 (a relative step of 2^-8), so h only needs to be accurate
where |GELU(-a)| > 1e-3 (a < ~3.4); past that only the absolute error
|x| Phi(-|x|) ln2 dh matters.  The fit weights the error that way and is
iteratively reweighted to near-minimax; a degree-4 h then holds GELU to
2.8e-4 relative wherever |GELU| > 1e-3 and to 4.1e-5 absolute on [-12, 12].
The argument is clamped at 5.5 (Phi(-5.5) ~ 2e-8), which keeps the tail
decreasing where the quartic would turn.

Run: python fit_gelu_poly.py  -> prints the float32 coefficients c0..c4 and the
fp32-evaluated GELU error.
"""
import numpy as np
from scipy.special import log_ndtr, ndtr

CLAMP = 5.5
DEG = 4


def h_exact(a):
    return -log_ndtr(-a) / np.log(2.0)


def fit():
    n = 8000
    a = (np.cos(np.pi * (np.arange(n) + 0.5) / n)[::-1] + 1.0) * CLAMP / 2.0
    gneg = a * ndtr(-a)
    # per point: relative GELU error where |GELU(-a)| > 1e-3, else the absolute
    # error, scaled so that 1e-5 absolute weighs like 1e-4 relative
    scale = np.where(gneg > 1e-3, 1.0, gneg * np.log(2.0) / 1e-1)
    w = np.ones_like(a)
    for _ in range(200):
        c = np.polynomial.polynomial.polyfit(a, h_exact(a), DEG, w=np.sqrt(w) * scale)
        err = np.abs(np.polynomial.polynomial.polyval(a, c) - h_exact(a)) * scale
        w = w * (err / err.max() + 1e-4)
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
    x = np.linspace(-12, 12, 2400001)
    y = gelu_fp32(x, c).astype(np.float64)
    ref = x * ndtr(x)
    big = np.abs(ref) > 1e-3
    print("coefficients c0..c4:", ", ".join(f"{v:.9g}f" for v in c))
    print("max abs err", np.abs(y - ref).max(), "max rel err (|y| > 1e-3)",
          (np.abs(y - ref)[big] / np.abs(ref[big])).max())
