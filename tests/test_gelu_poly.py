"""The bf16 epilogue's GELU (act_fn<0> in vlb_common.h) against x * Phi(x).

The coefficients are read from the kernel header and the epilogue's float32
arithmetic is replayed in numpy; scipy's normal CDF is the exact reference.
Bounds (the output is rounded to bf16, a relative step of 2^-8): relative
error <= 3e-4 wherever |GELU(x)| > 1e-3, absolute error <= 5e-5 on [-12, 12],
and the two asymptotes (x for large x, 0 for very negative x).
"""
import os
import re

import numpy as np
from scipy.special import ndtr

HDR = os.path.join(os.path.dirname(__file__), "..", "patch_merge_mlp_amd", "csrc", "vlb_common.h")


def _coeffs():
    src = open(HDR).read()
    body = src[src.index("float gauss_tail(float x)"):src.index("template <int ACT>")]
    clamp = float(re.search(r"fminf\(fabsf\(x\), ([0-9.e+-]+)f\)", body).group(1))
    top = float(re.search(r"float h = ([0-9.e+-]+)f;", body).group(1))
    rest = [float(v) for v in re.findall(r"h = fmaf\(h, a, ([0-9.e+-]+)f\);", body)]
    return clamp, [top] + rest  # highest degree first


def _gelu32(x):
    clamp, c = _coeffs()
    x = x.astype(np.float32)
    a = np.minimum(np.abs(x), np.float32(clamp))
    h = np.full_like(a, np.float32(c[0]))
    for ck in c[1:]:
        h = (h * a + np.float32(ck)).astype(np.float32)
    tail = np.exp2(-h).astype(np.float32)
    return (np.maximum(x, np.float32(0)) - np.abs(x) * tail).astype(np.float32)


def test_gelu_poly_accuracy():
    clamp, c = _coeffs()
    assert clamp == 5.5 and len(c) == 5
    x = np.linspace(-12.0, 12.0, 2400001)
    y = _gelu32(x).astype(np.float64)
    ref = x * ndtr(x)
    err = np.abs(y - ref)
    assert err.max() <= 5e-5, err.max()
    big = np.abs(ref) > 1e-3
    assert (err[big] / np.abs(ref[big])).max() <= 3e-4
    # asymptotes and the origin
    assert _gelu32(np.array([0.0]))[0] == 0.0
    assert np.allclose(_gelu32(np.array([8.0, 30.0, 1e4])), [8.0, 30.0, 1e4], rtol=1e-7)
    assert np.all(np.abs(_gelu32(np.array([-8.0, -30.0, -1e4]))) <= 1e-7 * np.array([8, 30, 1e4]))
    # the error is not one-signed: it changes sign across the fit interval
    d = (y - ref)[(x > -3.4) & (x < 0)]
    assert (d > 0).any() and (d < 0).any()
