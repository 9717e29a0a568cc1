"""Coefficients of the Gaussian-tail polynomial in tp_device.hpp.

The bf16 GELU kernels evaluate the upper tail Q(x) = Phi(-x) = erfc(x/sqrt 2)/2
(x >= 0) as

    Q(x) = 2^( -x^2 log2(e)/2 + g(min(x, 5)) ),   g(x) ~ (ln Q(x) + x^2/2) log2(e),

g a degree-6 polynomial in x: ln Q(x) + x^2/2 is smooth and slowly varying
(ln 1/2 at 0, about -ln(x sqrt(2 pi)) for large x), so a low-degree fit gives
a relative error of Q near 1.5e-5 over [0, 5] in fp32 evaluation; past x = 5
(Q < 3e-7, GELU(-x) > -1.5e-6) the fit is held at 5.  The fit is least
squares in the power basis on 4000 Chebyshev nodes of [0, 5].

Run: python gelu_tail_fit.py   (prints the constants and the fp32 errors)
"""
import numpy as np
from scipy.special import erfc

X, DEG, NODES = 5.0, 6, 4000


def fit():
    xs = np.cos(np.pi * (np.arange(NODES) + 0.5) / NODES) * X / 2 + X / 2
    g = (np.log(0.5 * erfc(xs / np.sqrt(2))) + xs ** 2 / 2) / np.log(2.0)
    c, *_ = np.linalg.lstsq(np.vander(xs, DEG + 1, increasing=True), g, rcond=None)
    return c


def tail_fp32(c, x):
    c32 = c.astype(np.float32)
    x = np.asarray(x, dtype=np.float32)
    xc = np.minimum(x, np.float32(X))
    p = np.float32(c32[DEG])
    for k in range(DEG - 1, -1, -1):
        p = (p * xc + c32[k]).astype(np.float32)
    e = (x * np.float32(-0.5 / np.log(2.0)) * x + p).astype(np.float32)
    return np.exp2(e.astype(np.float64))


if __name__ == "__main__":
    c = fit()
    for k, v in enumerate(c):
        print(f"constexpr float kQc{k} = {float(np.float32(v))!r}f;")
    x = np.linspace(0, X, 200001)
    rel = np.abs(tail_fp32(c, x) / (0.5 * erfc(x / np.sqrt(2))) - 1)
    print(f"max relative error of Q on [0, {X}]: {rel.max():.3e}")
    z = np.linspace(-8, 8, 400001)
    gelu = np.maximum(z, 0) - np.abs(z) * tail_fp32(c, np.abs(z))
    print(f"max absolute GELU error on [-8, 8]: {np.abs(gelu - z * 0.5 * erfc(-z / np.sqrt(2))).max():.3e}")
