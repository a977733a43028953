"""Fit of the upper normal tail used by the GEMM epilogue's GELU.

GELU(x) = x * Phi(x).  The kernel evaluates the tail Q(x) = Phi(-|x|) =
erfc(z) / 2, z = |x| / sqrt 2, in the form

    Q = t * 2^(P(t) - z^2 log2 e),   t = 1 / (1 + 0.4 z),

and Phi(x) = 1 - Q for x >= 0, Q otherwise.  erfc(z) e^(z^2) is smooth and
slowly varying, so after taking out the Gaussian factor and the 1/z decay
(through t) what is left, P, is well fitted by a low-degree polynomial in t.
P is fitted in log2 (so an error in P is a relative error of Q) over
0 <= z <= 9.5 (t in [1/4.8, 1]); past that Q < 2^-128 and P stays near its
value at the end of the range.

The fit is a weighted least-squares polynomial, re-weighted towards its largest
residuals until it is close to equi-oscillating (a poor man's minimax).
Running this file prints the coefficients, rounded to binary32, and the
largest error of the whole GELU when evaluated step by step in binary32; they
are pasted into gemm_kernels.h.  This is a development script: nothing imports
it.
"""
import numpy as np
from scipy.special import log_ndtr, ndtr

LOG2E = 1.4426950408889634
K_T = 0.4
Z_MAX = 9.5
DEGREE = 8


def target(t):
    z = (1.0 / t - 1.0) / K_T
    return (log_ndtr(-z * np.sqrt(2.0)) - np.log(t)) * LOG2E + z * z * LOG2E


def fit():
    tmin = 1.0 / (1.0 + K_T * Z_MAX)
    n = 4000
    u = np.cos(np.pi * (np.arange(n) + 0.5) / n)
    t = tmin + (1 - tmin) * (u + 1) / 2
    f = target(t)
    V = np.vander(t, DEGREE + 1, increasing=True)
    w = np.ones(n)
    for _ in range(60):
        c, *_ = np.linalg.lstsq(V * w[:, None], f * w, rcond=None)
        e = V @ c - f
        w = w * (np.abs(e) / np.abs(e).max()) ** 0.5 + 1e-15
        w /= w.max()
    return c.astype(np.float32)


def gelu_binary32(x, c):
    """The kernel's steps, each rounded to binary32 (fma rounded once)."""
    f32 = np.float32

    def fma(a, b, d):
        return f32(np.float64(a) * np.float64(b) + np.float64(d))

    x = f32(x)
    zl = f32(np.abs(x) * f32(np.sqrt(LOG2E / 2)))        # z sqrt(log2 e)
    t = f32(1.0 / np.float64(fma(zl, f32(K_T / np.sqrt(LOG2E)), f32(1))))
    p = c[DEGREE]
    for k in range(DEGREE - 1, -1, -1):
        p = fma(p, t, c[k])
    q = f32(t * f32(2.0 ** np.float64(fma(-zl, zl, p))))
    phi = f32(1 - q) if x >= 0 else q
    return f32(x * phi)


def main():
    c = fit()
    print("P coefficients, c0 .. c%d:" % DEGREE)
    print(", ".join("%.9gf" % v for v in c))
    print("constants: sqrt(log2(e) / 2) = %.9gf, 0.4 / sqrt(log2(e)) = %.9gf"
          % (np.float32(np.sqrt(LOG2E / 2)), np.float32(K_T / np.sqrt(LOG2E))))
    xs = np.concatenate([np.linspace(-14, 14, 100001), -np.logspace(-8, 1.2, 1000),
                         np.logspace(-8, 1.2, 1000)]).astype(np.float32)
    g = np.array([gelu_binary32(x, c) for x in xs], dtype=np.float64)
    ref = xs.astype(np.float64) * ndtr(xs.astype(np.float64))
    err = np.abs(g - ref)
    print("max |GELU error| / |x| = 2^%.2f" % np.log2((err / np.maximum(np.abs(xs), 1e-30)).max()))


if __name__ == "__main__":
    main()
