"""Coefficients of the bf16-path GELU in rs_gemm.hip (run on a host with SciPy).

GELU(x) = x * Phi(x).  The kernel writes Phi(x) = logistic(t * P(t^2)) with
t = clamp(x, -6, 6), i.e. it approximates the logit of the standard normal CDF,
log(Phi / (1 - Phi)), by an odd polynomial.  The coefficients minimise the maximum
GELU error: a linear program (minimax) on the logit residual weighted by
d GELU / d logit = x * Phi * (1 - Phi), on a grid over [0, 6] (the logit is odd, so
negative x follow).  log2(e) is folded in so the kernel evaluates the logistic as
1 / (1 + 2^-(t * P)) with the hardware exp2.

    python gelu_fit.py          # prints the folded coefficients and the error
"""
import numpy as np
from scipy.optimize import linprog
from scipy.special import expit, ndtr

DEGREE = 4      # terms t, t^3, t^5, t^7
CLAMP = 6.0


def fit():
    z = np.linspace(1e-4, CLAMP, 12000)
    phi = ndtr(z)
    logit = np.log(phi) - np.log1p(-phi)
    w = z * phi * (1 - phi)
    A = np.stack([z ** (2 * j + 1) for j in range(DEGREE)], 1)
    n = DEGREE
    cost = np.zeros(n + 1)
    cost[-1] = 1.0
    a_ub = np.vstack([np.hstack([w[:, None] * A, -np.ones((len(z), 1))]),
                      np.hstack([-w[:, None] * A, -np.ones((len(z), 1))])])
    b_ub = np.concatenate([w * logit, -w * logit])
    res = linprog(cost, A_ub=a_ub, b_ub=b_ub, bounds=[(None, None)] * n + [(0, None)],
                  method="highs")
    return (res.x[:n] * np.log2(np.e)).astype(np.float32)


def gelu_fitted_f32(x, c):
    """The kernel's evaluation order in float32."""
    x = np.asarray(x, np.float32)
    t = np.clip(x, -CLAMP, CLAMP).astype(np.float32)
    u = (t * t).astype(np.float32)
    p = np.float32(0)
    for cj in c[::-1]:
        p = (p * u + cj).astype(np.float32)
    e = np.exp2(-(t * p).astype(np.float64)).astype(np.float32)
    return (x * (np.float32(1) / (np.float32(1) + e))).astype(np.float32)


if __name__ == "__main__":
    c = fit()
    xs = np.linspace(-30, 30, 600001)
    err = np.abs(gelu_fitted_f32(xs, c).astype(np.float64) - xs * ndtr(xs))
    print("coefficients (t, t^3, t^5, t^7), log2(e) folded:", [float(v) for v in c])
    print("max |GELU error| over [-30, 30]:", err.max())
