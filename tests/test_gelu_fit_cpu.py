"""Accuracy of the GELU the bf16 fc1 epilogue evaluates, on the CPU: the constants are
read from the HIP source and evaluated in float32 in the kernel's order, then compared
with the exact erf form.  (The fp32 path uses the device erf.)"""
import os
import re
import sys

import numpy as np
from scipy.special import ndtr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "vit_token_pruning_amd", "csrc"))
import gelu_fit  # noqa: E402


def _kernel_coefficients():
    src = open(os.path.join(ROOT, "vit_token_pruning_amd", "csrc", "rs_gemm.hip")).read()
    body = src[src.index("float gelu_fitted(float x)"):]
    body = body[:body.index("}")]
    vals = [float(v) for v in re.findall(r"([-+]?\d\.\d+e[-+]\d+|[-+]?\d+\.\d+)f", body)]
    # the clamp first, then the Horner constants c4, c3, c2, c1, c0
    assert vals[0] == gelu_fit.CLAMP, vals
    c4, c3, c2, c1, c0 = vals[1:6]
    return np.array([c0, c1, c2, c3, c4], np.float32)


def test_kernel_gelu_constants_are_the_fit():
    np.testing.assert_allclose(_kernel_coefficients(), gelu_fit.fit(), rtol=1e-5)


def test_kernel_gelu_error_bound():
    c = _kernel_coefficients()
    x = np.concatenate([np.linspace(-30, 30, 400001), np.linspace(-1e4, 1e4, 200001),
                        [0.0, -0.0, 1e-30, -1e-30]]).astype(np.float32).astype(np.float64)
    err = np.abs(gelu_fit.gelu_fitted_f32(x, c).astype(np.float64) - x * ndtr(x))
    assert err.max() <= 1.3e-5
    # far outside: relative error negligible, no overflow of the tail term
    big = np.array([1e6, -1e6, 1e30, -1e30, 3e38, -3e38], np.float32)
    gb = gelu_fit.gelu_fitted_f32(big, c).astype(np.float64)
    want = np.where(big > 0, big.astype(np.float64), 0.0)
    assert np.all(np.abs(gb - want) <= 1e-20 * np.abs(big))
    assert gelu_fit.gelu_fitted_f32(np.array([0.0]), c)[0] == 0.0
