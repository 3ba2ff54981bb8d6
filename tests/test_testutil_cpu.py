"""CPU checks of the agreement helpers themselves."""
import numpy as np
import torch

from rs_testutil import bf16_half_ulp


def test_bf16_half_ulp_bounds_rounding():
    # every real value rounded to the nearest bf16 lies within half a bf16 ulp of the result
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 1.0, 7.9, 40.0)])
    r = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)
    err = np.abs(r - v.astype(np.float32).astype(np.float64))
    assert np.all(err <= bf16_half_ulp(r))


def test_bf16_half_ulp_values():
    assert bf16_half_ulp(np.array([1.0]))[0] == 2.0 ** -8
    assert bf16_half_ulp(np.array([-1.5]))[0] == 2.0 ** -8
    assert bf16_half_ulp(np.array([8.5]))[0] == 2.0 ** -5
    assert bf16_half_ulp(np.array([0.0]))[0] == 0.0
