"""The throughput probe behind the attention ceiling (rs_probe_throughput) runs every mode to
completion through the C ABI and leaves finite values in its sink (its timing is measured by
bench.py --probe, not tested)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5, 6])
def test_probe_modes_complete(mode):
    import torch
    from vit_token_pruning_amd import _native as N
    wg = 8
    sink = torch.full((wg * 256,), float("nan"), device="cuda", dtype=torch.float32)
    st = N.lib().rs_probe_throughput(mode, wg, 16, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == N.RS_OK, N.lib().rs_last_error()
    torch.cuda.synchronize()
    v = sink.cpu().numpy()
    assert np.isfinite(v).all()
