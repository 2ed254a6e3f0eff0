"""GPU check of the MFMA-loop probe (a measurement aid): its outputs have a
closed form, 256 * iters per thread, independent of timing."""
import pytest
import torch

import x3_conv2d_epilogue_amd as x3

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_out,iters", [(256, 1), (256 * 3, 37), (256 * 8, 4096)])
def test_probe_mfma_closed_form(n_out, iters):
    out = torch.full((n_out,), -1.0, device="cuda:0")
    x3.probe_mfma(out, iters)
    torch.cuda.synchronize()
    assert bool((out == 256.0 * iters).all())


def test_probe_mfma_rejects_bad_sizes():
    out = torch.empty(300, device="cuda:0")
    with pytest.raises(x3.X3Error):
        x3.probe_mfma(out, 10)
    with pytest.raises(x3.X3Error):
        x3.probe_mfma(torch.empty(256, device="cuda:0"), 0)
