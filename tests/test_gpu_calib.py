"""The matrix-core calibration (a measurement aid) runs through the C ABI and
leaves finite sums; its FLOP count follows the documented launch shape."""
import pytest
import torch

import ulysses_sequence_attention_rank_amd as uly

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5])
def test_calibrate_mfma_runs(mode):
    say(f"calibrate_mfma mode={mode}")
    out = torch.full((512 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = uly.calibrate_mfma(64, mode, out)
    torch.cuda.synchronize()
    assert flops == 512 * 4 * 64 * 8 * 2 * 32 * 32 * 16
    assert torch.isfinite(out).all()
