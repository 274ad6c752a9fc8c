"""The MFMA-rate diagnostic runs every MFMA it counts: each sink element equals
its closed form 2048 * value^2 * iters (exact in float32 at these sizes)."""
import pytest
import torch

import bitwise_deterministic_moe_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("blocks,iters,value", [(1, 1, 1.0), (3, 7, 0.5), (512, 1000, 0.125)])
def test_mfma_rate_sink_closed_form(blocks, iters, value):
    print(f"moe_mfma_rate blocks={blocks} iters={iters} value={value}", flush=True)
    sink = moe.moe_mfma_rate(blocks, iters, value)
    torch.cuda.synchronize()
    assert sink.shape == (256 * blocks,)
    assert torch.all(sink == 2048.0 * value * value * iters)
