"""The measurement aids run on the GPU: the streaming read and the MFMA loop
launch cleanly, report the documented byte and flop counts, and leave the
sink untouched (it is written only on a 32-bit hash collision)."""

import pytest
import torch

from tests.gpu_util import say

import head_latent_attention_rmsnorm_amd as M  # noqa: E402

pytestmark = pytest.mark.gpu
api = M.api


def test_hbm_read_runs():
    say("[ceiling] hbm read 1 MiB + 48 B")
    buf = torch.zeros((1 << 20) + 48, dtype=torch.uint8, device="cuda")  # XOR 0: never the sink value
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert api.mla_ceiling_hbm_read(buf, sink) == (1 << 20) + 48
    torch.cuda.synchronize()
    assert sink.item() == 0


@pytest.mark.parametrize("lds", [False, True])
def test_mfma_loop_runs(lds):
    say(f"[ceiling] mfma loop lds={lds}")
    g = torch.Generator(device="cuda").manual_seed(3)
    ops = torch.randn(24576, generator=g, device="cuda").to(torch.float16)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    flops = api.mla_ceiling_mfma(ops, 3, lds, sink)
    torch.cuda.synchronize()
    assert flops == 12 * (2 if lds else 4) * 32768 * 3 * 8 * 512
    assert sink.item() == 0.0


def test_device_info():
    info = api.mla_device_info(0)
    say(f"[ceiling] device info {info}")
    assert info["compute_units"] == torch.cuda.get_device_properties(0).multi_processor_count
    assert info["peak_sclk_mhz"] > 0 and info["peak_mclk_mhz"] > 0
