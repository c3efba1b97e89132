"""The matrix-core calibration launch behind the bench line's measured peak:
its flop count follows the instruction shapes, and every workgroup computes
the same sums (the launch does the products it counts, on every CU)."""
import pytest
import torch

import variable_length_packed_pack_amd as vlp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,k_dim", [(torch.bfloat16, 16), (torch.float16, 16), (torch.float32, 2)])
def test_mfma_rate_counts_and_sums(dtype, k_dim):
    dev = torch.device("cuda:0")
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 64
    print(f"[calibrate] {dtype} blocks={blocks} iters={iters}", flush=True)
    sink = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device=dev)
    flops = vlp.mfma_rate(dtype, blocks, iters, sink)
    torch.cuda.synchronize()
    assert flops == 2.0 * 32 * 32 * k_dim * 4 * 8 * blocks * iters
    got = sink.view(blocks, 512).cpu()
    assert torch.isfinite(got).all()
    assert (got[0] != 0).all()
    assert torch.equal(got, got[0].expand_as(got))


def test_mfma_rate_binding_checks_the_sink():
    dev = torch.device("cuda:0")
    with pytest.raises(ValueError):
        vlp.mfma_rate(torch.bfloat16, 4, 8, torch.empty(4 * 512 - 1, dtype=torch.float32, device=dev))
    with pytest.raises(TypeError):
        vlp.mfma_rate(torch.bfloat16, 4, 8, torch.empty(4 * 512, dtype=torch.float16, device=dev))
    with pytest.raises(TypeError):
        vlp.mfma_rate(torch.bfloat16, 4, 8, torch.empty(4 * 512, dtype=torch.float32))
