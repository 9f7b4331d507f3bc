"""The measurement helpers of sgl_probe.h on the GPU: the copy probe copies
exactly, and the MFMA probe's output equals its closed form (so the rate the
benchmark derives from it counts work that was done)."""
import pytest
import torch

import prefix_shared_paged_amd as sp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * 12345, 64 << 20])
def test_copy_probe_is_exact(nbytes):
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    assert sp.probe_copy(src, dst) == 2 * nbytes
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("n_wg,iters,x", [(1, 1, 1.0), (300, 64, 1.5), (2048, 16, -0.75)])
def test_mfma_probe_closed_form(n_wg, iters, x):
    out = torch.full((n_wg * sp.PROBE_THREADS,), -1.0, dtype=torch.float32, device="cuda")
    flop = sp.probe_mfma_bf16(out, iters, x)
    assert flop == n_wg * 4 * iters * 8 * 32768
    torch.cuda.synchronize()
    # 8 accumulators, each iters MFMAs adding 16 products x*x (x exact in bf16)
    assert torch.all(out == 8 * 16 * iters * x * x)
