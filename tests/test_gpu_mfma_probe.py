"""GPU: the matrix-core rate probe (pkv_debug_mfma_rate) issues every product
it claims. With every operand 1.0, each 32x32x16 product adds 16 to each of
the 16 values a lane holds of its accumulator; per iteration the four PV
accumulators take 4 products each and the QK^T one 8, so a lane's sum over
its 80 values grows by 16 x 16 x (4 x 4 + 8) = 6144 per iteration, exactly,
in every lane of every wave. With every operand 0.5, a quarter of that."""

import pytest
import torch

import paged_kv_cache_430_amd as pkv

from gpu_helpers import device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("value,iterations,nwg", [(1.0, 1, 1), (1.0, 37, 3), (0.5, 100, 256), (1.0, 0, 2)])
def test_mfma_probe_issues_every_product(value, iterations, nwg):
    dev = device()
    ops = torch.full((1024,), value, dtype=torch.bfloat16, device=dev)
    sink = pkv.pkv_debug_mfma_rate(ops, iterations, nwg)
    torch.cuda.synchronize()
    expected = 6144.0 * iterations * value * value
    got = sink.cpu()
    assert got.numel() == nwg * 512
    assert torch.all(got == expected), (got.min().item(), got.max().item(), expected)


@pytest.mark.parametrize("iterations,nwg", [(1, 1), (9, 5), (64, 256)])
def test_prefill_mix_modes_agree(iterations, nwg):
    """pkv_debug_prefill_mix: the tile loads of mode 2 land in an LDS region
    the products never read, so modes 1 and 2 give the same bits for any
    data; with zero operands and tiles every product is zero whatever its
    source, so all three modes agree and the sums are finite."""
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(4308)
    ops = torch.randn(1024, generator=gen, device=dev).to(torch.bfloat16)
    tiles = torch.randn((1 << 20) // 2, generator=gen, device=dev).to(torch.bfloat16)
    s1 = pkv.pkv_debug_prefill_mix(ops, tiles, 1, iterations, nwg).cpu()
    s2 = pkv.pkv_debug_prefill_mix(ops, tiles, 2, iterations, nwg).cpu()
    assert torch.equal(s1, s2)
    zo, zt = torch.zeros_like(ops), torch.zeros_like(tiles)
    z = [pkv.pkv_debug_prefill_mix(zo, zt, m, iterations, nwg).cpu() for m in (0, 1, 2)]
    assert torch.isfinite(z[0]).all()
    assert torch.equal(z[0], z[1]) and torch.equal(z[0], z[2])
