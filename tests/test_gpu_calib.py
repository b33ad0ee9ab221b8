"""The calibration kernels (include/moe_calib.h) the benchmark measures its
ceilings with: the streaming copy must copy every byte (also with a size
that is not a multiple of the grid stride), and the matrix-core loop must
run and report its flop count."""

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_calib_copy_copies_every_byte():
    import grouped_gemm_shard_amd as g
    for n in (16, 4096 * 16 + 48, 3 << 20):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(n)
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
        dst = torch.zeros_like(src)
        g.calib_copy(src, dst, blocks=64)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), n


def test_calib_mfma_runs_and_counts():
    import grouped_gemm_shard_amd as g
    sink = torch.full((512,), float("nan"), dtype=torch.float32, device="cuda")
    flops = g.calib_mfma(8, 10, sink)
    torch.cuda.synchronize()
    assert flops == 8 * 8 * 10 * 8 * 2 * 16 * 16 * 32
    assert torch.isfinite(sink).all()
