"""The attainable-peak probes on the GPU: the copy moves every byte, and the
matrix-core loop runs and produces finite sums (its exact value has no
meaning beyond keeping the products alive)."""
import pytest
import torch

from block_sparse_token_amd import binding as Bd

pytestmark = pytest.mark.gpu


def test_gpu_peak_copy_moves_every_byte():
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    n = (1 << 22) + 16 * 37  # not a multiple of the launch's stride
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    Bd.up_peak_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_gpu_peak_mfma_loop_runs():
    sink = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    Bd.up_peak_mfma_bf16(8, 64, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    with pytest.raises(Bd.UniprefillError):
        Bd.up_peak_mfma_bf16(9, 64, sink)
