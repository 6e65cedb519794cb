"""The measurement kernels (libtmm_probes.so) run and return: a small read
stream, and a few rounds of each matrix-instruction shape on all-ones
operands, whose accumulator sums are known exactly."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_stream_read_runs():
    import tiled_matrix_multiplication_amd.probes as probes
    src = torch.randn(64 * 4096, device="cuda:0").to(torch.bfloat16)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for w in (4, 8, 16):
        probes.stream_read(src, 64, 8192, w, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


@pytest.mark.parametrize("shape", [0, 1])
def test_mfma_loop_runs(shape):
    import tiled_matrix_multiplication_amd.probes as probes
    ops = torch.ones(1 << 23, device="cuda:0", dtype=torch.bfloat16)   # 16 MiB
    sink = torch.full((4 * 512,), float("nan"), device="cuda:0")
    probes.mfma_loop(ops, shape, 4, 3, sink)
    torch.cuda.synchronize()
    # all-ones operands: each accumulator element gets 64 per round (shape 0:
    # four 32x32x16 instructions per block; shape 1: two 16x16x32), so after
    # 3 rounds every one of a lane's 128 accumulator values is 192
    s = sink.cpu()
    assert torch.all(s == 128 * 192)
