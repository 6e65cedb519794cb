"""GPU parity of every tile kernel: the tile shape is pinned through
the override tile=... (tmm_set_override, read by every call), so the 256x256 kernels,
which the automatic choice only takes at large sizes, are checked against the
oracle on small ragged problems too.  "256x256r" runs the four-stage ring
kernel whenever K is a multiple of its 32-element step ("256x256" only for an
N-contiguous B), "256x256s2" the two-stage kernel on the same tiles.

Every tile accumulates each output over the same sequence of 16-wide (fp8:
64-wide) matrix instructions in ascending K, so all tiles must also agree bit
for bit."""
import pytest
import torch

from gpu_cases import gemm_case
from parity import check

pytestmark = pytest.mark.gpu

TILES = ["256x256", "256x256r", "256x256s2", "256x256w4", "256x128", "128x128"]

# (M, N, K, in, out, trans_b, dist, bias, pad); pads keep rows 16-byte aligned
CASES = [
    (520, 776, 320, "bf16", "f32", False, "normal", False, 0),
    (520, 776, 320, "bf16", "bf16", True, "normal", True, 0),
    (300, 520, 352, "bf16", "bf16", True, "int", True, 8),
    (264, 512, 96, "f16", "f16", False, "normal", True, 8),
    (700, 300, 64, "f16", "f32", True, "normal", False, 0),
    # one, two, three and four K-steps of the ring (its prologue and tail)
    (257, 264, 32, "bf16", "f32", False, "int", False, 0),
    (300, 280, 64, "bf16", "f32", True, "normal", False, 0),
    (300, 280, 96, "bf16", "f32", False, "normal", False, 0),
    (513, 520, 128, "f16", "f16", False, "normal", False, 0),
    # K not a multiple of the ring step: two-stage kernel with a K tail
    (520, 776, 200, "bf16", "f32", False, "normal", False, 0),
    # fp8 (two-stage kernel on every 256-wide tile)
    (512, 512, 512, "e4m3", "bf16", False, "normal", False, 0),
    (384, 640, 384, "e4m3", "bf16", True, "normal", True, 0),
]


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


def _id(c):
    M, N, K, f, o, tb, d, b, pad = c
    return f"{f}-{o}-{'NT' if tb else 'NN'}-{M}x{N}x{K}-{d}{'-bias' if b else ''}{f'-pad{pad}' if pad else ''}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_every_tile(tmm, case, force):
    M, N, K, fmt, out, tb, dist, bias, pad = case
    first = None
    for tile in TILES:
        force(tile)
        dC, o, T, ops = gemm_case(tmm, M, N, K, fmt, out, tb, dist, bias,
                                  seed=100 + 10 * CASES.index(case), pad=pad, want_ops=True)
        check(dC, o, T, K, exact=(dist == "int"), what=f"{_id(case)} tile {tile}", f8=(fmt == "e4m3"),
              f8_ops=ops)
        bits = dC.view(torch.int32 if dC.element_size() == 4 else torch.int16)
        if first is None:
            first = bits
        else:
            assert torch.equal(bits, first), f"tile {tile} differs from {TILES[0]} in some bits"
