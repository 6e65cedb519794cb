"""GPU parity of every tile kernel: the tile shape is pinned through
the override tile=... (tmm_set_override, read by every call), so the 256x256 kernels,
which the automatic choice only takes at large sizes, are checked against the
oracle on small ragged problems too.  "256x256r" runs the four-stage ring
kernel whenever K is a multiple of its 32-element step, "256x256s2" the
two-stage kernel on the same tiles, "256x256" (the automatic choice) the
four-wave kernel where it applies (16-bit inputs, K a multiple of 64 and at
least 128) and the ring or two-stage kernel elsewhere.

The 32x32x16 kernels accumulate each output over the same sequence of
16-wide (fp8: 64-wide) matrix instructions in ascending K, so they must also
agree bit for bit; the four-wave kernel's 16x16x32 instructions sum 32 at a
time and are held to the oracle (bit for bit on integer inputs)."""
import pytest
import torch

from gpu_cases import gemm_case
from parity import check

pytestmark = pytest.mark.gpu

# kernels on 32x32x16 instructions (one summation order: bit-identical results)
TILES = ["256x256r", "256x256s2", "256x256w4", "256x128", "128x128"]
# the automatic 256x256 choice, which takes the four-wave 16x16x32 kernel
# wherever it applies: held to the oracle only (bit for bit on integers)
OTHER_TILES = ["256x256"]

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
    for tile in OTHER_TILES:
        force(tile)
        dC, o, T, ops = gemm_case(tmm, M, N, K, fmt, out, tb, dist, bias,
                                  seed=100 + 10 * CASES.index(case), pad=pad, want_ops=True)
        check(dC, o, T, K, exact=(dist == "int"), what=f"{_id(case)} tile {tile}", f8=(fmt == "e4m3"),
              f8_ops=ops)


# The four-wave 128x128-per-wave kernel: 16x16x32 matrix instructions sum the
# products in another order than the 32x32x16 kernels, so it is held to the
# oracle (and bit for bit on integer inputs), not to the other tiles' bits.
# K must be a multiple of 64 and at least 128 (4 steps: the loop runs zero
# times and only the written-out tail does, 6 steps: one loop pass).
QUAD_CASES = [
    (520, 776, 320, "bf16", "f32", False, "normal", False, 0),
    (520, 776, 320, "bf16", "bf16", True, "normal", True, 0),
    (300, 520, 384, "bf16", "bf16", True, "int", True, 8),
    (264, 512, 128, "f16", "f16", False, "normal", True, 8),
    (700, 300, 256, "f16", "f32", True, "normal", False, 0),
    (257, 264, 128, "bf16", "f32", False, "int", False, 0),
    (513, 520, 192, "f16", "f16", False, "normal", False, 0),
    (256, 256, 1024, "bf16", "f32", False, "normal", True, 0),
]


QUAD_TILES = ["256x256q", "256x128q", "128x128q"]


@pytest.mark.parametrize("tile", QUAD_TILES)
@pytest.mark.parametrize("case", QUAD_CASES, ids=[_id(c) for c in QUAD_CASES])
def test_quad_kernel(tmm, case, tile, force):
    M, N, K, fmt, out, tb, dist, bias, pad = case
    force(tile)
    dC, o, T = gemm_case(tmm, M, N, K, fmt, out, tb, dist, bias, seed=300 + 10 * QUAD_CASES.index(case),
                         pad=pad)
    check(dC, o, T, K, exact=(dist == "int"), what=f"{_id(case)} four-wave {tile}")


@pytest.mark.parametrize("tile", QUAD_TILES)
@pytest.mark.parametrize("tb", [False, True], ids=["NN", "NT"])
def test_quad_kernel_batched(tmm, tb, tile, force):
    """Batch of 3 with padded rows: every slice against the oracle."""
    import numpy as np
    import oracle
    import synthetic as syn
    from gpu_cases import DEV, on_gpu
    force(tile)
    Z, M, N, K, pad = 3, 300, 264, 192, 8
    a = syn.to_bits(syn.normal((Z * M, K + pad), 401), "bf16").reshape(Z, M, K + pad)
    bshape = (N, K) if tb else (K, N)
    b = syn.to_bits(syn.normal((Z * bshape[0], bshape[1] + pad), 402), "bf16").reshape(Z, bshape[0], bshape[1] + pad)
    bvec = syn.normal((N,), 403, 0.02).astype(np.float32)
    dA = on_gpu(np.ascontiguousarray(a), "bf16")[:, :, :K]
    dB = on_gpu(np.ascontiguousarray(b), "bf16")[:, :, :bshape[1]]
    C = torch.full((Z, M, N), float("nan"), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm_strided_batched(dA, dB, C, bias=torch.from_numpy(bvec).to(DEV), trans_b=tb)
    torch.cuda.synchronize()
    for z in range(Z):
        o, T = oracle.gemm("bf16", np.ascontiguousarray(a[z][:, :K]), np.ascontiguousarray(b[z][:, :bshape[1]]),
                           trans_b=tb, bias=bvec, want_abs=True)
        check(C[z], o, T, K, what=f"four-wave batch {z}")


# The fp8 four-wave kernel (gemm_quad8.h): K a multiple of 128 and at least
# 256; chunks of 16 fp8 whole (N % 16 == 0 for an N-contiguous B).
QUAD8_CASES = [
    (512, 512, 512, "e4m3", "bf16", False, "normal", False, 0),
    (384, 640, 512, "e4m3", "f32", True, "normal", True, 0),
    (300, 528, 256, "e4m3", "bf16", False, "int", True, 16),
    (256, 256, 1024, "e4m3", "f32", False, "normal", False, 0),
    (520, 272, 384, "e4m3", "bf16", True, "int", False, 0),
]


@pytest.mark.parametrize("case", QUAD8_CASES, ids=[_id(c) for c in QUAD8_CASES])
def test_quad8_kernel(tmm, case, force):
    M, N, K, fmt, out, tb, dist, bias, pad = case
    force("256x256q")
    dC, o, T, ops = gemm_case(tmm, M, N, K, fmt, out, tb, dist, bias, seed=500 + 10 * QUAD8_CASES.index(case),
                              pad=pad, want_ops=True)
    check(dC, o, T, K, exact=(dist == "int"), what=f"{_id(case)} fp8 four-wave", f8=True, f8_ops=ops)
