"""GPU parity on seeded random problems: element type, output type, layout,
shape (ragged, sometimes tiny), row padding, bias, batch count and tile shape
are all drawn from a fixed seed, and every output is compared with the
oracle.  Complements the hand-picked cases with combinations nobody listed."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, TORCH_DT, on_gpu
from parity import check, f8_operands

pytestmark = pytest.mark.gpu

OUTS = {"f32": ["f32"], "bf16": ["f32", "bf16"], "f16": ["f32", "f16"], "e4m3": ["f32", "bf16"]}
TILES = ["256x256", "256x256r", "256x256s2", "256x256w4", "256x128", "128x128", None]
NCASE = 40


def draw(i):
    g = np.random.default_rng([20261202, i])
    fmt = ["bf16", "f16", "e4m3", "f32"][g.integers(0, 4)]
    out = OUTS[fmt][g.integers(0, len(OUTS[fmt]))]
    tb = bool(g.integers(0, 2))
    small = g.random() < 0.25
    M = int(g.integers(1, 40 if small else 700))
    N = int(g.integers(1, 40 if small else 700))
    K = int(g.integers(1, 40 if small else 600))
    if g.random() < 0.5:            # whole 64-element K-steps: ring-kernel eligible
        K = max(64, (K // 64) * 64)
    if g.random() < 0.5:            # multiples of 8: 16-byte-aligned rows for 16-bit types
        M, N = max(8, M // 8 * 8), max(8, N // 8 * 8)
    pad = int(g.choice([0, 0, 8, 16, 3]))
    Z = int(g.choice([1, 1, 2, 3]))
    bias = bool(g.integers(0, 2))
    tile = TILES[g.integers(0, len(TILES))]
    if fmt == "f32":    # fp32 always runs 128x128 tiles
        tile = None
    return fmt, out, tb, M, N, K, pad, Z, bias, tile


def operand(rows, cols, fmt, seed, pad, Z):
    """Z stacked (rows, cols) operands with `pad` extra elements per row."""
    x = syn.normal((Z * rows, cols + pad), seed)
    if fmt == "e4m3":
        s = syn.e4m3_scale(x)
        bits = syn.quantize_e4m3(x, s)
    else:
        s = np.float32(1.0)
        bits = syn.to_bits(x, fmt)
    return bits.reshape(Z, rows, cols + pad), s


@pytest.mark.parametrize("i", range(NCASE))
def test_random_problem(tmm, i, force):
    fmt, out, tb, M, N, K, pad, Z, bias, tile = draw(i)
    if tile is None:
        force()
    else:
        force(tile)
    seed = 9000 + 10 * i
    Ab, sa = operand(M, K, fmt, seed + 1, pad, Z)
    Bb, sb = operand(N, K, fmt, seed + 2, pad, Z) if tb else operand(K, N, fmt, seed + 2, pad, Z)
    bvec = syn.normal((N,), seed + 3, 0.02).astype(np.float32) if bias else None
    dA = on_gpu(np.ascontiguousarray(Ab), fmt)[:, :, :K]
    dB = on_gpu(np.ascontiguousarray(Bb), fmt)[:, :, :(K if tb else N)]
    C = torch.full((Z, M, N), float("nan"), dtype=TORCH_DT[out], device=DEV)
    dbias = torch.from_numpy(bvec).to(DEV) if bias else None
    tmm.tmm_gemm_strided_batched(dA, dB, C, bias=dbias, trans_b=tb, scale_a=float(sa),
                                 scale_b=float(sb))
    torch.cuda.synchronize()
    what = f"case {i}: {fmt}->{out} {'NT' if tb else 'NN'} {Z}x{M}x{N}x{K} pad {pad} tile {tile}"
    for z in range(Z):
        A = np.ascontiguousarray(Ab[z][:, :K])
        B = np.ascontiguousarray(Bb[z][:, :(K if tb else N)])
        o, T = oracle.gemm(fmt, A, B, trans_b=tb, bias=bvec, scale_a=sa, scale_b=sb, want_abs=True)
        ops = f8_operands(A, B, tb, float(sa) * float(sb)) if fmt == "e4m3" else None
        check(C[z], o, T, K, what=f"{what} z {z}", f8=(fmt == "e4m3"), f8_ops=ops)


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t
