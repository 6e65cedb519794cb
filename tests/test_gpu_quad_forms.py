"""GPU parity of the four-wave kernel's K-tail form (gemm_quad.h, kQuadTail)
and of its eight-stage ring on 128x128 tiles (kQuadDeep) against the
oracle.  K-tail form: K not a multiple of 64, its last K mod 64 elements
(one or two 32-element steps) loaded and multiplied before the main loop,
and NN B rows that end inside a 16-byte chunk (the last 64 k-rows taken that
way when 64 divides K).  Each case runs on the 128x128 tiles with four and
with eight ring stages, on the 256x128 and 256x256 tiles and through the
automatic choice; rows at
2-byte alignment (odd K or N, odd padding), ragged M and N, every output
type, bias, the plain, ReLU and beta forms, batches, and small integers held
bit for bit.  Shapes just outside a form (K - (K mod 64) < 128, fewer than 8
ring steps for eight stages, a cut NN row shorter than 8 elements) take the
next kernel down and are checked the same way."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, TORCH_DT, gemm_case, on_gpu
from parity import check
from test_gpu_gemm_ex import run_case

pytestmark = pytest.mark.gpu

# (tile, ring stages): None = the automatic choice
TILES = [("128x128q", 4), ("128x128q", 8), ("256x128q", None), ("256x256q", None), (None, None)]

# (M, N, K, in, out, trans_b, dist, bias, pad)
CASES = [
    (300, 264, 200, "bf16", "f32", False, "normal", False, 0),   # one tail step (8), whole chunks
    (300, 260, 191, "bf16", "bf16", False, "normal", True, 0),   # two tail steps (63), cut rows
    (257, 511, 1023, "f16", "f16", False, "normal", True, 0),    # the ragged shape's pattern
    (129, 300, 192, "bf16", "bf16", False, "int", True, 0),      # 64 | K, cut rows: tail of 64
    (200, 136, 129, "f16", "f32", True, "normal", True, 0),      # NT, tail of 1
    (520, 300, 777, "bf16", "bf16", True, "normal", True, 3),    # NT, odd padding
    (64, 9, 300, "bf16", "f32", False, "normal", False, 0),      # N = 9: one cut chunk per row
    (70, 8, 160, "bf16", "bf16", False, "int", False, 0),        # N = 8, tail of exactly one step
    (100, 520, 1000, "bf16", "f32", False, "int", True, 0),      # tail of 40, integers
    (40, 100, 150, "f16", "f16", False, "normal", True, 5),      # K - KT = 128 exactly
    (33, 7, 256, "bf16", "bf16", False, "normal", True, 0),      # cut row of 7: two-stage kernel
    (50, 100, 127, "bf16", "f32", True, "normal", False, 0),     # K - KT = 64: two-stage kernel
    (300, 384, 256, "bf16", "f32", False, "normal", True, 0),    # 64 | K: 8 ring steps exactly
    (260, 200, 261, "f16", "f16", True, "int", True, 0),         # tail of 5 after 8 ring steps
    (130, 264, 2048, "bf16", "bf16", False, "normal", True, 0),  # 64 ring steps
    (129, 136, 230, "bf16", "f32", False, "normal", False, 0),   # 6 ring steps: four stages only
]


def _id(c):
    M, N, K, f, o, tb, d, b, pad = c
    return f"{f}-{o}-{'NT' if tb else 'NN'}-{M}x{N}x{K}-{d}{'-bias' if b else ''}{f'-pad{pad}' if pad else ''}"


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_tail_and_ring_forms(tmm, case, force):
    M, N, K, fmt, out, tb, dist, bias, pad = case
    for tile, ring in TILES:
        force(tile, ring=ring)
        dC, o, T = gemm_case(tmm, M, N, K, fmt, out, tb, dist, bias, seed=7000 + 10 * CASES.index(case),
                             pad=pad)
        check(dC, o, T, K, exact=(dist == "int"), what=f"{_id(case)} tile {tile or 'auto'} ring {ring}")


@pytest.mark.parametrize("tile", ["128x128q", "256x128q"])
@pytest.mark.parametrize("tb", [False, True], ids=["NN", "NT"])
def test_tail_form_relu_and_beta(tmm, tile, tb, force):
    """The ReLU and beta epilogues on the K-tail form (cut NN rows, K = 333)."""
    force(tile)
    run_case(tmm, 260, 262, 333, "bf16", "bf16", False, tb, 0.75, 0.0, True, True, seed=7300,
             what=f"tail relu {tile}")
    run_case(tmm, 260, 262, 333, "f16", "f32", False, tb, 1.5, -0.5, True, True, seed=7310,
             what=f"tail beta relu {tile}")


@pytest.mark.parametrize("ring", [4, 8])
def test_tail_form_batched(tmm, force, ring):
    """Three batch entries with cut NN rows and a K tail: each entry's last
    k-rows are read by words, the rows before them reach into the next k-row
    of the same entry only."""
    force("128x128q", ring=ring)
    Z, M, N, K = 3, 200, 250, 421
    A = syn.to_bits(syn.normal((Z, M, K), 7401), "bf16")
    B = syn.to_bits(syn.normal((Z, K, N), 7402), "bf16")
    bvec = syn.normal((N,), 7403, 0.02).astype(np.float32)
    dC = torch.full((Z, M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    tmm.tmm_gemm_strided_batched(on_gpu(A, "bf16"), on_gpu(B, "bf16"), dC,
                                 bias=torch.from_numpy(bvec).to(DEV))
    torch.cuda.synchronize()
    for z in range(Z):
        o, T = oracle.gemm("bf16", A[z], B[z], bias=bvec, want_abs=True)
        check(dC[z], o, T, K, what=f"batched tail z {z} ring {ring}")


def test_ragged_shape_takes_the_tail_form(tmm, force):
    """4097 x 511 x 1023 NN bf16 (cut rows, K tail of 63) on the automatic
    choice, every output against the oracle; and the same bits when the
    128x128 four-wave tile with eight stages is pinned (the automatic choice
    for its one round of 132 tiles)."""
    force()
    M, N, K = 4097, 511, 1023
    dC, o, T = gemm_case(tmm, M, N, K, "bf16", "bf16", False, "normal", False, seed=7500)
    check(dC, o, T, K, what="ragged 4097x511x1023 tail form")
    force("128x128q", ring=8)
    dC2, _, _ = gemm_case(tmm, M, N, K, "bf16", "bf16", False, "normal", False, seed=7500)
    assert torch.equal(dC.view(torch.int16), dC2.view(torch.int16))


def _draw(i):
    g = np.random.default_rng([20261203, i])
    fmt = ["bf16", "f16"][g.integers(0, 2)]
    out = [fmt, "f32"][g.integers(0, 2)]
    tb = bool(g.integers(0, 2))
    M, N, K = int(g.integers(1, 600)), int(g.integers(8, 600)), int(g.integers(129, 1400))
    pad = int(g.choice([0, 0, 1, 3, 8]))
    dist = ["normal", "int"][g.integers(0, 2)]
    bias = bool(g.integers(0, 2))
    tile, ring = TILES[g.integers(0, len(TILES))]
    return M, N, K, fmt, out, tb, dist, bias, pad, tile, ring


@pytest.mark.parametrize("i", range(48))
def test_random_shapes_on_the_four_wave_forms(tmm, force, i):
    """Seeded random shapes (any K from 129, rows at any alignment, ragged M
    and N) on the four- and eight-stage 128x128 tiles, the 256x128 tiles and
    the automatic choice."""
    M, N, K, fmt, out, tb, dist, bias, pad, tile, ring = _draw(i)
    force(tile, ring=ring)
    dC, o, T = gemm_case(tmm, M, N, K, fmt, out, tb, dist, bias, seed=90000 + 10 * i, pad=pad)
    check(dC, o, T, K, exact=(dist == "int"),
          what=f"{M}x{N}x{K} {fmt}->{out} {'NT' if tb else 'NN'} pad {pad} {dist} tile {tile} ring {ring}")
