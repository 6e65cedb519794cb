"""GPU parity of the skinny-M GEMM (16-bit inputs, B stored N x K as a
linear layer's weight, few rows): the batch sizes of the GEMM page's
batch-size table for a 4096 x 4096 weight, plus ragged M, N and K (K tails
that are not a multiple of the 32-element step, or of 8), padded rows, bias,
both output widths, unaligned outputs and a batched case, all against the
oracle.  The kernel is reached both by the automatic choice (M <= 256) and by
the override tile=skinny (tmm_set_override)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, TORCH_DT, gemm_case, on_gpu
from parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


# (M, N, K, in, out, dist, bias, pad, forced); pad keeps rows 16-byte aligned
CASES = [
    (1, 4096, 4096, "bf16", "bf16", "normal", True, 0, True),
    (4, 4096, 4096, "bf16", "bf16", "normal", True, 0, False),
    (16, 4096, 4096, "f16", "f16", "normal", False, 0, False),
    (64, 4096, 4096, "f16", "f32", "normal", True, 0, False),
    (256, 4096, 4096, "bf16", "bf16", "normal", True, 0, False),
    (2, 300, 100, "bf16", "f32", "normal", False, 4, False),
    (7, 24, 9, "f16", "f16", "normal", True, 7, False),
    (33, 1030, 777, "bf16", "bf16", "normal", True, 7, False),
    (100, 520, 1000, "f16", "f16", "int", True, 0, False),
    (250, 777, 64, "bf16", "f32", "int", False, 0, False),
    (300, 200, 160, "bf16", "bf16", "normal", True, 0, True),
]


def _id(c):
    M, N, K, f, o, d, b, pad, forced = c
    return f"{f}-{o}-{M}x{N}x{K}-{d}{'-bias' if b else ''}{f'-pad{pad}' if pad else ''}" \
           f"{'-forced' if forced else ''}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_skinny_parity(tmm, case, force):
    M, N, K, fmt, out, dist, bias, pad, forced = case
    if forced:
        force("skinny")
    else:
        force()
    dC, o, T = gemm_case(tmm, M, N, K, fmt, out, True, dist, bias, seed=700 + 10 * CASES.index(case),
                         pad=pad)
    check(dC, o, T, K, exact=(dist == "int"), what=_id(case))


def test_skinny_batched_and_unaligned_output(tmm, force):
    """Three problems through the strided-batched entry point, written into
    an output with a row pitch that is not a multiple of 4 elements (element
    stores) and a gap between the matrices."""
    force()
    Z, M, N, K = 3, 12, 200, 96
    A = syn.to_bits(syn.normal((Z, M, K), 811), "bf16")
    B = syn.to_bits(syn.normal((Z, N, K), 812, 0.02), "bf16")
    bvec = syn.normal((N,), 813, 0.02).astype(np.float32)
    ldc, strideC = N + 3, M * (N + 3) + 5
    Cfull = torch.full((Z * strideC,), float("nan"), dtype=torch.bfloat16, device=DEV)
    C = Cfull.as_strided((Z, M, N), (strideC, ldc, 1))
    tmm.tmm_gemm_strided_batched(on_gpu(A, "bf16"), on_gpu(B, "bf16"), C,
                                 bias=torch.from_numpy(bvec).to(DEV), trans_b=True)
    torch.cuda.synchronize()
    for z in range(Z):
        o, T = oracle.gemm("bf16", A[z], B[z], trans_b=True, bias=bvec, want_abs=True)
        check(C[z], o, T, K, what=f"batched z {z}")
    keep = torch.zeros(Z, strideC, dtype=torch.bool, device=DEV)
    for z in range(Z):
        for m in range(M):
            keep[z, m * ldc:m * ldc + N] = True
    assert torch.isnan(Cfull.view(Z, strideC)[~keep].float()).all(), "a store landed outside C"


def test_skinny_matches_gemv_entry(tmm, force):
    """M = 1 through the skinny kernel (forced) and through the GEMV kernel
    agree with the oracle on the decode shape."""
    N, K = 4096, 4096
    W = syn.to_bits(syn.normal((N, K), 821, 0.02), "bf16")
    x = syn.to_bits(syn.normal((1, K), 822), "bf16")
    bvec = syn.normal((N,), 823, 0.02).astype(np.float32)
    o, T = oracle.gemm("bf16", x, W, trans_b=True, bias=bvec, want_abs=True)
    dW, dx, db = on_gpu(W, "bf16"), on_gpu(x, "bf16"), torch.from_numpy(bvec).to(DEV)
    for forced in (True, False):
        if forced:
            force("skinny")
        else:
            force()
        y = torch.full((1, N), float("nan"), dtype=TORCH_DT["bf16"], device=DEV)
        tmm.tmm_gemm(dx, dW, y, bias=db, trans_b=True)
        torch.cuda.synchronize()
        check(y, o, T, K, what=f"M=1 {'skinny' if forced else 'gemv'}")


@pytest.mark.parametrize("tile", [f"{m}x{n}" for m in (16, 32, 64) for n in (16, 32, 64)])
def test_every_skinny_tile(tmm, tile, force):
    """Each of the nine workgroup tiles on one ragged problem (M, N not
    multiples of any tile, a K tail) with bias, through the override skinny=<bm>x<bn>."""
    force("skinny", skinny=tile)
    dC, o, T = gemm_case(tmm, 70, 300, 200, "bf16", "bf16", True, "normal", True, seed=900, pad=0)
    check(dC, o, T, 200, what=f"skinny tile {tile}")


# (M, N, K, in, out, bias, pad): the several-row GEMV (2 <= M <= 8, K*E a
# multiple of 16): whole 4096-element passes, a partial pass, several passes
# with a partial one, ragged N, padded rows of X and W
GEMVM = [
    (2, 1000, 4096, "bf16", "bf16", True, 0),
    (3, 4100, 1000, "f16", "f16", False, 8),
    (4, 4096, 4096, "bf16", "f32", True, 0),
    (5, 777, 8256, "f16", "f32", True, 0),
    (8, 2048, 4104, "bf16", "bf16", True, 16),
]


@pytest.mark.parametrize("case", GEMVM, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-{c[3]}-{c[4]}" for c in GEMVM])
@pytest.mark.parametrize("forced", [False, True], ids=["auto", "forced"])
def test_gemv_multi(tmm, case, forced, force):
    """A few rows through one weight (Y = X . W^T): the several-row GEMV,
    reached automatically and through the override tile=gemvm, against the
    oracle."""
    M, N, K, fmt, out, bias, pad = case
    if forced:
        force("gemvm")
    else:
        force()
    dC, o, T = gemm_case(tmm, M, N, K, fmt, out, True, "normal", bias, seed=950 + 10 * GEMVM.index(case),
                         pad=pad)
    check(dC, o, T, K, what=f"gemv-multi M={M} N={N} K={K}")


def test_gemv_multi_keeps_fp16_subnormals(tmm, force):
    """fp16 subnormal activations (2^-20) against unit weights: every output
    is K * 2^-20 exactly, which a flush to zero would lose."""
    force("gemvm")
    M, N, K = 4, 256, 4096
    X = torch.full((M, K), 2.0 ** -20, dtype=torch.float16, device=DEV)
    W = torch.ones((N, K), dtype=torch.float16, device=DEV)
    Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm(X, W, Y, trans_b=True)
    torch.cuda.synchronize()
    assert torch.all(Y == K * 2.0 ** -20)
