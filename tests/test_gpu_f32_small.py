"""GPU parity of the small fp32 kernel (gemm_f32_small.hip: 32x32 tiles, K
split over a workgroup's four waves), which the automatic choice takes for
fp32 products of at most one 128x128 tile per two CUs, against the oracle
and beside the two-stage kernel pinned on the same problem: the fp32 256^3
configuration in both layouts, K of 1 and of odd lengths (a quarter that is
cut short or empty), M and N ending mid-tile, batches, bias, the full form
(beta and ReLU), small integers held bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, gemm_case, on_gpu
from parity import check
from test_gpu_gemm_ex import run_case

pytestmark = pytest.mark.gpu

# (M, N, K, trans_b, dist, bias)
CASES = [
    (256, 256, 256, False, "normal", False),
    (256, 256, 256, True, "normal", True),
    (256, 256, 256, False, "int", True),
    (8, 8, 8, False, "int", False),
    (1, 1, 1, False, "normal", True),
    (33, 70, 5, True, "normal", False),
    (100, 300, 1001, True, "normal", True),
    (64, 40, 130, False, "int", False),
]


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


def _id(c):
    M, N, K, tb, d, b = c
    return f"{M}x{N}x{K}-{'NT' if tb else 'NN'}-{d}{'-bias' if b else ''}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_small_fp32_kernel(tmm, force, case):
    M, N, K, tb, dist, bias = case
    for tile in (None, "128x128"):
        force(tile)
        dC, o, T = gemm_case(tmm, M, N, K, "f32", "f32", tb, dist, bias, seed=9500 + 10 * CASES.index(case))
        check(dC, o, T, K, exact=(dist == "int"), what=f"{_id(case)} tile {tile or 'auto'}")


def test_small_fp32_batched(tmm, force):
    force()
    Z, M, N, K = 3, 70, 90, 77
    A = syn.to_bits(syn.normal((Z, M, K), 9601), "f32")
    B = syn.to_bits(syn.normal((Z, N, K), 9602), "f32")
    bvec = syn.normal((N,), 9603, 0.02).astype(np.float32)
    dC = torch.full((Z, M, N), float("nan"), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm_strided_batched(on_gpu(A, "f32"), on_gpu(B, "f32"), dC, bias=torch.from_numpy(bvec).to(DEV),
                                 trans_b=True)
    torch.cuda.synchronize()
    for z in range(Z):
        o, T = oracle.gemm("f32", A[z], B[z], trans_b=True, bias=bvec, want_abs=True)
        check(dC[z], o, T, K, what=f"small fp32 batched z {z}")


@pytest.mark.parametrize("tb", [False, True], ids=["NN", "NT"])
def test_small_fp32_full_form(tmm, force, tb):
    force()
    run_case(tmm, 96, 80, 150, "f32", "f32", False, tb, 0.5, -1.5, True, True, seed=9700, what="small fp32 full")
    run_case(tmm, 40, 50, 64, "f32", "f32", False, tb, 2.0, 1.0, False, False, seed=9710, dist="int",
             what="small fp32 full int")
