"""The allocation-free split-K entry point (tmm_gemm_splitk_noalloc, partials in
the library's per-GPU scratch) against tmm_gemm_splitk with a caller
workspace: the same kernels and order of sums, so the same bits, checked on
two calls in a row, the second smaller (the scratch keeps the first call's
partials), and each against the oracle's product."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, on_gpu
from parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


def _case(M, N, K, fmt, trans_b, seed):
    A = syn.to_bits(syn.normal((M, K), seed + 1), fmt)
    B = syn.to_bits(syn.normal((N, K) if trans_b else (K, N), seed + 2, 0.5), fmt)
    bias = syn.normal((N,), seed + 3, 0.02).astype(np.float32)
    o, T = oracle.gemm(fmt, A, B, trans_b=trans_b, bias=bias, want_abs=True)
    return on_gpu(A, fmt), on_gpu(B, fmt), torch.from_numpy(bias).to(DEV), o, T


def test_noalloc_matches_the_workspace_entry_point(tmm):
    cases = [(256, 1024, 2048, "f16", True, 4, torch.float16, 6000),
             (72, 300, 768, "bf16", False, 3, torch.bfloat16, 6100)]
    for M, N, K, fmt, tb, S, odt, seed in cases:
        dA, dB, dbias, o, T = _case(M, N, K, fmt, tb, seed)
        ws = torch.full((tmm.splitk_workspace_bytes(M, N, S) // 4,), float("nan"), dtype=torch.float32,
                        device=DEV)
        ref = torch.full((M, N), float("nan"), dtype=odt, device=DEV)
        tmm.tmm_gemm_splitk(dA, dB, ref, bias=dbias, trans_b=tb, splits=S, workspace=ws)
        got = torch.full((M, N), float("nan"), dtype=odt, device=DEV)
        # through the C ABI directly
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = tmm.lib.tmm_gemm_splitk_noalloc(
            M, N, K, tmm._dtype(dA), tmm._dtype(got), int(tb), ctypes.c_void_p(dA.data_ptr()), dA.stride(0),
            ctypes.c_void_p(dB.data_ptr()), dB.stride(0), ctypes.c_void_p(got.data_ptr()), got.stride(0),
            ctypes.c_void_p(dbias.data_ptr()), 1.0, 1.0, S, stream)
        assert rc == 0, tmm.tmm_status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), f"{M}x{N}x{K} S{S}"
        check(got, o, T, K, what=f"noalloc {M}x{N}x{K} S{S}")
