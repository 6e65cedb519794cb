"""GPU parity of the split-K product (tmm_gemm_splitk) against the oracle's
one-pass product: K cut into S slices whose fp32 partials are summed in a
fixed order and rounded once, so the same tolerance as tmm_gemm applies (the
fp32 summation bound over K).  Shapes: the decode-size layer it is meant for
(M = 256 rows through a 4096-wide weight, the bench configuration), rows and
columns that end mid-tile, both layouts, every output type, S from 1 to 8,
fp8 inputs with their scales, small integers held bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, TORCH_DT, make_operand, on_gpu
from parity import check, f8_operands

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


def splitk_case(tmm, M, N, K, fmt, out, trans_b, dist, bias, splits, seed, pad=0):
    A_full, A, sa = make_operand((M, K), fmt, dist, seed + 1, pad)
    bshape = (N, K) if trans_b else (K, N)
    B_full, B, sb = make_operand(bshape, fmt, dist, seed + 2, pad)
    bvec = None
    if bias:
        bvec = (syn.small_ints((N,), seed + 3) if dist == "int" else syn.normal((N,), seed + 3, 0.02))
        bvec = bvec.astype(np.float32)
    o, T = oracle.gemm(fmt, A, B, trans_b=trans_b, bias=bvec, scale_a=sa, scale_b=sb, want_abs=True)
    dA = on_gpu(A_full, fmt)[:, :K]
    dB = on_gpu(B_full, fmt)[:, :bshape[1]]
    dC = torch.full((M, N), float("nan"), dtype=TORCH_DT[out], device=DEV)
    dbias = torch.from_numpy(bvec).to(DEV) if bvec is not None else None
    ws = torch.full((tmm.splitk_workspace_bytes(M, N, splits) // 4,), float("nan"), dtype=torch.float32,
                    device=DEV)
    tmm.tmm_gemm_splitk(dA, dB, dC, bias=dbias, trans_b=trans_b, splits=splits, workspace=ws,
                        scale_a=float(sa), scale_b=float(sb))
    torch.cuda.synchronize()
    ops = f8_operands(A, B, trans_b, float(sa) * float(sb)) if fmt == "e4m3" else None
    return dC, o, T, ops, (dA, dB, dbias, ws, sa, sb)


# (M, N, K, in, out, trans_b, dist, bias, splits, pad)
CASES = [
    (256, 1024, 2048, "bf16", "bf16", True, "normal", True, 4, 0),
    (200, 520, 1536, "f16", "f16", True, "normal", True, 3, 0),
    (64, 700, 1024, "bf16", "f32", False, "normal", False, 2, 0),
    (300, 256, 960, "f16", "f32", True, "normal", True, 5, 8),
    (96, 384, 4096, "bf16", "bf16", False, "normal", True, 8, 0),
    (128, 300, 1024, "e4m3", "bf16", False, "normal", False, 4, 0),
    (128, 256, 2048, "e4m3", "f32", True, "normal", True, 2, 0),
    (96, 128, 512, "bf16", "f32", True, "int", True, 4, 0),
    (70, 90, 640, "f16", "f16", False, "int", True, 5, 0),
    (33, 257, 768, "f16", "f16", True, "normal", True, 1, 0),
    (40, 72, 96, "f32", "f32", True, "normal", True, 3, 0),
]


def _id(c):
    M, N, K, f, o, tb, d, b, s, pad = c
    return f"{M}x{N}x{K}-{f}-{o}-{'NT' if tb else 'NN'}-{d}{'-bias' if b else ''}-S{s}{f'-pad{pad}' if pad else ''}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_splitk_matches_oracle(tmm, case):
    M, N, K, fmt, out, tb, dist, bias, splits, pad = case
    dC, o, T, ops, _ = splitk_case(tmm, M, N, K, fmt, out, tb, dist, bias, splits,
                                   seed=5000 + 10 * CASES.index(case), pad=pad)
    check(dC, o, T, K, exact=(dist == "int"), what=_id(case), f8=(fmt == "e4m3"), f8_ops=ops)


def test_decode_layer_full_size(tmm):
    """The bench configuration: 256 rows through a 4096 x 4096 fp16 weight + bias,
    fp16 out, 4 slices, every element against the oracle."""
    dC, o, T, ops, _ = splitk_case(tmm, 256, 4096, 4096, "f16", "f16", True, "normal", True, 4, seed=5200)
    check(dC, o, T, 4096, what="splitk 256x4096x4096 S4")


def test_deterministic_and_workspace_reuse(tmm):
    """Two calls on the same inputs give the same bits; a smaller problem then
    reuses the larger one's workspace."""
    dC, o, T, ops, (dA, dB, dbias, ws, sa, sb) = splitk_case(
        tmm, 160, 384, 1024, "bf16", "bf16", True, "normal", True, 4, seed=5300)
    first = dC.clone()
    tmm.tmm_gemm_splitk(dA, dB, dC, bias=dbias, trans_b=True, splits=4, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), dC.view(torch.int16))
    small = torch.full((40, 100), float("nan"), dtype=torch.bfloat16, device=DEV)
    tmm.tmm_gemm_splitk(dA[:40, :512], dB[:100, :512], small, bias=dbias[:100], trans_b=True, splits=2,
                        workspace=ws)
    torch.cuda.synchronize()
    A = syn.normal((160, 1024), 5301)
    B = syn.normal((384, 1024), 5302)
    a_bits, b_bits = syn.to_bits(A, "bf16")[:40, :512], syn.to_bits(B, "bf16")[:100, :512]
    bvec = syn.normal((384,), 5303, 0.02).astype(np.float32)[:100]
    o2, T2 = oracle.gemm("bf16", a_bits, b_bits, trans_b=True, bias=bvec, want_abs=True)
    check(small, o2, T2, 512, what="splitk reused workspace, smaller problem")


def test_one_split_is_the_one_pass_product(tmm):
    """splits = 1 runs tmm_gemm itself (no workspace needed): the same bits."""
    A = on_gpu(syn.to_bits(syn.normal((96, 512), 5401), "f16"), "f16")
    B = on_gpu(syn.to_bits(syn.normal((200, 512), 5402), "f16"), "f16")
    c1 = torch.empty((96, 200), dtype=torch.float16, device=DEV)
    c2 = torch.empty((96, 200), dtype=torch.float16, device=DEV)
    tmm.tmm_gemm(A, B, c1, trans_b=True)
    tmm.tmm_gemm_splitk(A, B, c2, trans_b=True, splits=1, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
