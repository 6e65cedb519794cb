"""GPU parity at the full workload sizes, in the launch configuration bench.py
times: every output of a seeded sample of rows and of columns is compared with
the oracle (which computes those outputs one row / one column at a time)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from parity import check, f8_operands

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda:0"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


def on_gpu(bits, fmt):
    return syn.as_torch(bits, fmt).to(DEV)


def sampled_check(C, A, B, fmt, trans_b, bias=None, sa=1.0, sb=1.0, nrows=32, ncols=32, seed=0,
                  what="", f8=False):
    """Check rows `I` (all columns) and columns `J` (all rows) of the GPU result C."""
    M, K = A.shape
    N = B.shape[0] if trans_b else B.shape[1]
    g = np.random.default_rng(seed)
    I = np.sort(g.choice(M, size=min(nrows, M), replace=False))
    J = np.sort(g.choice(N, size=min(ncols, N), replace=False))
    o_r, t_r = oracle.gemm(fmt, np.ascontiguousarray(A[I]), B, trans_b=trans_b, bias=bias,
                           scale_a=sa, scale_b=sb, want_abs=True)
    ops_r = ops_c = None
    if f8:
        qa, qb, sc = f8_operands(A, B, trans_b, sa * sb)
        ops_r = (qa[I], qb, sc)
        ops_c = (qa, qb[:, J], sc)
    check(C[torch.as_tensor(I, device=C.device)], o_r, t_r, K, what=f"{what} rows", f8=f8, f8_ops=ops_r)
    Bj = np.ascontiguousarray(B[J]) if trans_b else np.ascontiguousarray(B[:, J])
    bj = None if bias is None else np.ascontiguousarray(bias[J])
    o_c, t_c = oracle.gemm(fmt, A, Bj, trans_b=trans_b, bias=bj, scale_a=sa, scale_b=sb, want_abs=True)
    check(C[:, torch.as_tensor(J, device=C.device)].contiguous(), o_c, t_c, K, what=f"{what} cols", f8=f8,
          f8_ops=ops_c)


def test_square_bf16_4096(tmm):
    """bf16 4096^3 NN, fp32 output, no bias (the headline workload)."""
    n = syn.SQUARE_BF16
    A = syn.to_bits(syn.normal((n, n), syn.seed_of(2, "A")), "bf16")
    B = syn.to_bits(syn.normal((n, n), syn.seed_of(2, "B")), "bf16")
    C = torch.empty((n, n), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm(on_gpu(A, "bf16"), on_gpu(B, "bf16"), C)
    torch.cuda.synchronize()
    sampled_check(C, A, B, "bf16", False, nrows=48, ncols=48, seed=2, what="bf16 4096^3")


@pytest.mark.parametrize("layer", ["qkv", "ffn_up", "ffn_down"])
def test_linear_layers(tmm, layer):
    """X . W^T + b in bf16 with fp32 accumulation and bf16 output (and fp32 output)."""
    M, N, K = syn.LINEAR_LAYERS[layer]
    X = syn.to_bits(syn.normal((M, K), syn.seed_of(3, "A")), "bf16")
    W = syn.to_bits(syn.normal((N, K), syn.seed_of(3, "B"), 0.02), "bf16")
    b = syn.normal((N,), syn.seed_of(3, "bias"), 0.02)
    dX, dW, db = on_gpu(X, "bf16"), on_gpu(W, "bf16"), torch.from_numpy(b).to(DEV)
    for out in ("bf16", "f32"):
        C = torch.empty((M, N), dtype=TDT[out], device=DEV)
        tmm.tmm_gemm(dX, dW, C, bias=db, trans_b=True)
        torch.cuda.synchronize()
        sampled_check(C, X, W, "bf16", True, bias=b, nrows=16, ncols=16, seed=3,
                      what=f"{layer} {out}")
        del C


def test_attention_products(tmm):
    """S = Q . K^T (NT) and O = P . V (NN), batch 4 x 32 heads, sequence 2048, head dim 128, fp16."""
    a = syn.ATTENTION
    Z, n, d = a["batch"] * a["heads"], a["seq"], a["head_dim"]
    Q = syn.to_bits(syn.normal((Z, n, d), syn.seed_of(4, "A")), "f16")
    Kt = syn.to_bits(syn.normal((Z, n, d), syn.seed_of(4, "B")), "f16")
    S = torch.empty((Z, n, n), dtype=torch.float16, device=DEV)
    tmm.tmm_gemm_strided_batched(on_gpu(Q, "f16"), on_gpu(Kt, "f16"), S, trans_b=True)
    torch.cuda.synchronize()
    for z in (0, 77, Z - 1):
        sampled_check(S[z], Q[z], Kt[z], "f16", True, nrows=16, ncols=16, seed=z, what=f"S[{z}]")
    del S
    P = syn.softmax_rows_f16(Z, n, syn.seed_of(4, "logits"))
    V = syn.to_bits(syn.normal((Z, n, d), syn.seed_of(4, "V")), "f16")
    O = torch.empty((Z, n, d), dtype=torch.float16, device=DEV)
    tmm.tmm_gemm_strided_batched(on_gpu(P, "f16"), on_gpu(V, "f16"), O)
    torch.cuda.synchronize()
    for z in (0, 77, Z - 1):
        sampled_check(O[z], P[z], V[z], "f16", False, nrows=16, ncols=16, seed=z, what=f"O[{z}]")


def test_fp8_8192(tmm):
    """e4m3 8192^3 NN with per-tensor scales, bf16 output."""
    n = syn.SQUARE_FP8
    xa = syn.normal((n, n), syn.seed_of(5, "A"))
    xb = syn.normal((n, n), syn.seed_of(5, "B"))
    sa, sb = syn.e4m3_scale(xa), syn.e4m3_scale(xb)
    A, B = syn.quantize_e4m3(xa, sa), syn.quantize_e4m3(xb, sb)
    del xa, xb
    C = torch.empty((n, n), dtype=torch.bfloat16, device=DEV)
    tmm.tmm_gemm(on_gpu(A, "e4m3"), on_gpu(B, "e4m3"), C, scale_a=float(sa), scale_b=float(sb))
    torch.cuda.synchronize()
    sampled_check(C, A, B, "e4m3", False, sa=float(sa), sb=float(sb), nrows=12, ncols=12, seed=5,
                  what="fp8 8192^3", f8=True)


def test_decode_gemv_via_gemm_dispatch(tmm):
    """M = 1 through tmm_gemm (GEMV kernel) at the decode shape, every output checked."""
    N, K = syn.GEMV_SHAPE
    W = syn.to_bits(syn.normal((N, K), syn.seed_of(3, "B"), 0.02), "bf16")
    x = syn.to_bits(syn.normal((1, K), syn.seed_of(3, "A")), "bf16")
    b = syn.normal((N,), syn.seed_of(3, "bias"), 0.02)
    y = torch.empty((1, N), dtype=torch.bfloat16, device=DEV)
    tmm.tmm_gemm(on_gpu(x, "bf16"), on_gpu(W, "bf16"), y, bias=torch.from_numpy(b).to(DEV), trans_b=True)
    torch.cuda.synchronize()
    o, T = oracle.gemm("bf16", x, W, trans_b=True, bias=b, want_abs=True)
    check(y, o, T, K, what="decode GEMV")
