"""Seeded GEMM cases for the GPU parity tests: operands built by the synthetic
generators, the expected result from the oracle, the result from the HIP path
through the C ABI."""
import numpy as np
import torch

import oracle
import synthetic as syn
from parity import f8_operands

DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
            "e4m3": torch.float8_e4m3fn}


def on_gpu(bits: np.ndarray, fmt: str) -> torch.Tensor:
    return syn.as_torch(bits, fmt).to(DEV)


def make_operand(shape, fmt, dist, seed, pad=0, scale=None):
    """Bits of a (rows, cols) operand, stored with `pad` extra elements per row.
    Returns (full padded bits, view of the logical part, fp8 scale)."""
    rows, cols = shape
    if dist == "int":
        x = syn.small_ints((rows, cols + pad), seed)
    else:
        x = syn.normal((rows, cols + pad), seed)
    s = np.float32(1.0)
    if fmt == "e4m3":
        if dist != "int":
            s = syn.e4m3_scale(x[:, :cols])
        bits = syn.quantize_e4m3(x, s)
    else:
        bits = syn.to_bits(x, fmt)
    return bits, bits[:, :cols], s


def gemm_case(tmm, M, N, K, fmt, out, trans_b, dist, bias, seed=0, pad=0, want_ops=False):
    """(C on the GPU, oracle o, oracle T[, fp8 operands for parity.check or None])."""
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
    tmm.tmm_gemm(dA, dB, dC, bias=dbias, trans_b=trans_b, scale_a=float(sa), scale_b=float(sb))
    torch.cuda.synchronize()
    if want_ops:
        ops = f8_operands(A, B, trans_b, float(sa) * float(sb)) if fmt == "e4m3" else None
        return dC, o, T, ops
    return dC, o, T
