"""Seeded synthetic inputs for the GEMM/GEMV workloads.

This module is the only thing the oracle side and the GPU side share.  It
draws random numbers and stores them in the input formats; it holds none of
the matrix-product arithmetic.  Rounding of the drawn float32 values into
bf16 / fp16 / fp8-e4m3 bit patterns uses torch's CPU conversions (round to
nearest even); fp8 inputs get one float32 scale per tensor, amax/448, so the
quantised values span the E4M3 range given in the CMU 15-418 Lecture 27
notes, section 2.7 (fp8 E4M3 range 0..448).

Seeds: numpy PCG64 ``default_rng``; large tensors are drawn in row blocks,
each block from its own stream ``default_rng([seed, block])`` so a sampled
subset of rows can be regenerated without drawing the whole tensor.

Workloads (sizes of the transformer layers and attention shapes of the
"GEMM to FlashAttention" page; linear weights are (out, in) as in its
linear-layer formula, so a linear layer is X . W^T):
  * fp32 256^3, N(0,1);
  * bf16 4096^3, N(0,1), fp32 output;
  * bf16 linear layers, activations N(0,1), weights and bias N(0, 0.02^2):
    QKV 8192x4096 -> 12288, FFN-up 8192x4096 -> 14336, FFN-down
    8192x14336 -> 4096, and the M=1 decode GEMV with W 4096x4096;
  * fp16 attention products, batch 4 x 32 heads, sequence 2048, head dim 128;
  * fp8 e4m3 8192^3 with per-tensor scales, bf16 output; and the ragged bf16
    shapes (1000, 3000, 777) and (4097, 511, 1023).
"""
from __future__ import annotations

import numpy as np
import torch

ROW_BLOCK = 1024  # rows per independent random stream

FP8_MAX = 448.0  # largest finite OCP E4M3 value

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
          "e4m3": torch.float8_e4m3fn}
_NP_BITS = {"f32": np.uint32, "bf16": np.uint16, "f16": np.uint16, "e4m3": np.uint8}
_TORCH_BITS = {"f32": torch.int32, "bf16": torch.int16, "f16": torch.int16,
               "e4m3": torch.uint8}


def seed_of(config: int, tensor: str) -> int:
    """Seed of one tensor of a workload: 1000*config + {A:1,B:2,bias:3,logits:4,V:5}."""
    return 1000 * config + {"A": 1, "B": 2, "bias": 3, "logits": 4, "V": 5}[tensor]


def normal(shape, seed: int, std: float = 1.0, rows=None) -> np.ndarray:
    """float32 N(0, std^2) of ``shape`` (2-D or 3-D); ``rows`` selects rows of the last-but-one axis."""
    shape = tuple(int(s) for s in shape)
    return _blocked(shape, seed, rows, lambda g, n: g.standard_normal(n, dtype=np.float32) * np.float32(std))


def uniform(shape, seed: int, lo: float = -0.5, hi: float = 0.5, rows=None) -> np.ndarray:
    """float32 uniform in [lo, hi) (the conv_fused listing's rand()/RAND_MAX - 0.5)."""
    shape = tuple(int(s) for s in shape)
    return _blocked(shape, seed, rows,
                    lambda g, n: (g.random(n, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)))


def small_ints(shape, seed: int, lo: int = -4, hi: int = 4, rows=None) -> np.ndarray:
    """float32 integers drawn uniformly from {lo, ..., hi}."""
    shape = tuple(int(s) for s in shape)
    return _blocked(shape, seed, rows, lambda g, n: g.integers(lo, hi + 1, n).astype(np.float32))


def _blocked(shape, seed, rows, draw):
    """Fill a 2-D (R, C) or 3-D (batch, R, C) array block of rows by block of rows."""
    if len(shape) == 1:
        g = np.random.default_rng([seed, 0])
        return draw(g, shape[0]).reshape(shape)
    lead = shape[:-2]
    R, C = shape[-2], shape[-1]
    nb = int(np.prod(lead)) if lead else 1
    sel = np.arange(R) if rows is None else np.asarray(rows)
    out = np.empty((nb, len(sel), C), dtype=np.float32)
    for b in range(nb):
        blocks = np.unique(sel // ROW_BLOCK)
        for blk in blocks:
            g = np.random.default_rng([seed, b, int(blk)])
            r0 = int(blk) * ROW_BLOCK
            nr = min(ROW_BLOCK, R - r0)
            vals = draw(g, nr * C).reshape(nr, C)
            m = (sel // ROW_BLOCK) == blk
            out[b, m] = vals[sel[m] - r0]
    return out.reshape(lead + (len(sel), C))


def to_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    """Bit patterns of float32 ``x`` stored in ``fmt`` (torch CPU conversion, RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if fmt == "f32":
        return t.numpy().view(np.uint32).copy()
    q = t.to(_TORCH[fmt])
    return q.view(_TORCH_BITS[fmt]).numpy().view(_NP_BITS[fmt]).copy()


def e4m3_scale(x: np.ndarray) -> np.float32:
    """Per-tensor fp8 scale: amax(|x|) / 448 in float32 (1 for an all-zero tensor)."""
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    return np.float32(amax / np.float32(FP8_MAX)) if amax > 0 else np.float32(1)


def quantize_e4m3(x: np.ndarray, scale: np.float32) -> np.ndarray:
    """E4M3 bit patterns of x/scale, clamped into [-448, 448] before rounding."""
    y = np.clip(x / np.float32(scale), -FP8_MAX, FP8_MAX).astype(np.float32)
    return to_bits(y, "e4m3")


def softmax_rows_f16(batch: int, n: int, seed: int, rows=None) -> np.ndarray:
    """fp16 bit patterns of row-softmax(N(0,1) logits) of shape (batch, n, n).

    The softmax is evaluated in float64 and rounded once to fp16 (RNE, keeping
    subnormals).  These are the attention weights of the unfused attention
    product weights x V.
    """
    out = []
    for b in range(batch):
        z = _blocked((n, n), seed + 7919 * b, rows, lambda g, m: g.standard_normal(m, dtype=np.float32))
        z = z.astype(np.float64)
        z -= z.max(axis=1, keepdims=True)
        e = np.exp(z)
        p = e / e.sum(axis=1, keepdims=True)
        out.append(torch.from_numpy(p).to(torch.float16).view(torch.int16).numpy().view(np.uint16))
    return np.stack(out)


def as_torch(bits: np.ndarray, fmt: str) -> torch.Tensor:
    """A CPU torch tensor of dtype ``fmt`` over the given bit patterns (copied)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(
        {np.uint32: np.int32, np.uint16: np.int16, np.uint8: np.uint8}[np.dtype(bits.dtype).type]).copy())
    return t.view(_TORCH[fmt])


# Shapes of the workloads, by name.
LINEAR_LAYERS = {
    "qkv": (8192, 12288, 4096),       # (M tokens, N out features, K in features)
    "ffn_up": (8192, 14336, 4096),
    "ffn_down": (8192, 4096, 14336),
}
GEMV_SHAPE = (4096, 4096)             # W (out, in)
ATTENTION = {"batch": 4, "heads": 32, "seq": 2048, "head_dim": 128}
SQUARE_BF16 = 4096
SQUARE_FP8 = 8192
RAGGED = [(1000, 3000, 777), (4097, 511, 1023)]
