"""GPU parity of the fused attention forward, O = softmax(scale Q K^T) V per
head ("GEMM to FlashAttention" page: attention formula; online evaluation as
in its flash_attention_simplified listing), against the oracle's fp64
attention on the same seeded inputs.

Tolerance (the page gives none; this follows from the kernel's arithmetic):
scores and running sums are fp32, and the only coarse step is the rounding
of each unnormalised weight e_j = exp(s_j - m) in (0, 1] to the input type
before the second product.  That changes e_j by at most u e_j (u = 2^-11
for fp16, 2^-8 for bf16, half an ulp) plus, for fp16, half the subnormal
spacing 2^-25; the exp-sum l >= 1 uses the unrounded e_j.  So

  |g - o| <= 2 u T + 2^-25 sum_j |v_jc| (fp16 only) [+ 1 ulp(R(o)) for a
  16-bit output]

with T = sum_j w_j |v_jc| (the oracle's companion); the factor 2 covers the
fp32 score error (< 1e-5 relative for these sizes, times |s| <= 10) and the
fp32 sums.  A wrong key, a missed rescale or a dropped block moves outputs
by O(T) and fails it; the exact cases below are held bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, TORCH_DT, on_gpu
from parity import fmt_of, to_bits, ulp

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


def check_attn(g: torch.Tensor, o: np.ndarray, T: np.ndarray, vabs: np.ndarray, fmt: str, what: str):
    """g: (Nq, D) GPU output; o, T: oracle; vabs: sum_j |v_jc| per column."""
    f = fmt_of(g)
    gv = oracle.decode(f, to_bits(g))
    assert np.all(np.isfinite(gv)), f"{what}: non-finite output"
    bound = 2 * U[fmt] * T + (2.0 ** -25 * vabs[None, :] if fmt == "f16" else 0.0)
    if f != "f32":
        bound = bound + ulp(f, oracle.decode(f, oracle.round_to(f, o)))
    bad = np.abs(gv - o) > bound
    n = int(bad.sum())
    if n:
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {n} of {bad.size} outputs beyond the bound; first {list(i)}: "
                             f"gpu {gv[i]!r} oracle {o[i]!r} bound {bound[i]!r}")


def operands(Z, Nq, Nk, D, fmt, seed, pad=0, qscale=1.0):
    """Bits of Q (Z, Nq, D+pad), K and V (Z, Nk, D+pad); N(0,1) entries
    (Q times qscale), the recipe of the attention workloads."""
    Q = syn.to_bits(syn.normal((Z, Nq, D + pad), seed + 1) * np.float32(qscale), fmt)
    K = syn.to_bits(syn.normal((Z, Nk, D + pad), seed + 2), fmt)
    V = syn.to_bits(syn.normal((Z, Nk, D + pad), seed + 5), fmt)
    return Q, K, V


def run(tmm, Q, K, V, D, fmt, out, scale, ostride_pad=0):
    """Upload (views of the first D columns), run, return the (Z, Nq, D) output view."""
    dQ, dK, dV = (on_gpu(X, fmt)[:, :, :D] for X in (Q, K, V))
    Z, Nq = Q.shape[0], Q.shape[1]
    Ofull = torch.full((Z, Nq * D + ostride_pad), float("nan"), dtype=TORCH_DT[out], device=DEV)
    dO = Ofull[:, :Nq * D].view(Z, Nq, D)
    tmm.tmm_attention_fwd(dQ, dK, dV, dO, scale=scale)
    torch.cuda.synchronize()
    return dO, Ofull


# (Z, Nq, Nk, D, in, out, pad): ragged query and key counts, one key, one
# query, several blocks of both, padded rows, both head sizes, every output type.
CASES = [
    (1, 128, 64, 128, "f16", "f16", 0),
    (2, 200, 77, 128, "f16", "f16", 0),
    (3, 130, 300, 64, "bf16", "bf16", 0),
    (1, 1, 1, 128, "f16", "f32", 0),
    (2, 5, 64, 64, "bf16", "f32", 0),
    (1, 257, 1000, 128, "bf16", "bf16", 8),
    (2, 300, 129, 64, "f16", "f32", 16),
    (1, 64, 513, 128, "f16", "f16", 24),
    (4, 129, 65, 128, "bf16", "f32", 0),
]


def _id(c):
    Z, Nq, Nk, D, f, o, pad = c
    return f"{f}-{o}-Z{Z}-{Nq}x{Nk}-D{D}{f'-pad{pad}' if pad else ''}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_attention_parity(tmm, case):
    Z, Nq, Nk, D, fmt, out, pad = case
    seed = 500 + 10 * CASES.index(case)
    Q, K, V = operands(Z, Nq, Nk, D, fmt, seed, pad)
    scale = 1.0 / math.sqrt(D)
    dO, Ofull = run(tmm, Q, K, V, D, fmt, out, scale, ostride_pad=8 if Z > 1 else 0)
    for z in range(Z):
        q, k, v = (np.ascontiguousarray(X[z][:, :D]) for X in (Q, K, V))
        o, T = oracle.attention(fmt, q, k, v, scale, want_abs=True)
        vabs = np.abs(oracle.decode(fmt, v)).sum(axis=0)
        check_attn(dO[z], o, T, vabs, fmt, f"{_id(case)} z {z}")
    if Z > 1:   # the padding between O matrices is left alone
        assert torch.isnan(Ofull[:, Nq * D:].float()).all()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_sharp_scores(tmm, fmt):
    """Large scale: the running maximum jumps between key blocks, so the
    rescaling of earlier partial sums is exercised at full strength."""
    Z, Nq, Nk, D = 2, 128, 512, 64
    Q, K, V = operands(Z, Nq, Nk, D, fmt, 777)
    scale = 2.0
    dO, _ = run(tmm, Q, K, V, D, fmt, "f32", scale)
    for z in range(Z):
        o, T = oracle.attention(fmt, Q[z], K[z], V[z], scale, want_abs=True)
        vabs = np.abs(oracle.decode(fmt, V[z])).sum(axis=0)
        check_attn(dO[z], o, T, vabs, fmt, f"sharp {fmt} z {z}")


@pytest.mark.parametrize("D", [64, 128])
def test_zero_queries_average_exactly(tmm, D):
    """Q = 0: every weight is exp(0) = 1 exactly, so O is the column mean of
    V; with small-integer V and a power-of-two key count every step is exact."""
    Nq, Nk = 150, 256
    Q = syn.to_bits(np.zeros((1, Nq, D), np.float32), "f16")
    K = syn.to_bits(syn.normal((1, Nk, D), 31), "f16")
    Vf = syn.small_ints((1, Nk, D), 32)
    V = syn.to_bits(Vf, "f16")
    dO, _ = run(tmm, Q, K, V, D, "f16", "f32", 0.125)
    want = np.broadcast_to(Vf[0].astype(np.float64).mean(axis=0), (Nq, D))
    got = oracle.decode("f32", to_bits(dO[0]))
    assert np.array_equal(got, want)


def test_single_key_is_copied(tmm):
    """Nk = 1: the weight is 1 and l = 1, so O equals the value row exactly."""
    Q, K, V = operands(2, 70, 1, 128, "bf16", 41)
    dO, _ = run(tmm, Q, K, V, 128, "bf16", "bf16", 0.5)
    got = to_bits(dO)
    assert np.array_equal(got, np.broadcast_to(V[:, :1, :], got.shape))


def test_dominant_key_is_selected(tmm):
    """One key scores 1280 above the rest (in a block past the first, so the
    maximum changes on the way): every other weight underflows to 0 in fp32
    and each output row is that key's value row, bit for bit."""
    D, Nk, star = 64, 200, 150
    Qf = np.zeros((1, 90, D), np.float32); Qf[0, :, 0] = 8.0
    Kf = syn.normal((1, Nk, D), 51) * np.float32(0.01); Kf[0, star, :] = 0; Kf[0, star, 0] = 8.0
    Q, K = syn.to_bits(Qf, "f16"), syn.to_bits(Kf, "f16")
    V = syn.to_bits(syn.normal((1, Nk, D), 52), "f16")
    dO, _ = run(tmm, Q, K, V, D, "f16", "f16", 20.0)
    got = to_bits(dO[0])
    assert np.array_equal(got, np.broadcast_to(V[0, star], got.shape))


def test_rows_are_independent_of_other_queries(tmm):
    """Each query's output depends on that query alone: the first 40 rows of
    a 300-query problem equal a 40-query problem's bit for bit."""
    Q, K, V = operands(1, 300, 333, 128, "f16", 61)
    a, _ = run(tmm, Q, K, V, 128, "f16", "f16", 0.09)
    b, _ = run(tmm, np.ascontiguousarray(Q[:, :40]), K, V, 128, "f16", "f16", 0.09)
    assert torch.equal(a[0, :40].view(torch.int16), b[0].view(torch.int16))


@pytest.mark.slow
def test_full_size_sampled(tmm):
    """The attention workload at full size, batch 4 x 32 heads, 2048 queries
    and keys, head size 128, fp16 in and out, as the benchmark runs it;
    sampled query rows of a few heads against the oracle."""
    Z, N, D = 128, 2048, 128
    Q, K, V = (syn.to_bits(syn.normal((Z, N, D), syn.seed_of(7, t)), "f16") for t in ("A", "B", "V"))
    scale = 1.0 / math.sqrt(D)
    dO, _ = run(tmm, Q, K, V, D, "f16", "f16", scale)
    g = np.random.default_rng(7)
    for z in (0, 37, 127):
        rows = np.sort(g.choice(N, 24, replace=False))
        o, T = oracle.attention("f16", np.ascontiguousarray(Q[z][rows]), K[z], V[z], scale, want_abs=True)
        vabs = np.abs(oracle.decode("f16", V[z])).sum(axis=0)
        check_attn(dO[z][torch.from_numpy(rows).to(DEV)], o, T, vabs, "f16", f"full z {z}")
