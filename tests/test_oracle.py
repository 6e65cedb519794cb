"""Pins of the oracle against facts that do not come from the oracle.

Each test would fail under a plausible mistake in oracle.c: a dropped term, a
transposed operand, a wrong stride, a sign or index slip, a wrong exponent
bias in a decoder, or a rounding rule other than nearest-even.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


def f32bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------- products


def test_brute_force_2x2_all_ternary():
    """All 3^8 pairs of 2x2 matrices over {-1,0,1}, against the expanded 2x2 product."""
    vals = (-1.0, 0.0, 1.0)
    for a00, a01, a10, a11, b00, b01, b10, b11 in itertools.product(vals, repeat=8):
        A = np.array([[a00, a01], [a10, a11]], dtype=np.float32)
        B = np.array([[b00, b01], [b10, b11]], dtype=np.float32)
        want = np.array([[a00 * b00 + a01 * b10, a00 * b01 + a01 * b11],
                         [a10 * b00 + a11 * b10, a10 * b01 + a11 * b11]])
        got = oracle.gemm("f32", f32bits(A), f32bits(B))
        assert np.array_equal(got, want), (A, B, got)
        # same product with B given transposed (stored N x K)
        got_t = oracle.gemm("f32", f32bits(A), f32bits(B.T.copy()), trans_b=True)
        assert np.array_equal(got_t, want)


@pytest.mark.parametrize("seed", range(40))
def test_tiny_random_against_numpy(seed):
    """Random shapes up to 7 (including empty ones) against numpy's float64 matmul."""
    g = np.random.default_rng(seed)
    M, N, K = (int(v) for v in g.integers(0, 8, 3))
    A = g.standard_normal((M, K)).astype(np.float32)
    B = g.standard_normal((K, N)).astype(np.float32)
    bias = g.standard_normal(N).astype(np.float32)
    want = A.astype(np.float64) @ B.astype(np.float64) + bias.astype(np.float64)
    got = oracle.gemm("f32", f32bits(A), f32bits(B), bias=bias)
    assert got.shape == (M, N)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_leading_dimension_is_a_stride():
    """Sub-matrix views with row stride > row length read the right elements."""
    g = np.random.default_rng(5)
    big_a = g.integers(-4, 5, (9, 13)).astype(np.float32)
    big_b = g.integers(-4, 5, (11, 17)).astype(np.float32)
    A = f32bits(big_a)[:, 2:9]         # 9 x 7, lda = 13
    B = f32bits(big_b)[4:11, 3:8]      # 7 x 5, ldb = 17
    want = big_a[:, 2:9].astype(np.int64) @ big_b[4:11, 3:8].astype(np.int64)
    assert np.array_equal(oracle.gemm("f32", A, B), want)


def test_identity_and_all_ones():
    g = np.random.default_rng(7)
    X = g.standard_normal((24, 24)).astype(np.float32)
    I = np.eye(24, dtype=np.float32)
    assert np.array_equal(oracle.gemm("f32", f32bits(X), f32bits(I)), X.astype(np.float64))
    assert np.array_equal(oracle.gemm("f32", f32bits(I), f32bits(X)), X.astype(np.float64))
    # all-ones: every entry is K (+ bias)
    M, N, K = 5, 9, 37
    bias = np.arange(N, dtype=np.float32) - 4
    got = oracle.gemm("bf16", np.full((M, K), 0x3F80, np.uint16), np.full((K, N), 0x3F80, np.uint16), bias=bias)
    assert np.array_equal(got, np.broadcast_to(K + bias.astype(np.float64), (M, N)))


def test_row_and_column_sums():
    """B = ones gives the row sums of A; A = ones gives the column sums of B (exact integers)."""
    g = np.random.default_rng(11)
    A = g.integers(-4, 5, (13, 29)).astype(np.float32)
    B = g.integers(-4, 5, (29, 6)).astype(np.float32)
    ones_b = np.ones((29, 6), np.float32)
    ones_a = np.ones((13, 29), np.float32)
    row = [sum(int(v) for v in A[i]) for i in range(13)]
    col = [sum(int(B[k, j]) for k in range(29)) for j in range(6)]
    got_r = oracle.gemm("f32", f32bits(A), f32bits(ones_b))
    got_c = oracle.gemm("f32", f32bits(ones_a), f32bits(B))
    for i in range(13):
        assert all(got_r[i, j] == row[i] for j in range(6))
        assert all(got_c[i, j] == col[j] for j in range(6))


def test_block_decomposition_identity_8x8x8():
    """The tiling figure of the "GEMM to FlashAttention" page: M=N=K=8 in 4x4 tiles,
    C00 = A00 B00 + A01 B10, C01 = A00 B01 + A01 B11, C10 = A10 B00 + A11 B10,
    C11 = A10 B01 + A11 B11."""
    g = np.random.default_rng(8)
    A = g.integers(-4, 5, (8, 8)).astype(np.float32)
    B = g.integers(-4, 5, (8, 8)).astype(np.float32)
    C = oracle.gemm("f32", f32bits(A), f32bits(B))
    t = lambda X, r, c: X[4 * r:4 * r + 4, 4 * c:4 * c + 4]
    mm = lambda X, Y: oracle.gemm("f32", f32bits(X.copy()), f32bits(Y.copy()))
    for r, c in itertools.product(range(2), range(2)):
        want = mm(t(A, r, 0), t(B, 0, c)) + mm(t(A, r, 1), t(B, 1, c))
        assert np.array_equal(t(C, r, c), want), (r, c)
    # The 4x4x4 tile product has 4*4*4 = 64 multiply-adds; an entry of C sums 8 of them.
    assert 4 * 4 * 4 == 64


@pytest.mark.parametrize("M,N,K", [(37, 37, 37), (50, 40, 300), (3, 200, 1023)])
def test_closed_form(M, N, K):
    """a_ik = i + k, b_kj = k - j  =>  C_ij = -K i j + (i - j) K(K-1)/2 + (K-1)K(2K-1)/6."""
    i = np.arange(M)[:, None]
    k = np.arange(K)
    j = np.arange(N)[None, :]
    A = (i + k[None, :]).astype(np.float32)
    B = (k[:, None] - j).astype(np.float32)
    s1 = K * (K - 1) // 2
    s2 = (K - 1) * K * (2 * K - 1) // 6
    want = -K * i * j + (i - j) * s1 + s2
    got = oracle.gemm("f32", f32bits(A), f32bits(B))
    assert np.array_equal(got, want.astype(np.float64))


def test_transpose_flag_matches_stored_transpose():
    g = np.random.default_rng(3)
    A = g.standard_normal((17, 33)).astype(np.float32)
    B = g.standard_normal((33, 21)).astype(np.float32)
    nn = oracle.gemm("f32", f32bits(A), f32bits(B))
    nt = oracle.gemm("f32", f32bits(A), f32bits(B.T.copy()), trans_b=True)
    assert np.array_equal(nn, nt)


def test_bias_and_scales():
    g = np.random.default_rng(4)
    A = g.integers(-4, 5, (6, 10)).astype(np.float32)
    B = g.integers(-4, 5, (10, 7)).astype(np.float32)
    bias = g.integers(-4, 5, 7).astype(np.float32)
    plain = A.astype(np.int64) @ B.astype(np.int64)
    got = oracle.gemm("f32", f32bits(A), f32bits(B), bias=bias, scale_a=0.5, scale_b=8.0)
    assert np.array_equal(got, 4.0 * plain + bias)


def test_abs_sum_bound_scale():
    """T = sum_k |a_ik b'_kj| equals |A| . |B| (and C itself when all entries are >= 0)."""
    g = np.random.default_rng(9)
    A = g.integers(-4, 5, (8, 19)).astype(np.float32)
    B = g.integers(-4, 5, (19, 5)).astype(np.float32)
    C, T = oracle.gemm("f32", f32bits(A), f32bits(B), want_abs=True)
    assert np.array_equal(T, np.abs(A).astype(np.int64) @ np.abs(B).astype(np.int64))
    C2, T2 = oracle.gemm("f32", f32bits(np.abs(A)), f32bits(np.abs(B)), want_abs=True)
    assert np.array_equal(C2, T2)


def test_empty_sum_and_empty_output():
    bias = np.array([1.5, -2.0, 0.25], np.float32)
    got = oracle.gemm("bf16", np.zeros((4, 0), np.uint16), np.zeros((0, 3), np.uint16), bias=bias)
    assert np.array_equal(got, np.broadcast_to(bias.astype(np.float64), (4, 3)))
    assert oracle.gemm("bf16", np.zeros((0, 5), np.uint16), np.zeros((5, 3), np.uint16)).shape == (0, 3)
    with pytest.raises(ValueError):
        oracle.gemm("bf16", np.zeros((2, 5), np.uint16), np.zeros((4, 3), np.uint16))


def test_low_precision_product_uses_decoded_values():
    """bf16 / fp16 / e4m3 products equal float64 products of the library-decoded inputs."""
    g = np.random.default_rng(12)
    x = g.standard_normal((9, 31)).astype(np.float32)
    y = g.standard_normal((31, 4)).astype(np.float32)
    for fmt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16), ("e4m3", torch.float8_e4m3fn)):
        ta, tb = torch.from_numpy(x).to(tdt), torch.from_numpy(y).to(tdt)
        bits_dt = torch.uint8 if fmt == "e4m3" else torch.int16
        npdt = np.uint8 if fmt == "e4m3" else np.uint16
        abits = ta.view(bits_dt).numpy().view(npdt)
        bbits = tb.view(bits_dt).numpy().view(npdt)
        want = ta.double().numpy() @ tb.double().numpy()
        got = oracle.gemm(fmt, abits, bbits)
        np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- codecs


def test_decode_bf16_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.decode("bf16", bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_f16_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = oracle.decode("f16", bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    assert oracle.decode("f16", np.array([1], np.uint16))[0] == 2.0 ** -24   # smallest subnormal


def test_decode_e4m3_all_patterns():
    bits = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(bits).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.decode("e4m3", bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2                     # S.1111.111 only: no infinities
    assert np.array_equal(got[~nan], want[~nan])
    # Lecture 27 notes, section 2.7: E4M3 spans 0 .. 448.
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0


def test_decode_f32_roundtrip():
    g = np.random.default_rng(1)
    x = g.standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.decode("f32", x.view(np.uint32)), x.astype(np.float64))


def _finite_grid(fmt):
    bits = np.arange(1 << 16, dtype=np.uint16)
    v = oracle.decode(fmt, bits)
    keep = np.isfinite(v) & (bits < 0x8000)           # non-negative finite values
    order = np.argsort(v[keep], kind="stable")
    return bits[keep][order], v[keep][order]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_round_exact_values_and_midpoints(fmt):
    """Every representable value rounds to itself; every midpoint rounds to the even neighbour."""
    bits, vals = _finite_grid(fmt)
    # drop the duplicate +0 / -0 ordering issue: vals strictly increasing after 0
    assert np.all(np.diff(vals) > 0)
    assert np.array_equal(oracle.round_to(fmt, vals), bits)
    assert np.array_equal(oracle.round_to(fmt, -vals)[1:], bits[1:] | 0x8000)
    mids = (vals[:-1] + vals[1:]) / 2                 # exact in float64
    even = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(oracle.round_to(fmt, mids), even)
    # just off the midpoint goes to the nearer side
    assert np.array_equal(oracle.round_to(fmt, np.nextafter(mids, 0)), bits[:-1])
    assert np.array_equal(oracle.round_to(fmt, np.nextafter(mids, np.inf)), bits[1:])


def test_round_against_library_conversions():
    g = np.random.default_rng(2)
    x = np.concatenate([g.standard_normal(200000) * s for s in (1e-6, 1e-3, 1.0, 1e3)])
    x = np.concatenate([x, g.standard_normal(20000) * 2.0 ** -20])       # fp16 subnormal range
    # fp16: numpy converts float64 -> float16 with one correct rounding
    assert np.array_equal(oracle.round_to("f16", x), x.astype(np.float16).view(np.uint16))
    # bf16: torch converts float32 -> bf16 with nearest-even; use float32-exact inputs
    x32 = x.astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to("bf16", x32), want)


def test_round_overflow_and_ties_at_edges():
    r16 = lambda v: int(oracle.round_to("f16", np.array([v]))[0])
    assert r16(65504.0) == 0x7BFF
    assert r16(65519.99) == 0x7BFF
    assert r16(65520.0) == 0x7C00                      # tie past the top rounds to infinity
    assert r16(2.0 ** -25) == 0x0000                   # half the smallest subnormal: tie to even (0)
    assert r16(3 * 2.0 ** -25) == 0x0002               # 1.5 quanta: tie to even (2)
    assert r16(-0.0) == 0x8000
    rb = lambda v: int(oracle.round_to("bf16", np.array([v]))[0])
    assert rb(1.0 + 2.0 ** -8) == 0x3F80               # tie between 1 and 1+2^-7 -> 1 (even)
    assert rb(1.0 + 3 * 2.0 ** -8) == 0x3F82           # tie -> 1+2^-6 (even)
    assert rb(float(np.finfo(np.float32).max)) == 0x7F80   # rounds past the top -> infinity
