"""Pins of the oracle's full BLAS form o = act(alpha op(A) op(B) + bias +
beta C) ("GEMM to FlashAttention" page: BLAS level 3 and the GEMM interface
box with transa / transb / alpha / beta; Lecture 27 notes section 2.1: a
unit computes f(sum x w + b), f = ReLU), against facts that do not come from
the oracle: numpy float64 products on the decoded inputs for tiny shapes,
integer closed forms, and the special cases alpha = 0, K = 0, beta = 0."""
import itertools

import numpy as np
import pytest

import oracle


def f16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def dec(bits):
    return oracle.decode("f16", bits)


@pytest.mark.parametrize("ta,tb", list(itertools.product([False, True], repeat=2)))
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 4), (6, 2, 7), (5, 8, 3)])
def test_against_numpy(ta, tb, shape):
    """All four layouts on tiny random problems: numpy's float64 product of
    the decoded, explicitly transposed operands."""
    M, N, K = shape
    g = np.random.default_rng([M, N, K, ta, tb])
    A = f16(g.normal(size=(K, M) if ta else (M, K)))
    B = f16(g.normal(size=(N, K) if tb else (K, N)))
    Cin = g.normal(size=(M, N))
    bias = g.normal(size=N).astype(np.float32)
    a = dec(A).T if ta else dec(A)
    b = dec(B).T if tb else dec(B)
    for alpha, beta, relu in [(1.0, 0.0, False), (0.75, -1.5, False), (-2.0, 0.5, True)]:
        o = oracle.gemm_ex("f16", A, B, ta, tb, alpha, beta, Cin if beta else None, bias, relu)
        want = alpha * (a @ b) + bias.astype(np.float64) + beta * Cin
        if relu:
            want = np.maximum(want, 0.0)
        np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-13)


def test_integer_closed_form():
    """a_ik = i + k, b_kj = k - j (stored transposed on both sides), alpha =
    2, beta = -3, c_ij = i - 2j, bias_j = j: every step is an exact integer,
    and sum_k (i+k)(k-j) = -Kij + (i-j)K(K-1)/2 + (K-1)K(2K-1)/6."""
    M, N, K = 7, 9, 11
    i = np.arange(M)[:, None].astype(np.float64)
    j = np.arange(N)[None, :].astype(np.float64)
    k = np.arange(K)
    A_t = f16((k[:, None] + np.arange(M)[None, :]))          # stored K x M
    B_t = f16((k[None, :] - np.arange(N)[:, None]))           # stored N x K
    Cin = i - 2 * j
    bias = np.arange(N, dtype=np.float32)
    s = -K * i * j + (i - j) * K * (K - 1) / 2 + (K - 1) * K * (2 * K - 1) / 6
    o = oracle.gemm_ex("f16", A_t, B_t, True, True, 2.0, -3.0, Cin, bias)
    assert np.array_equal(o, 2 * s + j - 3 * Cin)
    r = oracle.gemm_ex("f16", A_t, B_t, True, True, 2.0, -3.0, Cin, bias, relu=True)
    assert np.array_equal(r, np.maximum(2 * s + j - 3 * Cin, 0))


def test_alpha_zero_and_empty_sum_leave_beta_c_plus_bias():
    g = np.random.default_rng(7)
    M, N, K = 4, 6, 5
    A, B = f16(g.normal(size=(M, K))), f16(g.normal(size=(K, N)))
    Cin = g.normal(size=(M, N))
    bias = g.normal(size=N).astype(np.float32)
    o = oracle.gemm_ex("f16", A, B, alpha=0.0, beta=0.25, C_in=Cin, bias=bias)
    assert np.array_equal(o, 0.25 * Cin + bias.astype(np.float64))
    o = oracle.gemm_ex("f16", A[:, :0], B[:0], alpha=3.0, beta=0.25, C_in=Cin, bias=bias)
    assert np.array_equal(o, 0.25 * Cin + bias.astype(np.float64))


def test_beta_zero_ignores_c_and_matches_plain_product():
    """beta = 0 without C equals the plain oracle product (pinned on its own)."""
    g = np.random.default_rng(8)
    A, B = f16(g.normal(size=(6, 9))), f16(g.normal(size=(7, 9)))
    bias = g.normal(size=7).astype(np.float32)
    assert np.array_equal(oracle.gemm_ex("f16", A, B, trans_b=True, bias=bias),
                          oracle.gemm("f16", A, B, trans_b=True, bias=bias))


def test_relu_is_max_with_zero_and_abs_companion():
    g = np.random.default_rng(9)
    A, B = f16(g.normal(size=(5, 8))), f16(g.normal(size=(8, 6)))
    Cin = g.normal(size=(5, 6))
    o, T = oracle.gemm_ex("f16", A, B, alpha=1.5, beta=-0.5, C_in=Cin, want_abs=True)
    r = oracle.gemm_ex("f16", A, B, alpha=1.5, beta=-0.5, C_in=Cin, relu=True)
    assert np.array_equal(r, np.where(o > 0, o, 0.0))
    assert (r == 0).any() and (r > 0).any()
    assert np.all(np.abs(o) <= T * (1 + 1e-15))
    a, b = dec(A), dec(B)
    np.testing.assert_allclose(T, 1.5 * (np.abs(a) @ np.abs(b)) + 0.5 * np.abs(Cin), rtol=1e-13)


def test_rejects_bad_arguments():
    A = f16(np.ones((2, 3)))
    with pytest.raises(ValueError):
        oracle.gemm_ex("f16", A, f16(np.ones((4, 5))))
    with pytest.raises(ValueError):
        oracle.gemm_ex("f16", A, f16(np.ones((3, 2))), C_in=np.zeros((3, 3)), beta=1.0)


@pytest.mark.parametrize("ta,tb", list(itertools.product([False, True], repeat=2)))
def test_abs_companion_exact_with_bias_and_beta(ta, tb):
    """T = |alpha| |a'| |b'| + |bias| + |beta c| exactly on small integers
    (numpy's float64 product of the absolute values is exact here), with a
    negative alpha, beta and mixed-sign bias and C."""
    M, N, K = 5, 7, 9
    g = np.random.default_rng([51, ta, tb])
    a = g.integers(-4, 5, size=(M, K)).astype(np.float64)
    b = g.integers(-4, 5, size=(K, N)).astype(np.float64)
    A = f16(a.T if ta else a)
    B = f16(b.T if tb else b)
    bias = g.integers(-4, 5, size=N).astype(np.float32)
    Cin = g.integers(-4, 5, size=(M, N)).astype(np.float64)
    o, T = oracle.gemm_ex("f16", A, B, trans_a=ta, trans_b=tb, alpha=-1.5, beta=-0.75, C_in=Cin,
                          bias=bias, want_abs=True)
    want_T = 1.5 * (np.abs(a) @ np.abs(b)) + np.abs(bias.astype(np.float64))[None, :] + 0.75 * np.abs(Cin)
    assert np.array_equal(T, want_T)
    assert np.array_equal(o, -1.5 * (a @ b) + bias.astype(np.float64)[None, :] - 0.75 * Cin)


def test_abs_companion_equals_output_for_nonnegative_terms():
    """alpha, a, b, bias, beta and C all >= 0: every term is >= 0, so T = o exactly."""
    g = np.random.default_rng(52)
    A, B = f16(np.abs(g.normal(size=(6, 11)))), f16(np.abs(g.normal(size=(11, 4))))
    bias = np.abs(g.normal(size=4)).astype(np.float32)
    Cin = np.abs(g.normal(size=(6, 4)))
    o, T = oracle.gemm_ex("f16", A, B, alpha=0.75, beta=1.25, C_in=Cin, bias=bias, want_abs=True)
    assert np.array_equal(T, o)
