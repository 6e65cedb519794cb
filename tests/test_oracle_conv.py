"""Pins of the oracle's fused convolution (CMU 15-418 Lecture 27 notes:
the convolution loop nest of section 2.2 and the conv_fused listing of
section 3.1 -- NHWC input with a zero halo, weights [K][R][S][C],
per-filter scale and bias, ReLU, 2 x 2 max pooling) against facts that do
not come from the oracle: a numpy brute force over an explicitly padded
input on tiny shapes, the 1 x 1 convolution as a matrix product, an
identity filter, and the count of in-image taps for all-ones inputs."""
import numpy as np
import pytest

import oracle


def f16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def numpy_conv(x, w, pad, scale, bias, relu, pool):
    N, H, W, C = x.shape
    K, R, S, _ = w.shape
    xp = np.zeros((N, H + 2 * pad, W + 2 * pad, C))
    xp[:, pad:pad + H, pad:pad + W, :] = x
    P, Q = H + 2 * pad - R + 1, W + 2 * pad - S + 1
    out = np.zeros((N, P, Q, K))
    for y in range(P):
        for xx in range(Q):
            patch = xp[:, y:y + R, xx:xx + S, :]                    # N R S C
            out[:, y, xx, :] = np.tensordot(patch, w, axes=([1, 2, 3], [1, 2, 3]))
    out = out * scale[None, None, None, :] + bias[None, None, None, :]
    if relu:
        out = np.maximum(out, 0)
    if pool == 2:
        out = out.reshape(N, P // 2, 2, Q // 2, 2, K).max(axis=(2, 4))
    return out


@pytest.mark.parametrize("shape", [(1, 4, 4, 3, 2, 3, 3, 1), (2, 6, 5, 4, 3, 3, 3, 1),
                                   (1, 5, 7, 2, 5, 1, 3, 0), (2, 4, 6, 3, 4, 3, 1, 2),
                                   (1, 6, 6, 8, 4, 5, 5, 2)])
@pytest.mark.parametrize("relu,pool", [(False, 1), (True, 1), (True, 2), (False, 2)])
def test_against_numpy(shape, relu, pool):
    N, H, W, C, K, R, S, pad = shape
    P, Q = H + 2 * pad - R + 1, W + 2 * pad - S + 1
    if pool == 2 and (P % 2 or Q % 2):
        pytest.skip("odd output for pooling")
    g = np.random.default_rng(list(shape) + [relu, pool])
    xb = f16(g.normal(size=(N, H, W, C)))
    wb = f16(g.normal(size=(K, R, S, C)))
    scale = (1 + 0.1 * g.normal(size=K)).astype(np.float32)
    bias = g.normal(size=K).astype(np.float32)
    o = oracle.conv2d("f16", xb, wb, pad, scale, bias, relu, pool)
    want = numpy_conv(oracle.decode("f16", xb), oracle.decode("f16", wb), pad,
                      scale.astype(np.float64), bias.astype(np.float64), relu, pool)
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-12)


def test_one_by_one_is_the_matrix_product():
    """R = S = 1, pad 0: conv = X (NHW x C) . W^T (C x K), the pinned GEMM."""
    g = np.random.default_rng(11)
    N, H, W, C, K = 2, 5, 3, 16, 7
    xb = f16(g.normal(size=(N, H, W, C)))
    wb = f16(g.normal(size=(K, 1, 1, C)))
    o = oracle.conv2d("f16", xb, wb, 0)
    ref = oracle.gemm("f16", xb.reshape(N * H * W, C), wb.reshape(K, C), trans_b=True)
    assert np.array_equal(o.reshape(N * H * W, K), ref)


def test_identity_filter_copies_the_input():
    """K = C, w[f][1][1][c] = [f == c]: a 3 x 3 'same' convolution returns the input."""
    N, H, W, C = 2, 6, 5, 4
    x = np.random.default_rng(12).normal(size=(N, H, W, C))
    w = np.zeros((C, 3, 3, C))
    for f in range(C):
        w[f, 1, 1, f] = 1.0
    o = oracle.conv2d("f16", f16(x), f16(w), 1)
    assert np.array_equal(o, oracle.decode("f16", f16(x)))


def test_all_ones_counts_in_image_taps():
    """Ones everywhere, 3 x 3, pad 1: corners see 4 taps, edges 6, the rest 9 (times C)."""
    N, H, W, C, K = 1, 5, 6, 3, 2
    o = oracle.conv2d("f16", f16(np.ones((N, H, W, C))), f16(np.ones((K, 3, 3, C))), 1)
    taps = np.full((H, W), 9.0)
    taps[0, :] = taps[-1, :] = 6
    taps[:, 0] = taps[:, -1] = 6
    taps[0, 0] = taps[0, -1] = taps[-1, 0] = taps[-1, -1] = 4
    assert np.array_equal(o[0, :, :, 0], C * taps)
    assert np.array_equal(o[0, :, :, 1], C * taps)


def test_pooled_is_max_of_unpooled_and_abs_companion():
    g = np.random.default_rng(13)
    xb = f16(g.normal(size=(2, 6, 8, 5)))
    wb = f16(g.normal(size=(3, 3, 3, 5)))
    bias = g.normal(size=3).astype(np.float32)
    full, T = oracle.conv2d("f16", xb, wb, 1, None, bias, True, 1, want_abs=True)
    pooled = oracle.conv2d("f16", xb, wb, 1, None, bias, True, 2)
    assert np.array_equal(pooled, full.reshape(2, 3, 2, 4, 2, 3).max(axis=(2, 4)))
    assert np.all(np.abs(full) <= T * (1 + 1e-15))


def test_rejects_odd_pooling():
    with pytest.raises(ValueError):
        oracle.conv2d("f16", f16(np.ones((1, 5, 5, 2))), f16(np.ones((1, 3, 3, 2))), 1, pool=2)


@pytest.mark.parametrize("pool", [1, 2])
def test_abs_companion_equals_output_for_nonnegative_terms(pool):
    """With x, w, scale and bias all >= 0 every term is >= 0, so the
    companion |scale| sum |w x| + |bias| is the output itself, exactly --
    unpooled and as the largest over each 2 x 2 window."""
    g = np.random.default_rng(21 + pool)
    xb = f16(np.abs(g.normal(size=(2, 6, 8, 5))))
    wb = f16(np.abs(g.normal(size=(4, 3, 3, 5))))
    scale = np.abs(g.normal(size=4)).astype(np.float32)
    bias = np.abs(g.normal(size=4)).astype(np.float32)
    o, T = oracle.conv2d("f16", xb, wb, 1, scale, bias, False, pool, want_abs=True)
    assert np.array_equal(T, o)
    assert np.all(o > 0)


def test_abs_companion_sign_terms_exact():
    """Small integers (exact in float64): x >= 0, w <= 0 and a negative
    scale give |scale| sum |w x| = scale * sum w x; a negative bias adds
    2 |bias| to the companion: T = o + 2 |bias| (no ReLU, no pooling)."""
    g = np.random.default_rng(31)
    x = g.integers(0, 5, size=(1, 5, 6, 3)).astype(np.float64)
    w = -g.integers(0, 5, size=(2, 3, 3, 3)).astype(np.float64)
    scale = np.array([-2.0, -0.5], dtype=np.float32)
    bias = np.array([-3.0, -1.0], dtype=np.float32)
    o, T = oracle.conv2d("f16", f16(x), f16(w), 1, scale, bias, False, 1, want_abs=True)
    assert np.array_equal(T, o + 2 * np.abs(bias.astype(np.float64))[None, None, None, :])
    # and the numpy brute force gives the same o (so T is pinned, not o against itself)
    assert np.array_equal(o, numpy_conv(x, w, 1, scale.astype(np.float64), bias.astype(np.float64),
                                        False, 1))


def test_pooled_companion_is_window_max_of_companions():
    """Mixed signs: the pooled companion is the largest unpooled companion of
    its 2 x 2 window, and the unpooled one is |scale| (|w| conv |x|) + |bias|
    from the numpy brute force on absolute values (small integers: exact)."""
    g = np.random.default_rng(41)
    x = g.integers(-4, 5, size=(2, 6, 4, 3)).astype(np.float64)
    w = g.integers(-4, 5, size=(3, 3, 3, 3)).astype(np.float64)
    scale = np.array([1.5, -2.0, 0.25], dtype=np.float32)
    bias = np.array([-1.0, 2.0, 0.0], dtype=np.float32)
    _, T1 = oracle.conv2d("f16", f16(x), f16(w), 1, scale, bias, True, 1, want_abs=True)
    _, T2 = oracle.conv2d("f16", f16(x), f16(w), 1, scale, bias, True, 2, want_abs=True)
    ref = numpy_conv(np.abs(x), np.abs(w), 1, np.abs(scale.astype(np.float64)),
                     np.abs(bias.astype(np.float64)), False, 1)
    assert np.array_equal(T1, ref)
    assert np.array_equal(T2, ref.reshape(2, 3, 2, 2, 2, 3).max(axis=(2, 4)))
