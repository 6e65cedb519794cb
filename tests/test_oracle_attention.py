"""Pins of the oracle's attention, o = softmax(scale * Q K^T) V ("GEMM to
FlashAttention" page: the attention formula and the attention_standard
listing), against facts that do not come from the oracle itself: an
independent softmax routine on tiny inputs, closed forms, exact special cases
and the invariances of softmax."""
import numpy as np
import pytest
import scipy.special

import oracle


def f16_bits(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def bf16_bits(x):
    import torch
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def decode16(bits, fmt):
    return oracle.decode(fmt, bits)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 4), (7, 2, 3), (4, 9, 8), (6, 6, 16)])
def test_against_scipy_softmax(fmt, shape):
    """Tiny random problems against scipy.special.softmax (independent routine)."""
    Nq, Nk, D = shape
    g = np.random.default_rng([Nq, Nk, D, 0 if fmt == "f16" else 1])
    enc = f16_bits if fmt == "f16" else bf16_bits
    Qb, Kb, Vb = (enc(g.normal(size=s)) for s in ((Nq, D), (Nk, D), (Nk, D)))
    scale = 0.7
    o = oracle.attention(fmt, Qb, Kb, Vb, scale)
    q, k, v = (decode16(b, fmt) for b in (Qb, Kb, Vb))
    want = scipy.special.softmax(scale * (q @ k.T), axis=1) @ v
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-14)


def test_zero_queries_average_the_values():
    """Q = 0: every weight is 1/Nk, so each output row is the mean of V's rows."""
    g = np.random.default_rng(1)
    Nq, Nk, D = 5, 37, 8
    Qb = f16_bits(np.zeros((Nq, D)))
    Kb = f16_bits(g.normal(size=(Nk, D)))
    V = np.asarray(g.integers(-8, 9, size=(Nk, D)), dtype=np.float64)
    o = oracle.attention("f16", Qb, Kb, f16_bits(V), 0.125)
    np.testing.assert_allclose(o, np.broadcast_to(V.mean(axis=0), (Nq, D)), rtol=1e-15, atol=0)


def test_single_key_copies_its_value():
    """Nk = 1: the only weight is 1, so o = v[0] exactly, whatever the scores."""
    g = np.random.default_rng(2)
    V = np.asarray(g.normal(size=(1, 16)), dtype=np.float16)
    o = oracle.attention("f16", f16_bits(g.normal(size=(9, 16))), f16_bits(g.normal(size=(1, 16))),
                         V.view(np.uint16), 1.0)
    assert np.array_equal(o, np.broadcast_to(V.astype(np.float64), (9, 16)))


def test_dominant_key_selects_its_value():
    """One score 1280 above all others: exp of the rest underflows to 0 in
    double, so each output row is exactly that key's value row."""
    D, Nk, star = 8, 11, 6
    Q = np.zeros((3, D)); Q[:, 0] = 8.0
    K = np.zeros((Nk, D)); K[star, 0] = 8.0
    V = np.arange(Nk * D, dtype=np.float64).reshape(Nk, D) - 40.0
    o = oracle.attention("f16", f16_bits(Q), f16_bits(K), f16_bits(V), 20.0)
    assert np.array_equal(o, np.broadcast_to(V[star], (3, D)))


def test_key_permutation_invariance():
    """Permuting the keys together with their values changes nothing."""
    g = np.random.default_rng(3)
    Nq, Nk, D = 6, 40, 16
    Qb, Kb, Vb = (f16_bits(g.normal(size=s)) for s in ((Nq, D), (Nk, D), (Nk, D)))
    perm = g.permutation(Nk)
    a = oracle.attention("f16", Qb, Kb, Vb, 0.25)
    b = oracle.attention("f16", Qb, Kb[perm], Vb[perm], 0.25)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_score_shift_invariance():
    """Adding one vector u to every key adds scale*q.u to all scores of query
    row q alike, which the softmax ignores (small integers: exact in fp16)."""
    g = np.random.default_rng(4)
    Nq, Nk, D = 5, 23, 8
    Q = g.integers(-3, 4, size=(Nq, D)).astype(np.float64)
    K = g.integers(-3, 4, size=(Nk, D)).astype(np.float64)
    u = g.integers(-3, 4, size=(1, D)).astype(np.float64)
    Vb = f16_bits(g.normal(size=(Nk, D)))
    a = oracle.attention("f16", f16_bits(Q), f16_bits(K), Vb, 0.3)
    b = oracle.attention("f16", f16_bits(Q), f16_bits(K + u), Vb, 0.3)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_two_halves_merge_like_online_softmax():
    """The result over all keys equals the merge of the results over two key
    halves, each weighted by its exp-sum relative to the common maximum (the
    associativity the page's flash_attention_simplified listing and the
    Lecture 27 online-softmax slide rely on).  Per-half maxima and sums come
    from numpy on the decoded inputs."""
    g = np.random.default_rng(5)
    Nq, Nk, D, h = 4, 30, 8, 13
    Qb, Kb, Vb = (f16_bits(g.normal(size=s)) for s in ((Nq, D), (Nk, D), (Nk, D)))
    scale = 0.9
    full = oracle.attention("f16", Qb, Kb, Vb, scale)
    o1 = oracle.attention("f16", Qb, Kb[:h], Vb[:h], scale)
    o2 = oracle.attention("f16", Qb, Kb[h:], Vb[h:], scale)
    q, k = decode16(Qb, "f16"), decode16(Kb, "f16")
    s = scale * (q @ k.T)
    m1, m2 = s[:, :h].max(1), s[:, h:].max(1)
    m = np.maximum(m1, m2)
    l1 = np.exp(s[:, :h] - m1[:, None]).sum(1) * np.exp(m1 - m)
    l2 = np.exp(s[:, h:] - m2[:, None]).sum(1) * np.exp(m2 - m)
    merged = (l1[:, None] * o1 + l2[:, None] * o2) / (l1 + l2)[:, None]
    np.testing.assert_allclose(full, merged, rtol=1e-12, atol=1e-14)


def test_abs_companion():
    """T = sum_j w_ij |v_jc|: equals o when V >= 0, and bounds |o| always."""
    g = np.random.default_rng(6)
    Nq, Nk, D = 5, 17, 8
    Qb, Kb = (f16_bits(g.normal(size=s)) for s in ((Nq, D), (Nk, D)))
    Vpos = f16_bits(np.abs(g.normal(size=(Nk, D))))
    o, T = oracle.attention("f16", Qb, Kb, Vpos, 0.5, want_abs=True)
    np.testing.assert_allclose(o, T, rtol=1e-15)
    Vb = f16_bits(g.normal(size=(Nk, D)))
    o, T = oracle.attention("f16", Qb, Kb, Vb, 0.5, want_abs=True)
    assert np.all(np.abs(o) <= T * (1 + 1e-15))


def test_rejects_empty_key_set():
    with pytest.raises(ValueError):
        oracle.attention("f16", f16_bits(np.ones((2, 4))), f16_bits(np.ones((0, 4))),
                         f16_bits(np.ones((0, 4))), 1.0)
