"""Comparison rules between the HIP path and the oracle.

Tolerances (the pages give none; these follow from the arithmetic):
  * small-integer inputs: every product and partial sum is an integer below
    2^24, exact in fp32, so the GPU result must equal the oracle bit for bit,
    also after rounding to bf16/fp16 (nearest-even on both sides);
  * fp32 outputs: relative Frobenius error  ||g - o||_F / ||o||_F <= 1e-5;
  * bf16/fp16 outputs: |g - R(o)| <= 1 ulp(R(o)) elementwise, where R is the
    oracle's nearest-even rounding; an element that misses this is accepted
    only where cancellation makes fp32 summation error exceed half an ulp:
    |g - o| <= ulp(R(o)) + 4 sqrt(K) 2^-24 T  with T = sum_k |a_ik b_kj|
    (probabilistic fp32 summation bound with lambda = 4);
  * fp8 inputs: the gfx950 fp8 matrix instruction (32x32x64) sums each run
    of 8 consecutive k (one 8-byte register piece per lane) by aligning the
    8 products to the largest one's binary exponent e and dropping every bit
    below 2^(e-13), toward zero; the accumulator and the group sums are then
    added without that loss.  Measured on gfx950 with single instructions:
    1 + 2^-13 is kept and 1 + 2^-14 comes back as 1 (also 1 - 2^-14 and
    -1 + 2^-14), 448 + 2^-5 is kept and 448 + 2^-6 is lost, 1 + 7 * 2^-14
    comes back as 1 (each product truncated alone), a run of 8 products
    with the large one in another run is exact, c = 448 plus 64 * 2^-9 is
    exact (the accumulator takes no part).  A product of two e4m3 values
    has at most 8 significant bits, so it loses bits only when its exponent
    is below e - 6, and then at most d_k = min(|p_k|, 2^(e-13)).  Per element
    the loss is  -sum_k sign(p_k) f_k  with 0 <= f_k < d_k; the allowance
    is its mean's size plus a lambda-sigma band,
        s_a s_b ( |sum_k sign(p_k) d_k| / 2 + LAMBDA_F8 sqrt(sum_k d_k^2 / 12) ),
    (f_k taken as uniform on [0, d_k)), added to the fp32 allowance above,
    and never more than the worst case s_a s_b sum_k d_k.  Beyond the
    elementwise rule, the fp8 target's 1e-3 is held as a relative
    Frobenius error on every 32x32 block (an accumulator tile), so an error
    confined to one block cannot hide in the whole matrix's norm.
  * the elements accepted only by an allowance beyond 1 ulp are counted;
    more than LOOSE_MAX of them fails the check.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

FRO_TOL_F32 = 1e-5
FRO_TOL_F8 = 1e-3
LAMBDA = 4.0
LAMBDA_F8 = 6.0
F8_KEEP = 13       # bits kept below a run's largest product exponent
F8_RUN = 8         # products aligned together (8 consecutive k)
LOOSE_MAX = 0.02   # largest share of elements accepted only by an allowance
BLOCK = 32         # accumulator tile edge for the blockwise Frobenius rule

_P = {"bf16": (8, -126), "f16": (11, -14)}   # significant bits, smallest normal exponent


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a CPU/GPU tensor as a numpy unsigned array."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def fmt_of(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16",
            torch.float8_e4m3fn: "e4m3"}[t.dtype]


def ulp(fmt: str, v: np.ndarray) -> np.ndarray:
    p, emin = _P[fmt]
    a = np.abs(v)
    e = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))), emin)
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int64))


def rel_fro(g: np.ndarray, o: np.ndarray) -> float:
    den = float(np.linalg.norm(o))
    num = float(np.linalg.norm(g - o))
    return num / den if den > 0 else num


def check_exact(g: torch.Tensor, o: np.ndarray, what: str = ""):
    """Bit-exact: fp32 output equals o; a rounded output equals R(o)."""
    f = fmt_of(g)
    gb = to_bits(g)
    if f == "f32":
        gv = oracle.decode("f32", gb)
        bad = gv != o
    else:
        bad = gb != oracle.round_to(f, o)
    n = int(bad.sum())
    assert n == 0, f"{what}: {n} of {bad.size} elements differ from the exact result; first at " \
                   f"{np.argwhere(bad)[0].tolist()}"


def check_f32(g: torch.Tensor, o: np.ndarray, tol: float = FRO_TOL_F32, what: str = ""):
    gv = oracle.decode("f32", to_bits(g))
    assert np.all(np.isfinite(gv)), f"{what}: non-finite output"
    err = rel_fro(gv, o)
    assert err <= tol, f"{what}: relative Frobenius error {err:.3e} > {tol:.0e}"
    return err


def f8_allowance(qa: np.ndarray, qb: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Per-element allowance for the fp8 matrix instruction's in-run
    truncation (see the module docstring): qa (m, K) and qb (K, n) are the
    decoded e4m3 values of the compared rows of A and columns of op(B),
    before the per-tensor scales, whose product is `scale`."""
    qa = np.asarray(qa, dtype=np.float64)
    qb = np.asarray(qb, dtype=np.float64)
    m, K = qa.shape
    n = qb.shape[1]
    kp = -(-K // F8_RUN) * F8_RUN
    if kp != K:    # the kernels zero-fill a K tail
        qa = np.concatenate([qa, np.zeros((m, kp - K))], axis=1)
        qb = np.concatenate([qb, np.zeros((kp - K, n))], axis=0)
    out = np.empty((m, n))
    qbr = qb.reshape(kp // F8_RUN, F8_RUN, n)
    step = max(1, (1 << 22) // kp)    # columns per pass: bounded temporaries
    for i in range(m):
        ar = qa[i].reshape(kp // F8_RUN, F8_RUN, 1)
        for c0 in range(0, n, step):
            p = ar * qbr[:, :, c0:c0 + step]                        # runs x 8 x cols
            ap = np.abs(p)
            mx = ap.max(axis=1, keepdims=True)
            e = np.floor(np.log2(np.where(mx > 0, mx, 1.0))).astype(np.int64)
            lost = (ap < np.ldexp(1.0, e - 6)) & (mx > 0)           # exponent below e - 6
            d = np.where(lost, np.minimum(ap, np.ldexp(1.0, e - F8_KEEP)), 0.0)
            mean = np.abs((np.sign(p) * d).sum(axis=(0, 1))) / 2.0
            band = LAMBDA_F8 * np.sqrt((d * d).sum(axis=(0, 1)) / 12.0)
            out[i, c0:c0 + step] = np.minimum(mean + band, d.sum(axis=(0, 1)))
    return out * abs(scale)


def check_blocks(gv: np.ndarray, o: np.ndarray, tol: float, what: str = ""):
    """Relative Frobenius error <= tol on every BLOCK x BLOCK tile of the
    last two axes (partial edge tiles included)."""
    o2 = o.reshape(-1, o.shape[-2], o.shape[-1]) if o.ndim >= 2 else o.reshape(1, 1, -1)
    g2 = gv.reshape(o2.shape)
    worst = 0.0
    for z in range(o2.shape[0]):
        for r in range(0, o2.shape[1], BLOCK):
            for c in range(0, o2.shape[2], BLOCK):
                ob = o2[z, r:r + BLOCK, c:c + BLOCK]
                err = rel_fro(g2[z, r:r + BLOCK, c:c + BLOCK], ob)
                worst = max(worst, err)
                assert err <= tol, f"{what}: block ({z}, {r}, {c}) relative Frobenius error " \
                                   f"{err:.3e} > {tol:.0e}"
    return worst


def _loose_ok(n_loose: int, size: int, what: str):
    print(f"[parity] {what}: {n_loose} of {size} elements within an allowance beyond 1 ulp")
    assert n_loose <= max(16, LOOSE_MAX * size), \
        f"{what}: {n_loose} of {size} elements only within the allowance (more than {LOOSE_MAX:.0%})"


def check_rounded(g: torch.Tensor, o: np.ndarray, T: np.ndarray, K: int, what: str = "",
                  fro_tol: float | None = None, extra: np.ndarray | float = 0.0):
    """1-ulp rule for bf16/fp16 outputs, with the cancellation allowance
    (plus `extra`, the fp8 truncation allowance per element).  An element may
    use the allowance only where it exceeds its own ulp (elsewhere the fp32
    error cannot move the rounded result by more than one ulp)."""
    f = fmt_of(g)
    gb = to_bits(g)
    gv = oracle.decode(f, gb)
    r = oracle.decode(f, oracle.round_to(f, o))
    u = ulp(f, r)
    ok = np.abs(gv - r) <= u
    bound = LAMBDA * math.sqrt(max(K, 1)) * 2.0 ** -24 * T + extra
    loose = ~ok & (bound > u) & (np.abs(gv - o) <= u + bound)
    bad = ~(ok | loose)
    n = int(bad.sum())
    if n:
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {n} of {bad.size} elements beyond 1 ulp; first {list(i)}: "
                             f"gpu {gv[i]!r} oracle {o[i]!r} rounded {r[i]!r} ulp {u[i]!r}")
    n_loose = int(loose.sum())
    _loose_ok(n_loose, loose.size, what)
    if fro_tol is not None:
        err = rel_fro(gv, r)
        assert err <= fro_tol, f"{what}: relative Frobenius error {err:.3e} > {fro_tol:.0e}"
        check_blocks(gv, r, fro_tol, what)
    return n_loose


def check_f8_f32(g: torch.Tensor, o: np.ndarray, T: np.ndarray, K: int, extra: np.ndarray,
                 what: str = ""):
    """fp32 output of fp8 inputs: elementwise |g - o| <= fp32 allowance + the
    fp8 truncation allowance, and the 1e-3 Frobenius figure on the whole
    result and on every 32x32 block."""
    gv = oracle.decode("f32", to_bits(g))
    assert np.all(np.isfinite(gv)), f"{what}: non-finite output"
    bound = LAMBDA * math.sqrt(max(K, 1)) * 2.0 ** -24 * T + extra
    bad = np.abs(gv - o) > bound
    n = int(bad.sum())
    if n:
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {n} of {bad.size} elements beyond the fp8 allowance; first "
                             f"{list(i)}: gpu {gv[i]!r} oracle {o[i]!r} allowance {bound[i]!r}")
    err = rel_fro(gv, o)
    assert err <= FRO_TOL_F8, f"{what}: relative Frobenius error {err:.3e} > {FRO_TOL_F8:.0e}"
    check_blocks(gv, o, FRO_TOL_F8, what)
    return err


def check(g: torch.Tensor, o: np.ndarray, T: np.ndarray | None, K: int, exact: bool = False,
          what: str = "", f8: bool = False, f8_ops=None):
    """f8_ops = (qa, qb, scale) for fp8 inputs: decoded e4m3 rows of A
    (m, K) and columns of op(B) (K, n) of the compared outputs and the
    product of the per-tensor scales (a batch axis, if any, leads)."""
    if exact:
        return check_exact(g, o, what)
    if f8:
        assert f8_ops is not None, f"{what}: fp8 check needs the decoded operands"
        qa, qb, sc = f8_ops
        if np.ndim(qa) == 3:
            extra = np.stack([f8_allowance(qa[z], qb[z], sc) for z in range(len(qa))])
        else:
            extra = f8_allowance(qa, qb, sc)
        extra = extra.reshape(o.shape)
        if fmt_of(g) == "f32":
            return check_f8_f32(g, o, T, K, extra, what=what)
        return check_rounded(g, o, T, K, what=what, fro_tol=FRO_TOL_F8, extra=extra)
    if fmt_of(g) == "f32":
        return check_f32(g, o, tol=FRO_TOL_F32, what=what)
    return check_rounded(g, o, T, K, what=what)


def f8_operands(A_bits: np.ndarray, B_bits: np.ndarray, trans_b: bool, scale: float):
    """(qa, qb, scale) for check(): decoded e4m3 A (m, K) and op(B) (K, n)."""
    qa = oracle.decode("e4m3", np.ascontiguousarray(A_bits)).reshape(A_bits.shape)
    qb = oracle.decode("e4m3", np.ascontiguousarray(B_bits)).reshape(B_bits.shape)
    if trans_b:
        qb = np.swapaxes(qb, -1, -2)
    return qa, qb, float(scale)
