"""GPU parity of the fused implicit-GEMM convolution (tmm_conv2d_fused)
against the oracle's direct convolution: the conv_fused listing's problem
(Lecture 27 notes section 3.1: batch 8, 64 x 64, 32 -> 64 channels, 3 x 3,
one-pixel zero halo, scale 1 + 0.01 f, bias 0.5, ReLU, 2 x 2 max pool,
inputs uniform in [-0.5, 0.5)), and shapes that exercise every edge:
channel counts that split a 32-wide step across taps, filter counts that
are not a multiple of the 64-filter tile, pixel counts that end mid-tile,
wide filters and padding, no pooling or activation, both output widths,
integer inputs held bit for bit.  Tolerance: the plain product's, with
K = R S C and T the oracle's |.| companion (the largest in each window)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, TORCH_DT, on_gpu
from parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


def run(tmm, N, H, W, C, K, R, S, pad, fmt, out, relu, pool, seed, dist="uniform", scale=True,
        bias=True):
    if dist == "int":
        x = syn.small_ints((N, H, W, C), seed + 1)
        w = syn.small_ints((K, R, S, C), seed + 2, -2, 2)
    else:
        x = syn.uniform((N, H, W, C), seed + 1)
        w = syn.uniform((K, R, S, C), seed + 2)
    xb, wb = syn.to_bits(x, fmt), syn.to_bits(w, fmt)
    sc = (1.0 + 0.01 * np.arange(K)).astype(np.float32) if scale else None
    bi = np.full(K, 0.5, dtype=np.float32) if bias else None
    if dist == "int":
        sc = np.full(K, 2.0, dtype=np.float32) if scale else None
        bi = (np.arange(K) % 5 - 2).astype(np.float32) if bias else None
    P, Q = H + 2 * pad - R + 1, W + 2 * pad - S + 1
    dout = torch.full((N, P // pool, Q // pool, K), float("nan"), dtype=TORCH_DT[out], device=DEV)
    tmm.tmm_conv2d_fused(on_gpu(xb, fmt), on_gpu(wb, fmt), dout, pad,
                         scale=None if sc is None else torch.from_numpy(sc).to(DEV),
                         bias=None if bi is None else torch.from_numpy(bi).to(DEV), relu=relu, pool=pool)
    torch.cuda.synchronize()
    o, T = oracle.conv2d(fmt, xb, wb, pad, sc, bi, relu, pool, want_abs=True)
    what = f"conv {N}x{H}x{W}x{C} -> {K} {R}x{S} pad {pad} {fmt}->{out} relu {relu} pool {pool}"
    check(dout.reshape(-1, K), o.reshape(-1, K), T.reshape(-1, K), R * S * C, exact=(dist == "int"),
          what=what)


def test_listing_problem(tmm, force):
    """The conv_fused listing's problem, bf16 inputs, fp32 output as there,
    through the automatic choice (the LDS-staged kernel) and the
    register-direct kernel."""
    run(tmm, 8, 64, 64, 32, 64, 3, 3, 1, "bf16", "f32", True, 2, seed=2000)
    force(conv="direct")
    run(tmm, 8, 64, 64, 32, 64, 3, 3, 1, "bf16", "f32", True, 2, seed=2000)


# (N, H, W, C, K, R, S, pad, in, out, relu, pool)
CASES = [
    (8, 64, 64, 32, 64, 3, 3, 1, "f16", "f16", True, 2),
    (2, 17, 13, 8, 100, 3, 3, 1, "bf16", "bf16", False, 1),
    (3, 10, 12, 40, 70, 3, 3, 1, "f16", "f32", True, 2),
    (1, 9, 9, 16, 64, 5, 3, 2, "bf16", "f32", True, 1),
    (2, 14, 14, 64, 128, 1, 1, 0, "f16", "f16", False, 2),
    (1, 6, 6, 24, 16, 3, 3, 0, "bf16", "bf16", True, 2),
    (4, 7, 5, 8, 5, 3, 3, 1, "f16", "f16", True, 1),
]


def _id(c):
    N, H, W, C, K, R, S, pad, f, o, relu, pool = c
    return f"{N}x{H}x{W}x{C}-{K}-{R}x{S}p{pad}-{f}-{o}{'-relu' if relu else ''}-pool{pool}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_shapes(tmm, case):
    N, H, W, C, K, R, S, pad, fmt, out, relu, pool = case
    run(tmm, N, H, W, C, K, R, S, pad, fmt, out, relu, pool, seed=2100 + 10 * CASES.index(case))


def test_integer_inputs_exact(tmm):
    """Small-integer inputs, scale 2, integer bias: exact in fp32, so the
    output is the oracle's rounding bit for bit, pooled and not."""
    run(tmm, 2, 12, 10, 16, 72, 3, 3, 1, "bf16", "f32", True, 2, seed=2200, dist="int")
    run(tmm, 2, 12, 10, 24, 40, 3, 3, 1, "f16", "f16", False, 1, seed=2210, dist="int")


def test_without_scale_and_bias(tmm):
    run(tmm, 2, 8, 8, 16, 32, 3, 3, 1, "bf16", "f32", False, 1, seed=2300, scale=False, bias=False)


# Channel counts that are multiples of 32, for the LDS-staged kernel (128
# pixels x 128 filters per workgroup, one tap per 32-channel K-step):
# pixels and filters that end mid-tile, two filter tiles, R != S with wide
# padding, an odd step count (padded with a zero step), the fewest steps it
# takes (1 x 1, C = 96: three, padded to four), no padding.
QUAD_CASES = [
    (8, 64, 64, 32, 64, 3, 3, 1, "bf16", "f32", True, 2),
    (2, 17, 13, 32, 100, 3, 3, 1, "bf16", "bf16", False, 1),
    (3, 10, 12, 64, 130, 3, 3, 1, "f16", "f32", True, 2),
    (1, 9, 9, 32, 64, 5, 3, 2, "bf16", "f32", True, 1),
    (2, 14, 14, 96, 128, 1, 1, 0, "f16", "f16", False, 2),
    (1, 6, 6, 32, 16, 3, 3, 0, "bf16", "bf16", True, 2),
    (2, 11, 7, 160, 200, 3, 3, 1, "f16", "f16", True, 1),
]


@pytest.mark.parametrize("case", QUAD_CASES, ids=[_id(c) for c in QUAD_CASES])
def test_lds_staged_kernel(tmm, force, case):
    N, H, W, C, K, R, S, pad, fmt, out, relu, pool = case
    force(conv="quad")
    run(tmm, N, H, W, C, K, R, S, pad, fmt, out, relu, pool, seed=2500 + 10 * QUAD_CASES.index(case))


def test_lds_staged_kernel_integer_exact(tmm, force):
    """Bit-exact on small integers through the LDS-staged kernel, pooled and
    not, with the zero taps of the halo and a padded step."""
    force(conv="quad")
    run(tmm, 2, 12, 10, 32, 72, 3, 3, 1, "bf16", "f32", True, 2, seed=2600, dist="int")
    run(tmm, 2, 12, 10, 32, 40, 5, 3, 2, "f16", "f16", False, 1, seed=2610, dist="int")


def test_lds_staged_kernel_is_chosen_for_full_grids(tmm):
    """16 x 64 x 64 pixels, C = 32: 512 workgroups of 128 x 128, enough for
    the automatic choice to be the LDS-staged kernel (no override)."""
    run(tmm, 16, 64, 64, 32, 128, 3, 3, 1, "bf16", "bf16", True, 2, seed=2700)


@pytest.mark.parametrize("case", [
    (17, 31, 31, 8, 520, 3, 3, 1, "bf16", "bf16", True, 1),   # pixels end mid-tile, K not a multiple of 64
    (16, 32, 32, 16, 512, 3, 3, 1, "f16", "f32", True, 2),    # pooled windows
], ids=["17x31x31x8-520-ragged", "16x32x32x16-512-pool2"])
def test_large_grids_take_wide_waves(tmm, case):
    """Problems with at least two 256-pixel workgroups per CU run 64 pixels
    per wave (the other tests' grids are smaller and run 32)."""
    N, H, W, C, K, R, S, pad, fmt, out, relu, pool = case
    run(tmm, N, H, W, C, K, R, S, pad, fmt, out, relu, pool, seed=2400)
