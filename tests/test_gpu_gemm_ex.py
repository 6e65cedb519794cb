"""GPU parity of the full BLAS form, C = act(alpha op(A) op(B) + bias + beta
C) (tmm_gemm_ex), against the oracle's gemm_ex: all four operand layouts,
every kernel the form reaches (the ring and two-stage tiles, the skinny-M
kernel, the any-layout kernel for a transposed A, the K == 0 fill), fp8 and
fp32 inputs, batching, integer inputs held bit for bit, and beta = 0 not
reading C.  Tolerance as for the plain product, with T the oracle's
|alpha| sum |a b| + |bias| + |beta c|."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, TORCH_DT, on_gpu
from parity import check, f8_operands, to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


def make(shape, fmt, seed, dist="normal"):
    x = syn.small_ints(shape, seed) if dist == "int" else syn.normal(shape, seed)
    if fmt == "e4m3":
        s = syn.e4m3_scale(x)
        return syn.quantize_e4m3(x, s), float(s)
    return syn.to_bits(x, fmt), 1.0


def run_case(tmm, M, N, K, fmt, out, ta, tb, alpha, beta, relu, bias, seed, dist="normal", batch=1,
             what=""):
    shapeA = (K, M) if ta else (M, K)
    shapeB = (N, K) if tb else (K, N)
    As, Bs, sa, sb = [], [], 1.0, 1.0
    for z in range(batch):
        a, sa = make(shapeA, fmt, seed + 10 * z + 1, dist)
        b, sb = make(shapeB, fmt, seed + 10 * z + 2, dist)
        As.append(a)
        Bs.append(b)
    bvec = None
    if bias:
        bvec = (syn.small_ints((N,), seed + 3) if dist == "int" else syn.normal((N,), seed + 3, 0.1))
        bvec = bvec.astype(np.float32)
    cdist = syn.small_ints((batch, M, N), seed + 4) if dist == "int" else syn.normal((batch, M, N), seed + 4)
    C0 = syn.to_bits(cdist, out)
    dA = on_gpu(np.stack(As), fmt)
    dB = on_gpu(np.stack(Bs), fmt)
    dC = on_gpu(C0, out)
    dbias = torch.from_numpy(bvec).to(DEV) if bvec is not None else None
    a_eff = alpha * sa * sb
    tmm.tmm_gemm_ex(dA, dB, dC, bias=dbias, trans_a=ta, trans_b=tb, alpha=a_eff, beta=beta, relu=relu)
    torch.cuda.synchronize()
    for z in range(batch):
        cin = oracle.decode(out, C0[z])
        o, T = oracle.gemm_ex(fmt, As[z], Bs[z], ta, tb, a_eff, beta, cin if beta else None, bvec, relu,
                              want_abs=True)
        ops = None
        if fmt == "e4m3":
            qa, qb, _ = f8_operands(As[z], Bs[z], tb, 1.0)
            ops = (qa.T if ta else qa, qb, a_eff)
        check(dC[z], o, T, K, exact=(dist == "int"), what=f"{what} z {z}", f8=(fmt == "e4m3"), f8_ops=ops)


LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("fmt,out", [("bf16", "bf16"), ("f16", "f32")])
@pytest.mark.parametrize("M", [200, 300])
def test_layouts(tmm, ta, tb, fmt, out, M, force):
    force()
    relu = (M == 300)
    run_case(tmm, M, 150, 104, fmt, out, ta, tb, 0.5, -1.25, relu, True, seed=1000 + M,
             what=f"{'T' if ta else 'N'}{'T' if tb else 'N'} {fmt}->{out} M {M}")


TILES = ["256x256", "256x256r", "256x256s2", "256x256w4", "256x128", "128x128", "skinny", "generic",
         "256x256q", "256x128q", "128x128q"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("tb", [False, True], ids=["NN", "NT"])
def test_every_kernel(tmm, tile, tb, force):
    """The full-form epilogue of each kernel (the skinny kernel takes NT only;
    for NN the forced name falls back to the automatic choice)."""
    force(tile)
    run_case(tmm, 520, 776, 320, "bf16", "bf16", False, tb, 1.5, 0.75, True, True, seed=1100,
             what=f"tile {tile} {'NT' if tb else 'NN'}")


def test_integer_inputs_exact(tmm, force):
    """Small-integer inputs, alpha = 2, beta = -1, ReLU: every intermediate is
    an exact integer in fp32, so the output equals R(o) bit for bit -- in all
    four layouts."""
    force()
    for ta, tb in LAYOUTS:
        run_case(tmm, 130, 270, 96, "bf16", "f32", ta, tb, 2.0, -1.0, True, True, seed=1200,
                 dist="int", what=f"int {ta}{tb}")
        run_case(tmm, 300, 270, 64, "f16", "f16", ta, tb, 2.0, -1.0, True, True, seed=1210,
                 dist="int", what=f"int f16 {ta}{tb}")


@pytest.mark.parametrize("tile", ["256x256q", "256x128q", "128x128q"])
def test_four_wave_full_form_integer_exact(tmm, tile, force):
    """The four-wave kernel's full-form epilogue, bit for bit on small
    integers (K a multiple of 64, at least 128), both B layouts."""
    force(tile)
    for tb in (False, True):
        run_case(tmm, 300, 272, 128, "bf16", "f32", False, tb, 2.0, -1.0, True, True, seed=1250, dist="int",
                 what=f"int {tile} {'NT' if tb else 'NN'}")
        run_case(tmm, 264, 520, 192, "f16", "f16", False, tb, -1.0, 0.5, True, False, seed=1260, dist="int",
                 what=f"int f16 {tile} {'NT' if tb else 'NN'}")


def test_fp8_and_fp32(tmm, force):
    force()
    run_case(tmm, 512, 512, 512, "e4m3", "bf16", False, False, 0.5, 1.0, True, True, seed=1300,
             what="fp8 NN")
    run_case(tmm, 384, 640, 200, "e4m3", "f32", False, True, 1.0, -0.5, False, True, seed=1310,
             what="fp8 NT K tail")
    run_case(tmm, 130, 70, 50, "f32", "f32", False, True, -1.0, 2.0, True, True, seed=1320, what="fp32")


def test_batched_transposed_a(tmm, force):
    force()
    run_case(tmm, 96, 80, 72, "f16", "f16", True, False, 0.25, 0.5, False, True, seed=1400, batch=3,
             what="batched TN")


def test_one_row(tmm, force):
    """M = 1 with the full form does not take the plain GEMV kernel."""
    force()
    run_case(tmm, 1, 4096, 4096, "bf16", "bf16", False, True, 1.0, 1.0, True, True, seed=1500, what="M=1")


def test_beta_zero_does_not_read_c_and_empty_sum(tmm, force):
    force()
    M, N, K = 70, 90, 40
    A = syn.to_bits(syn.normal((M, K), 1601), "bf16")
    B = syn.to_bits(syn.normal((N, K), 1602), "bf16")
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    tmm.tmm_gemm_ex(on_gpu(A, "bf16"), on_gpu(B, "bf16"), C, trans_b=True, alpha=1.0, beta=0.0, relu=True)
    torch.cuda.synchronize()
    assert not torch.isnan(C.float()).any(), "beta = 0 read the old C"
    o, T = oracle.gemm_ex("bf16", A, B, trans_b=True, relu=True, want_abs=True)
    check(C, o, T, K, what="beta 0 over NaN")
    # K == 0: C = relu(bias + beta * old C)
    c0 = syn.to_bits(syn.normal((M, N), 1603), "f32")
    C = on_gpu(c0, "f32")
    bvec = syn.normal((N,), 1604).astype(np.float32)
    empty_a = torch.empty((M, 0), dtype=torch.bfloat16, device=DEV)
    empty_b = torch.empty((N, 0), dtype=torch.bfloat16, device=DEV)
    tmm.tmm_gemm_ex(empty_a, empty_b, C, bias=torch.from_numpy(bvec).to(DEV), trans_b=True,
                    beta=-2.0, relu=True)
    torch.cuda.synchronize()
    want = np.maximum(bvec.astype(np.float64)[None, :] - 2.0 * oracle.decode("f32", c0), 0.0)
    got = oracle.decode("f32", to_bits(C))
    np.testing.assert_allclose(got, want, rtol=2 ** -22, atol=0)


# Transposed A on the 256x256 ring kernel: M and N ragged against the tile
# (multiples of 8, as its 16-byte chunks need), both B layouts, both
# epilogues (plain and full form), batched; a K that is not a multiple of 32
# falls back to the any-layout kernel under the same forced name.
RING_TA = [
    # (M, N, K, fmt, out, tb, alpha, beta, relu, bias, batch)
    (520, 776, 320, "bf16", "bf16", False, 1.5, 0.75, True, True, 1),
    (264, 392, 96, "f16", "f32", False, 1.0, 0.0, False, False, 1),
    (520, 776, 320, "bf16", "f32", True, 1.0, 0.0, False, True, 1),
    (296, 136, 64, "f16", "f16", True, -0.5, 1.0, True, False, 1),
    (300, 136, 64, "f16", "f16", True, -0.5, 1.0, True, False, 1),
    (136, 264, 128, "bf16", "bf16", False, 1.0, 0.0, False, True, 3),
    (200, 152, 104, "bf16", "bf16", False, 1.0, 0.5, False, True, 1),
]


@pytest.mark.parametrize("case", RING_TA, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}-{c[4]}-{'T' if c[5] else 'N'}"
                                               f"-b{c[10]}" for c in RING_TA])
def test_transposed_a_ring(tmm, case, force):
    M, N, K, fmt, out, tb, alpha, beta, relu, bias, batch = case
    force("256x256r")
    run_case(tmm, M, N, K, fmt, out, True, tb, alpha, beta, relu, bias, seed=1700 + M, batch=batch,
             what=f"ring TA {case}")


def test_transposed_a_ring_integer_exact(tmm, force):
    force("256x256r")
    for tb in (False, True):
        run_case(tmm, 264, 520, 96, "bf16", "f32", True, tb, 2.0, -1.0, True, True, seed=1800,
                 dist="int", what=f"int ring TA tb {tb}")


def test_transposed_a_automatic_choice(tmm, force):
    """A weight-gradient shape large enough that the ring kernel is chosen
    without forcing (2048 x 2048 outputs: 64 tiles of 256 x 256)."""
    force()
    run_case(tmm, 2048, 2048, 128, "bf16", "f32", True, False, 1.0, 0.0, False, False, seed=1900,
             what="auto TA 2048")
