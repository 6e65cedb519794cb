"""GPU parity: the HIP path (through the C ABI) against the oracle, element by
element, at sizes the oracle finishes in seconds, spanning several tiles and
ragged tails, plus the degenerate cases and the identities of the method."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_cases import DEV, TORCH_DT, gemm_case, on_gpu
from parity import check, to_bits

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


# (M, N, K, in, out, trans_b, dist, bias, pad)
CASES = [
    # fp32, 256^3 and its exact variants
    (256, 256, 256, "f32", "f32", False, "normal", False, 0),
    (256, 256, 256, "f32", "f32", True, "normal", False, 0),
    (8, 8, 8, "f32", "f32", False, "int", False, 0),
    (256, 256, 256, "f32", "f32", False, "int", True, 0),
    (200, 130, 70, "f32", "f32", True, "normal", True, 0),
    # bf16: several tiles, ragged M/N/K, padded leading dimensions (16-byte path with a K tail)
    (512, 512, 512, "bf16", "f32", False, "normal", False, 0),
    (520, 776, 328, "bf16", "f32", False, "normal", False, 0),
    (520, 776, 328, "bf16", "bf16", True, "normal", True, 0),
    (300, 520, 333, "bf16", "bf16", True, "normal", True, 3),
    (300, 520, 333, "bf16", "f32", False, "normal", False, 3),
    (257, 383, 200, "bf16", "f32", False, "int", False, 0),
    (512, 768, 512, "bf16", "bf16", True, "int", True, 0),
    (600, 1000, 1000, "bf16", "bf16", False, "int", True, 0),
    # fp16
    (512, 384, 256, "f16", "f16", False, "normal", False, 0),
    (512, 384, 256, "f16", "f32", True, "normal", True, 0),
    (333, 250, 190, "f16", "f16", True, "int", True, 0),
    # fp8 e4m3 with per-tensor scales
    (512, 512, 512, "e4m3", "bf16", False, "normal", False, 0),
    (512, 512, 512, "e4m3", "f32", True, "normal", False, 0),
    (384, 640, 384, "e4m3", "bf16", True, "normal", True, 0),
    (300, 200, 500, "e4m3", "bf16", False, "int", True, 4),
    (256, 256, 640, "e4m3", "f32", True, "int", False, 0),
    # shapes that select each tile size
    (1024, 1024, 256, "bf16", "f32", False, "normal", False, 0),
    (2048, 256, 128, "f16", "f16", True, "normal", False, 0),
    (4, 300, 64, "bf16", "f32", True, "normal", False, 0),
    (1, 64, 64, "bf16", "f32", False, "normal", False, 0),
]


def _id(c):
    M, N, K, f, o, tb, d, b, pad = c
    return f"{f}-{o}-{'NT' if tb else 'NN'}-{M}x{N}x{K}-{d}{'-bias' if b else ''}{f'-pad{pad}' if pad else ''}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_gemm_parity(tmm, case):
    M, N, K, fmt, out, tb, dist, bias, pad = case
    dC, o, T, ops = gemm_case(tmm, M, N, K, fmt, out, tb, dist, bias, seed=10 * CASES.index(case), pad=pad,
                              want_ops=True)
    check(dC, o, T, K, exact=(dist == "int"), what=_id(case), f8=(fmt == "e4m3"), f8_ops=ops)


RAGGED = [(1000, 3000, 777), (4097, 511, 1023)]


@pytest.mark.parametrize("trans_b", [False, True], ids=["NN", "NT"])
@pytest.mark.parametrize("shape", RAGGED, ids=["1000x3000x777", "4097x511x1023"])
def test_ragged_bf16_full(tmm, shape, trans_b):
    """The ragged bf16 workloads, every output checked (rows not 16-byte aligned)."""
    M, N, K = shape
    dC, o, T = gemm_case(tmm, M, N, K, "bf16", "bf16", trans_b, "normal", False, seed=50)
    check(dC, o, T, K, what=f"ragged {shape}")
    dC32, o32, _ = gemm_case(tmm, M, N, K, "bf16", "f32", trans_b, "normal", False, seed=50)
    check(dC32, o32, None, K, what=f"ragged {shape} f32")


def test_closed_form(tmm):
    """a_ik = i + k, b_kj = k - j  =>  C_ij = -K i j + (i - j) K(K-1)/2 + (K-1)K(2K-1)/6 (exact in fp32)."""
    M, N, K = 96, 80, 200
    i = np.arange(M)[:, None]
    k = np.arange(K)
    j = np.arange(N)[None, :]
    A = torch.tensor((i + k[None, :]), dtype=torch.float32, device=DEV)
    B = torch.tensor((k[:, None] - j), dtype=torch.float32, device=DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm(A, B, C)
    want = -K * i * j + (i - j) * (K * (K - 1) // 2) + (K - 1) * K * (2 * K - 1) // 6
    assert torch.equal(C.cpu(), torch.tensor(want, dtype=torch.float32))


def test_transpose_identity_bitwise(tmm):
    """NT with B stored transposed equals NN with B, bit for bit."""
    M, N, K = 384, 320, 256
    A = on_gpu(syn.to_bits(syn.normal((M, K), 11), "bf16"), "bf16")
    B = on_gpu(syn.to_bits(syn.normal((K, N), 12), "bf16"), "bf16")
    Bt = B.t().contiguous()
    c_nn = torch.empty((M, N), dtype=torch.float32, device=DEV)
    c_nt = torch.empty((M, N), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm(A, B, c_nn)
    tmm.tmm_gemm(A, Bt, c_nt, trans_b=True)
    assert torch.equal(c_nn, c_nt)


@pytest.mark.parametrize("trans_b", [False, True], ids=["NN", "NT"])
def test_batched_parity_and_batch_identity(tmm, trans_b):
    Z, M, N, K = 3, 300, 200, 136
    A = syn.to_bits(syn.normal((Z, M, K), 21), "f16")
    B = syn.to_bits(syn.normal((Z, N, K) if trans_b else (Z, K, N), 22), "f16")
    bias = syn.normal((N,), 23, 0.02)
    dA, dB = on_gpu(A, "f16"), on_gpu(B, "f16")
    dbias = torch.from_numpy(bias).to(DEV)
    C = torch.empty((Z, M, N), dtype=torch.float16, device=DEV)
    tmm.tmm_gemm_strided_batched(dA, dB, C, bias=dbias, trans_b=trans_b)
    for z in range(Z):
        o, T = oracle.gemm("f16", A[z], B[z], trans_b=trans_b, bias=bias, want_abs=True)
        check(C[z], o, T, K, what=f"batch {z}")
        one = torch.empty((M, N), dtype=torch.float16, device=DEV)
        tmm.tmm_gemm(dA[z], dB[z], one, bias=dbias, trans_b=trans_b)
        assert torch.equal(one, C[z]), f"batch slice {z} differs from the single call"


def _batched_nt(Z, M, N, K, fmt, seed):
    A = syn.to_bits(syn.normal((Z, M, K), seed), fmt)
    B = syn.to_bits(syn.normal((Z, N, K), seed + 1), fmt)
    return A, B


def _run_batched_nt(tmm, A, B, fmt, tile, force):
    if tile is None:
        force()
    else:
        force(tile)
    Z, M, K = A.shape
    N = B.shape[1]
    C = torch.full((Z, M, N), float("nan"), dtype=TORCH_DT[fmt], device=DEV)
    tmm.tmm_gemm_strided_batched(on_gpu(A, fmt), on_gpu(B, fmt), C, trans_b=True)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("Z,M,N,K,fmt", [
    (3, 512, 256, 128, "f16"),    # 6 tiles, 8 workgroups (two idle)
    (2, 256, 768, 64, "bf16"),    # K = 64: 128-byte operand rows
    (9, 512, 512, 64, "f16"),     # 36 tiles on 32 workgroups: four walk two
    (5, 768, 512, 128, "bf16"),   # 30 tiles on 24 workgroups, across batch entries
], ids=["f16-K128-6tiles", "bf16-K64", "f16-K64-walk", "bf16-K128-walk"])
def test_short_k_kernel(tmm, force, Z, M, N, K, fmt):
    """The persistent short-K kernel (forced): every batch entry against the
    oracle, and bit for bit against the two-stage kernel (same matrix
    instructions in the same K order)."""
    A, B = _batched_nt(Z, M, N, K, fmt, 61 + K)
    C = _run_batched_nt(tmm, A, B, fmt, "shortk", force)
    for z in range(Z):
        o, T = oracle.gemm(fmt, A[z], B[z], trans_b=True, want_abs=True)
        check(C[z], o, T, K, what=f"short-K batch {z}")
    ref = _run_batched_nt(tmm, A, B, fmt, "256x256s2", force)
    assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), "short-K and two-stage kernels differ"


def test_short_k_pitched_output(tmm, force):
    """The short-K kernel writing into a view of a wider and taller buffer
    (row pitch N + 64, batch stride past the view's rows): bit for bit the
    two-stage kernel's result, and nothing outside the view is written."""
    Z, M, N, K = 3, 512, 512, 128
    A, B = _batched_nt(Z, M, N, K, "f16", 91)
    force("shortk")
    big = torch.full((Z, M + 16, N + 64), float("nan"), dtype=torch.float16, device=DEV)
    view = big[:, 8:8 + M, 32:32 + N]
    tmm.tmm_gemm_strided_batched(on_gpu(A, "f16"), on_gpu(B, "f16"), view, trans_b=True)
    torch.cuda.synchronize()
    ref = _run_batched_nt(tmm, A, B, "f16", "256x256s2", force)
    assert torch.equal(view.contiguous().view(torch.int16), ref.view(torch.int16)), "pitched short-K output differs"
    outside = torch.ones(big.shape, dtype=torch.bool, device=DEV)
    outside[:, 8:8 + M, 32:32 + N] = False
    assert bool(torch.isnan(big[outside]).all()), "short-K kernel wrote outside its output view"


def test_attention_scores_shape_takes_short_k(tmm, force):
    """Short K over many whole tiles (64 problems x 16 tiles, K = 128) is what
    the dispatch sends to the short-K kernel without forcing: the result
    equals the two-stage kernel's bit for bit, and sampled problems match the
    oracle."""
    Z, M, N, K = 64, 1024, 1024, 128
    A, B = _batched_nt(Z, M, N, K, "f16", 81)
    C = _run_batched_nt(tmm, A, B, "f16", None, force)
    for z in (0, 37, 63):
        o, T = oracle.gemm("f16", A[z], B[z], trans_b=True, want_abs=True)
        check(C[z], o, T, K, what=f"scores batch {z}")
    ref = _run_batched_nt(tmm, A, B, "f16", "256x256s2", force)
    assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), "short-K and two-stage kernels differ"


def test_batched_broadcast_operand(tmm):
    """Stride 0 for B: one B for every problem."""
    Z, M, N, K = 4, 128, 192, 64
    A = syn.to_bits(syn.small_ints((Z, M, K), 31), "bf16")
    B = syn.to_bits(syn.small_ints((K, N), 32), "bf16")
    dA = on_gpu(A, "bf16")
    dB = on_gpu(B, "bf16").unsqueeze(0).expand(Z, K, N)
    C = torch.empty((Z, M, N), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm_strided_batched(dA, dB, C)
    for z in range(Z):
        check(C[z], oracle.gemm("bf16", A[z], B), None, K, exact=True, what=f"broadcast {z}")


def test_empty_sum_gives_bias(tmm):
    M, N = 37, 50
    bias = syn.normal((N,), 41)
    A = torch.empty((M, 0), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((0, N), dtype=torch.bfloat16, device=DEV)
    for out in (torch.float32, torch.bfloat16):
        C = torch.full((M, N), float("nan"), dtype=out, device=DEV)
        tmm.tmm_gemm(A, B, C, bias=torch.from_numpy(bias).to(DEV))
        check(C, np.broadcast_to(bias.astype(np.float64), (M, N)), None, 0, exact=True, what="K=0")
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm(A, B, C)
    assert torch.count_nonzero(C).item() == 0


def test_empty_output_calls_succeed(tmm):
    A = torch.ones((0, 16), dtype=torch.bfloat16, device=DEV)
    B = torch.ones((16, 8), dtype=torch.bfloat16, device=DEV)
    C = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm(A, B, C)
    sentinel = torch.full((4, 4), 7.0, device=DEV)
    tmm.tmm_gemm_strided_batched(torch.ones((0, 4, 16), dtype=torch.bfloat16, device=DEV),
                                 torch.ones((0, 16, 4), dtype=torch.bfloat16, device=DEV),
                                 sentinel.view(1, 4, 4)[:0])
    assert torch.all(sentinel == 7.0)


# ---------------------------------------------------------------- attention weights . V


def test_subnormal_weights_are_kept(tmm):
    """fp16 weights that are all subnormal (2^-20) times V = 1: O = K * 2^-20 exactly."""
    Z, N, K, D = 2, 256, 2048, 128
    P = torch.full((Z, N, K), 2.0 ** -20, dtype=torch.float16, device=DEV)
    V = torch.ones((Z, K, D), dtype=torch.float16, device=DEV)
    for out in (torch.float16, torch.float32):
        O = torch.empty((Z, N, D), dtype=out, device=DEV)
        tmm.tmm_gemm_strided_batched(P, V, O)
        assert torch.all(O.float() == K * 2.0 ** -20), f"subnormal weights flushed ({out})"


def test_uniform_weights_give_column_means(tmm):
    """P = 2^-11 (exact in fp16), K = 2048: O = column means of integer V, exactly."""
    Z, N, K, D = 2, 128, 2048, 128
    V = syn.small_ints((Z, K, D), 51)
    P = torch.full((Z, N, K), 2.0 ** -11, dtype=torch.float16, device=DEV)
    O = torch.empty((Z, N, D), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm_strided_batched(P, torch.from_numpy(V).to(torch.float16).to(DEV), O)
    want = V.astype(np.float64).sum(axis=1) / 2048.0
    for z in range(Z):
        assert np.array_equal(O[z].cpu().numpy().astype(np.float64), np.broadcast_to(want[z], (N, D)))


def test_softmax_weights_stay_in_value_hull(tmm):
    """Rows of P are nonnegative and sum to 1, so each output lies between the column min and max of V."""
    Z, N, D = 2, 512, 128
    P = syn.softmax_rows_f16(Z, N, 61)
    V = syn.to_bits(syn.normal((Z, N, D), 62), "f16")
    O = torch.empty((Z, N, D), dtype=torch.float32, device=DEV)
    tmm.tmm_gemm_strided_batched(on_gpu(P, "f16"), on_gpu(V, "f16"), O)
    for z in range(Z):
        v = oracle.decode("f16", V[z])
        o, _ = oracle.gemm("f16", P[z], V[z], want_abs=True)
        check(O[z], o, None, N, what=f"P.V {z}")
        g = O[z].cpu().numpy()
        slack = 1e-3
        assert np.all(g >= v.min(axis=0) - slack) and np.all(g <= v.max(axis=0) + slack)


# ---------------------------------------------------------------- GEMV


@pytest.mark.parametrize("N,K,fmt,out,dist,bias", [
    (4096, 4096, "bf16", "bf16", "normal", True),
    (4096, 4096, "bf16", "f32", "normal", True),
    (1000, 4096, "bf16", "bf16", "int", True),
    (96, 8192, "bf16", "bf16", "normal", True),       # two unchecked passes per row
    (777, 777, "bf16", "f32", "normal", False),       # element path (rows not 16-byte aligned)
    (513, 1032, "f16", "f16", "normal", True),
    (300, 2048, "f32", "f32", "normal", True),
    (1, 8, "bf16", "f32", "int", False),
])
def test_gemv_parity(tmm, N, K, fmt, out, dist, bias):
    gen = syn.small_ints if dist == "int" else syn.normal
    W = syn.to_bits(gen((N, K), 71) if dist == "int" else syn.normal((N, K), 71, 0.02), fmt)
    x = syn.to_bits(gen((1, K), 72), fmt)
    b = (syn.small_ints((N,), 73) if dist == "int" else syn.normal((N,), 73, 0.02)) if bias else None
    o, T = oracle.gemm(fmt, x, W, trans_b=True, bias=b, want_abs=True)
    y = torch.full((N,), float("nan"), dtype=TORCH_DT[out], device=DEV)
    tmm.tmm_gemv(on_gpu(W, fmt), on_gpu(x, fmt).view(K), y,
                 bias=torch.from_numpy(b).to(DEV) if b is not None else None)
    check(y.view(1, N), o, T, K, exact=(dist == "int"), what=f"gemv {N}x{K}")
    # the same product through tmm_gemm with M = 1 (dispatched to the GEMV kernel)
    y2 = torch.full((1, N), float("nan"), dtype=TORCH_DT[out], device=DEV)
    tmm.tmm_gemm(on_gpu(x, fmt), on_gpu(W, fmt), y2, trans_b=True,
                 bias=torch.from_numpy(b).to(DEV) if b is not None else None)
    assert torch.equal(y2.view(N), y)


def test_graph_replay_matches_eager(tmm):
    """GEMV and GEMM launches captured in a HIP graph (as the GEMV is timed)
    give the eager result on every replay, with eager work and
    synchronisations between the replays and new inputs written in place."""
    N, K = 1024, 768
    M = 300
    W = on_gpu(syn.to_bits(syn.normal((N, K), 81, 0.02), "bf16"), "bf16")
    A = on_gpu(syn.to_bits(syn.normal((M, K), 82), "bf16"), "bf16")
    x = torch.empty(K, dtype=torch.bfloat16, device=DEV)
    bias = torch.from_numpy(syn.normal((N,), 83, 0.02)).to(DEV)
    y = torch.empty(N, dtype=torch.bfloat16, device=DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    x.copy_(on_gpu(syn.to_bits(syn.normal((1, K), 84), "bf16"), "bf16").view(K))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tmm.tmm_gemv(W, x, y, bias=bias)
        tmm.tmm_gemm(A, W, C, bias=bias, trans_b=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tmm.tmm_gemv(W, x, y, bias=bias)
        tmm.tmm_gemm(A, W, C, bias=bias, trans_b=True)
    for r in range(4):
        x.copy_(on_gpu(syn.to_bits(syn.normal((1, K), 90 + r), "bf16"), "bf16").view(K))
        A.mul_(-1.0)
        y.fill_(float("nan"))
        C.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        y_ref = torch.empty_like(y)
        C_ref = torch.empty_like(C)
        tmm.tmm_gemv(W, x, y_ref, bias=bias)
        tmm.tmm_gemm(A, W, C_ref, bias=bias, trans_b=True)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"GEMV replay {r} differs from the eager call"
        assert torch.equal(C, C_ref), f"GEMM replay {r} differs from the eager call"
