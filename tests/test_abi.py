"""The C-ABI library loads, exports what include/tmm.h declares, and rejects bad
arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tmm.h")


@pytest.fixture(scope="module")
def tmm():
    import tiled_matrix_multiplication_amd as t
    return t


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tmm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["tmm_gemm", "tmm_gemm_strided_batched", "tmm_gemm_ex", "tmm_gemv", "tmm_attention_fwd",
         "tmm_conv2d_fused", "tmm_gemm_splitk", "tmm_gemm_splitk_noalloc", "tmm_status_string", "tmm_version",
         "tmm_set_override"])


def test_library_exports_every_declared_symbol(tmm):
    raw = ctypes.CDLL(tmm.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(tmm.EXPORTS) == set(declared_functions())


def declared_status_codes():
    """{value: name} of the status enum in include/tmm.h."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return {int(v): n for n, v in re.findall(r"\b(TMM_(?:OK|ERR_[A-Z]+))\s*=\s*(-?\d+)", text)}


def test_version_and_status_strings(tmm):
    assert tmm.tmm_version() == 10000
    codes = declared_status_codes()
    assert sorted(codes) == list(range(-10, 1))
    for code in codes:
        s = tmm.tmm_status_string(code)
        assert s and s != "unknown status code", code
    assert tmm.tmm_status_string(-99) == "unknown status code"


def test_binding_names_every_status_code(tmm):
    """The binding's STATUS map is the header's enum, name for name."""
    assert tmm.STATUS == declared_status_codes()


FAKE = ctypes.c_void_p(0x100000)     # never dereferenced: every call below fails validation
FAKE2 = ctypes.c_void_p(0x200000)
FAKE3 = ctypes.c_void_p(0x300000)


def gemm(tmm, M=64, N=64, K=64, ab=1, c=0, tb=0, A=FAKE, lda=None, B=FAKE2, ldb=None, C=FAKE3,
         ldc=None, bias=None, sa=1.0, sb=1.0):
    lda = K if lda is None else lda
    ldb = (K if tb else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return tmm.lib.tmm_gemm(M, N, K, ab, c, tb, A, lda, B, ldb, C, ldc, bias, sa, sb, None)


def batched(tmm, M=64, N=64, K=64, sA=4096, sB=4096, sC=4096, batch=2, **kw):
    return tmm.lib.tmm_gemm_strided_batched(M, N, K, kw.get("ab", 1), kw.get("c", 0), 0, FAKE, K, sA,
                                            FAKE2, N, sB, kw.get("C", FAKE3), N, sC, batch, None,
                                            1.0, 1.0, None)


def test_dimension_errors(tmm):
    assert gemm(tmm, M=-1) == -1
    assert gemm(tmm, N=-5) == -1
    assert gemm(tmm, K=-1, lda=1) == -1
    assert batched(tmm, batch=-1) == -1


def test_leading_dimension_errors(tmm):
    assert gemm(tmm, lda=63) == -2
    assert gemm(tmm, ldb=63) == -2
    assert gemm(tmm, tb=1, ldb=63) == -2          # NT: ldb >= K
    assert gemm(tmm, ldc=10) == -2
    assert gemm(tmm, K=0, lda=0) == -2            # ld must be at least 1


def test_type_errors(tmm):
    assert gemm(tmm, ab=7) == -4
    assert gemm(tmm, ab=0, c=1) == -4             # f32 -> bf16 not offered
    assert gemm(tmm, ab=1, c=2) == -4             # bf16 -> f16
    assert gemm(tmm, ab=2, c=1) == -4             # f16 -> bf16
    assert gemm(tmm, ab=3, c=2) == -4             # fp8 -> f16
    assert tmm.lib.tmm_gemv(8, 8, 3, 1, FAKE, 8, FAKE2, FAKE3, None, None) == -4   # no fp8 GEMV


def test_scale_errors(tmm):
    assert gemm(tmm, sa=2.0) == -5                # scales only for fp8
    assert gemm(tmm, ab=3, c=1, sa=float("nan")) == -5
    assert gemm(tmm, ab=3, c=1, sb=float("inf")) == -5


def test_null_and_alignment_errors(tmm):
    assert gemm(tmm, C=None) == -3
    assert gemm(tmm, A=None) == -3
    assert gemm(tmm, B=None) == -3
    assert gemm(tmm, A=ctypes.c_void_p(0x100001)) == -7     # bf16 at an odd address
    assert gemm(tmm, c=0, C=ctypes.c_void_p(0x300002)) == -7  # fp32 output at 2 mod 4
    assert gemm(tmm, bias=ctypes.c_void_p(0x400002)) == -7
    assert tmm.lib.tmm_gemv(8, 8, 1, 1, None, 8, FAKE2, FAKE3, None, None) == -3
    assert tmm.lib.tmm_gemv(8, 8, 1, 1, FAKE, 4, FAKE2, FAKE3, None, None) == -2


def test_batch_stride_errors(tmm):
    assert batched(tmm, sC=64 * 64 - 1) == -6     # C matrices would overlap
    assert batched(tmm, sA=-1) == -6
    # zero A/B strides (one operand for every problem) pass the stride check and
    # reach the NULL check behind it; no call here may pass validation
    assert batched(tmm, sC=64 * 64, sA=0, sB=0, C=None) == -3


def test_quick_returns_enqueue_nothing(tmm):
    # M == 0, N == 0, batch == 0: success without touching any pointer or the GPU
    assert gemm(tmm, M=0, A=None, B=None, C=None) == 0
    assert gemm(tmm, N=0, A=None, B=None, C=None, ldb=1, ldc=1) == 0
    assert batched(tmm, batch=0, C=None) == 0
    assert tmm.lib.tmm_gemv(0, 16, 1, 1, None, 16, None, None, None, None) == 0


def test_binding_rejects_host_tensors(tmm):
    import torch
    a = torch.zeros(4, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tmm.tmm_gemm(a, a, torch.zeros(4, 4))


def test_operand_span_limit(tmm):
    # 65536 x 32769 bf16 = 4 GiB + 128 KiB: rejected before any HIP call
    assert gemm(tmm, M=65536, N=64, K=32769) == -1


def attn(tmm, Z=2, Nq=64, Nk=64, D=128, it=2, ot=2, Q=FAKE, K=FAKE2, V=FAKE3, O=FAKE, ld=None,
         ldo=None, sq=None, so=None, scale=0.1):
    ld = D if ld is None else ld
    ldo = D if ldo is None else ldo
    sq = Nq * ld if sq is None else sq
    so = Nq * ldo if so is None else so
    return tmm.lib.tmm_attention_fwd(Z, Nq, Nk, D, it, ot, Q, ld, sq, K, ld, Nk * ld, V, ld, Nk * ld,
                                     O, ldo, so, scale, None)


def test_attention_validation(tmm):
    """Every bad argument is refused on the host with its code; the pointers
    are fake, so a call that passed validation would be a failure here too."""
    assert attn(tmm, D=96) == -1                      # D must be 64 or 128
    assert attn(tmm, Nq=-1) == -1
    assert attn(tmm, Nk=0) == -1                      # softmax over no keys
    assert attn(tmm, it=0, ot=0) == -4                # fp32 inputs are not accepted
    assert attn(tmm, it=3, ot=1) == -4                # nor fp8
    assert attn(tmm, it=2, ot=1) == -4                # f16 -> bf16 is not a pair
    assert attn(tmm, ld=64) == -2                     # ld below D
    assert attn(tmm, so=64 * 128 - 1) == -6           # O matrices overlap
    assert attn(tmm, scale=float("inf")) == -5
    assert attn(tmm, scale=3e38) == -5                # finite, but not once times log2(e)
    assert tmm.lib.tmm_attention_fwd(1, 64, 64, 128, 2, 2, FAKE, 128, 0, FAKE2, (1 << 24) + 8, 0,
                                     FAKE3, 128, 0, FAKE, 128, 0, 0.1, None) == -2
    assert attn(tmm, Q=None) == -3
    assert attn(tmm, ld=132, sq=64 * 132) == -7       # ld not a multiple of 8
    assert attn(tmm, Q=ctypes.c_void_p(0x100008)) == -7   # not 16-byte aligned


def test_attention_quick_returns(tmm):
    """batch == 0 or Nq == 0 enqueue nothing (NULL pointers are then fine)."""
    assert attn(tmm, Z=0, Q=None, K=None, V=None, O=None) == 0
    assert attn(tmm, Nq=0, Q=None, K=None, V=None, O=None) == 0


def gex(tmm, M=64, N=64, K=64, ab=1, c=1, ta=0, tb=0, A=FAKE, lda=None, B=FAKE2, ldb=None,
        C=FAKE3, ldc=None, batch=1, alpha=1.0, beta=0.0, act=0):
    lda = (M if ta else K) if lda is None else lda
    ldb = (K if tb else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return tmm.lib.tmm_gemm_ex(M, N, K, ab, c, ta, tb, A, lda, 0, B, ldb, 0, C, ldc, 0, batch, None,
                               alpha, beta, act, None)


def test_gemm_ex_validation(tmm):
    """The full form's own checks; the fake pointers would fault if a call
    got past validation."""
    assert gex(tmm, act=2) == -9                       # unknown activation
    assert gex(tmm, act=-1) == -9
    assert gex(tmm, ab=0, c=0, ta=1) == -4             # trans_a needs 16-bit inputs
    assert gex(tmm, ab=3, c=1, ta=1) == -4
    assert gex(tmm, alpha=float("inf")) == -5
    assert gex(tmm, beta=float("nan")) == -5
    assert gex(tmm, M=100, ta=1, lda=64) == -2         # A stored K x M needs lda >= M
    assert gex(tmm, ab=1, c=2) == -4                   # bf16 -> f16 is not a pair
    assert gex(tmm, A=None) == -3
    assert "activation" in tmm.lib.tmm_status_string(-9).decode()


def test_gemm_ex_quick_returns(tmm):
    assert gex(tmm, M=0, A=None, B=None, C=None) == 0
    assert gex(tmm, batch=0, A=None, B=None, C=None) == 0


def conv(tmm, N=2, H=8, W=8, C=16, K=8, R=3, S=3, pad=1, it=1, ot=1, x=FAKE, w=FAKE2, out=FAKE3,
         act=0, pool=1):
    return tmm.lib.tmm_conv2d_fused(N, H, W, C, K, R, S, pad, it, ot, x, w, None, None, act, pool,
                                    out, None)


def test_conv_validation(tmm):
    """Every call here fails a check before anything is launched."""
    assert conv(tmm, C=12) == -7                    # channels not a multiple of 8
    assert conv(tmm, pool=3) == -9
    assert conv(tmm, act=4) == -9
    assert conv(tmm, it=0, ot=0) == -4              # fp32 inputs are not accepted
    assert conv(tmm, it=1, ot=2) == -4
    assert conv(tmm, H=7, pool=2) == -1             # odd output cannot be pooled 2 x 2
    assert conv(tmm, R=11, pad=0) == -1             # filter larger than the padded image
    assert conv(tmm, H=0) == -1
    assert conv(tmm, x=None) == -3
    assert conv(tmm, x=ctypes.c_void_p(0x100008)) == -7   # input not 16-byte aligned


def splitk(tmm, M=256, N=512, K=1024, ab=2, c=2, tb=1, A=FAKE, lda=None, B=FAKE2, ldb=None, C=FAKE3,
           ldc=None, bias=None, splits=4, ws=ctypes.c_void_p(0x400000), ws_bytes=None):
    lda = K if lda is None else lda
    ldb = (K if tb else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    ws_bytes = splits * M * N * 4 if ws_bytes is None else ws_bytes
    return tmm.lib.tmm_gemm_splitk(M, N, K, ab, c, tb, A, lda, B, ldb, C, ldc, bias, 1.0, 1.0, splits,
                                   ws, ws_bytes, None)


def test_splitk_arguments_checked_on_host(tmm):
    """Split counts, the workspace and the usual GEMM checks, all before any
    HIP call (the fake pointers are never dereferenced)."""
    assert splitk(tmm, splits=0) == -9
    assert splitk(tmm, splits=65) == -9
    assert splitk(tmm, K=1000, splits=3) == -9               # 3 does not divide K
    assert splitk(tmm, ws=None) == -10
    assert splitk(tmm, ws_bytes=4 * 256 * 512 * 4 - 1) == -10
    assert splitk(tmm, ws=ctypes.c_void_p(0x400008)) == -10   # not 16-byte aligned
    assert splitk(tmm, lda=10) == -2
    assert splitk(tmm, ab=1, c=2) == -4
    assert splitk(tmm, A=None) == -3
    assert splitk(tmm, M=-1) == -1
    # quick returns: nothing to compute, nothing checked about the workspace
    assert splitk(tmm, M=0, ws=None) == 0
    assert splitk(tmm, N=0, ldc=1, ws=None) == 0


def test_splitk_noalloc_rejects_what_its_scratch_cannot_hold(tmm):
    """The allocation-free variant checks on the host, before touching its
    scratch: splits*M*N*4 above 32 MiB is TMM_ERR_WORKSPACE; the split checks
    and quick returns are those of tmm_gemm_splitk."""
    f = tmm.lib.tmm_gemm_splitk_noalloc
    # 4 x 1024 x 2049 fp32 partials: 32 MiB + 16 KiB
    assert f(1024, 2049, 4096, 2, 2, 1, FAKE, 4096, FAKE2, 4096, FAKE3, 2049, None, 1.0, 1.0, 4, None) == -10
    assert f(256, 512, 1024, 2, 2, 1, FAKE, 1024, FAKE2, 1024, FAKE3, 512, None, 1.0, 1.0, 0, None) == -9
    assert f(256, 512, 1000, 2, 2, 1, FAKE, 1000, FAKE2, 1000, FAKE3, 512, None, 1.0, 1.0, 3, None) == -9
    assert f(0, 512, 1024, 2, 2, 1, FAKE, 1024, FAKE2, 1024, FAKE3, 512, None, 1.0, 1.0, 4, None) == 0
    assert tmm.SPLITK_SCRATCH_BYTES == 32 << 20
    header = open(HEADER).read()
    assert re.search(r"#define TMM_SPLITK_SCRATCH_BYTES 33554432\b", header)


def test_conv_quick_return(tmm):
    assert conv(tmm, N=0, x=None, w=None, out=None) == 0


def test_override_accepts_the_documented_keys_and_rejects_others(tmm):
    """tmm_set_override parses on the host (no HIP call); a bad item leaves
    the setting as it was and returns TMM_ERR_ARG."""
    try:
        for spec in ["", "tile=128x128", "tile=skinny;skinny=32x64", "tile=gemvm", "gemv=2x16",
                     "tile=shortk skinny=16x16 gemv=1x4", "tile=generic", "tile=256x256r",
                     "conv=quad", "conv=direct;tile=256x256q", "ring=8", "tile=128x128q;ring=4"]:
            assert tmm.lib.tmm_set_override(spec.encode()) == 0, spec
        for spec in ["tile=99x99", "skinny=8x16", "gemv=3x4", "gemv=2,16", "foo=1", "tile", "tile=128x128;x",
                     "conv=fast", "ring=6", "ring="]:
            assert tmm.lib.tmm_set_override(spec.encode()) == -9, spec
        assert tmm.lib.tmm_set_override(None) == 0
    finally:
        tmm.tmm_set_override(None)


PROBES_HEADER = os.path.join(ROOT, "include", "tmm_probes.h")


def test_probe_library_exports_its_header():
    """libtmm_probes.so (measurement kernels) exports what include/tmm_probes.h declares."""
    import tiled_matrix_multiplication_amd.probes as probes
    text = re.sub(r"/\*.*?\*/", "", open(PROBES_HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(tmmp_[a-z0-9_]+)\s*\(", text)))
    assert declared == sorted(probes.EXPORTS)
    raw = ctypes.CDLL(probes.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name


def test_probe_arguments_checked_on_host():
    import tiled_matrix_multiplication_amd.probes as probes
    lib = probes.lib
    sink = ctypes.c_void_p(0x400000)
    assert lib.tmmp_stream_read(FAKE, 4, 1000, 16, sink, None) == -1       # row bytes not a multiple of 1 KiB
    assert lib.tmmp_stream_read(FAKE, 4, 3072, 16, sink, None) == -1       # not a power of two KiB
    assert lib.tmmp_stream_read(FAKE, 4, 8192, 3, sink, None) == -9        # waves per group
    assert lib.tmmp_stream_read(None, 4, 8192, 16, sink, None) == -3
    assert lib.tmmp_stream_read(ctypes.c_void_p(0x100004), 4, 8192, 16, sink, None) == -7
    assert lib.tmmp_stream_read(FAKE, 0, 8192, 16, sink, None) == 0       # nothing to read
    assert lib.tmmp_mfma_loop(FAKE, 1 << 20, 1, 256, 64, sink, None) == -1  # operands under 16 MiB
    assert lib.tmmp_mfma_loop(FAKE, 1 << 24, 4, 256, 64, sink, None) == -9  # shape
    assert lib.tmmp_mfma_loop(FAKE, 1 << 24, 2, 4, 65, sink, None) == -1    # fp8 shapes: iters % 4
    assert lib.tmmp_mfma_loop(None, 1 << 24, 1, 4, 64, sink, None) == -3
    assert lib.tmmp_mfma_loop(FAKE, 1 << 24, 1, 256, 64, sink, None) == -1  # 256 groups need 48 MiB
    assert lib.tmmp_mfma_loop(FAKE, 1 << 24, 1, 0, 64, sink, None) == 0
