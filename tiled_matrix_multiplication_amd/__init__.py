"""Python binding of libtmm.so (tiled GEMM / GEMV for MI355X, gfx950).

Argument marshalling only: each function takes torch tensors that already
live on the GPU, reads their shapes, strides, element types and data
pointers, and calls the C entry point of the same name (see
``include/tmm.h``) on the current torch stream (or the given one).  All
arithmetic happens in the library's HIP kernels.  There is no fallback: if
``libtmm.so`` is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtmm.so")

TMM_F32, TMM_BF16, TMM_F16, TMM_F8E4M3 = 0, 1, 2, 3

STATUS = {
    0: "TMM_OK", -1: "TMM_ERR_DIM", -2: "TMM_ERR_LD", -3: "TMM_ERR_NULL", -4: "TMM_ERR_DTYPE",
    -5: "TMM_ERR_SCALE", -6: "TMM_ERR_STRIDE", -7: "TMM_ERR_ALIGN", -8: "TMM_ERR_LAUNCH",
    -9: "TMM_ERR_ARG", -10: "TMM_ERR_WORKSPACE",
}

EXPORTS = ("tmm_gemm", "tmm_gemm_strided_batched", "tmm_gemm_ex", "tmm_gemv", "tmm_attention_fwd",
           "tmm_conv2d_fused", "tmm_gemm_splitk", "tmm_gemm_splitk_noalloc",
           "tmm_status_string", "tmm_version", "tmm_set_override")

_DTYPE = {torch.float32: TMM_F32, torch.bfloat16: TMM_BF16, torch.float16: TMM_F16,
          torch.float8_e4m3fn: TMM_F8E4M3}


class TmmError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn}: {STATUS.get(code, code)} ({tmm_status_string(code)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python tiled_matrix_multiplication_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, ci, cf = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.tmm_gemm.argtypes = [i64, i64, i64, ci, ci, ci, vp, i64, vp, i64, vp, i64, vp, cf, cf, vp]
    lib.tmm_gemm_strided_batched.argtypes = [i64, i64, i64, ci, ci, ci, vp, i64, i64, vp, i64, i64,
                                             vp, i64, i64, i64, vp, cf, cf, vp]
    lib.tmm_gemv.argtypes = [i64, i64, ci, ci, vp, i64, vp, vp, vp, vp]
    lib.tmm_conv2d_fused.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, ci, ci, vp, vp, vp, vp,
                                     ci, ci, vp, vp]
    lib.tmm_gemm_ex.argtypes = [i64, i64, i64, ci, ci, ci, ci, vp, i64, i64, vp, i64, i64, vp, i64,
                                i64, i64, vp, cf, cf, ci, vp]
    lib.tmm_attention_fwd.argtypes = [i64, i64, i64, i64, ci, ci, vp, i64, i64, vp, i64, i64,
                                      vp, i64, i64, vp, i64, i64, cf, vp]
    lib.tmm_gemm_splitk.argtypes = [i64, i64, i64, ci, ci, ci, vp, i64, vp, i64, vp, i64, vp, cf, cf, ci,
                                    vp, i64, vp]
    lib.tmm_gemm_splitk_noalloc.argtypes = [i64, i64, i64, ci, ci, ci, vp, i64, vp, i64, vp, i64, vp, cf, cf,
                                            ci, vp]
    lib.tmm_status_string.argtypes = [ci]
    lib.tmm_status_string.restype = ctypes.c_char_p
    lib.tmm_version.argtypes = []
    lib.tmm_set_override.argtypes = [ctypes.c_char_p]
    for f in (lib.tmm_gemm, lib.tmm_gemm_strided_batched, lib.tmm_gemm_ex, lib.tmm_gemv,
              lib.tmm_attention_fwd, lib.tmm_conv2d_fused, lib.tmm_gemm_splitk, lib.tmm_gemm_splitk_noalloc,
              lib.tmm_version, lib.tmm_set_override):
        f.restype = ci
    return lib


lib = _load()


def tmm_status_string(code: int) -> str:
    return lib.tmm_status_string(int(code)).decode()


def tmm_set_override(spec: str | None = None) -> None:
    """Pin kernel choices for measurements and tests (keys in include/tmm.h:
    tile=..., skinny=<bm>x<bn>, gemv=<r>x<w>); None or "" restores the
    automatic choice."""
    rc = lib.tmm_set_override(spec.encode() if spec else None)
    if rc:
        raise TmmError("tmm_set_override", rc)


def tmm_version() -> int:
    return int(lib.tmm_version())


# ---------------------------------------------------------------- marshalling


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported element type {t.dtype}") from None


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _ld(t: torch.Tensor) -> int:
    """Leading dimension of a row-major 2-D view (rows contiguous)."""
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous (stride 1)")
    return max(int(t.stride(-2)) if t.shape[-2] > 1 else int(t.shape[-1]), 1)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(fn: str, rc: int):
    if rc != 0:
        raise TmmError(fn, rc)


def tmm_gemm(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, bias: torch.Tensor | None = None,
             trans_b: bool = False, scale_a: float = 1.0, scale_b: float = 1.0, stream=None):
    """C = scale_a*scale_b * A . op(B) (+ bias).  A (M,K); B (K,N) or (N,K) with trans_b; C (M,N)."""
    _on_gpu(A, B, C, bias)
    M, K = A.shape
    N = B.shape[0] if trans_b else B.shape[1]
    if (B.shape[1] if trans_b else B.shape[0]) != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same element type")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (N,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous float32 vector of N entries")
    rc = lib.tmm_gemm(M, N, K, _dtype(A), _dtype(C), int(bool(trans_b)), _ptr(A), _ld(A), _ptr(B),
                      _ld(B), _ptr(C), _ld(C), _ptr(bias), float(scale_a), float(scale_b),
                      ctypes.c_void_p(_stream(stream)))
    _check("tmm_gemm", rc)
    return C


def splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    """Workspace tmm_gemm_splitk needs: splits fp32 planes of M x N."""
    return int(splits) * int(M) * int(N) * 4


def tmm_gemm_splitk(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, bias: torch.Tensor | None = None,
                    trans_b: bool = False, splits: int = 4, workspace: torch.Tensor | None = None,
                    scale_a: float = 1.0, scale_b: float = 1.0, stream=None):
    """C = scale_a*scale_b * A . op(B) (+ bias) with K cut into ``splits`` slices
    whose fp32 partials go to ``workspace`` (a GPU tensor of at least
    splitk_workspace_bytes(M, N, splits) bytes), then summed in order."""
    _on_gpu(A, B, C, bias, workspace)
    M, K = A.shape
    N = B.shape[0] if trans_b else B.shape[1]
    if (B.shape[1] if trans_b else B.shape[0]) != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same element type")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (N,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous float32 vector of N entries")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.tmm_gemm_splitk(M, N, K, _dtype(A), _dtype(C), int(bool(trans_b)), _ptr(A), _ld(A), _ptr(B),
                             _ld(B), _ptr(C), _ld(C), _ptr(bias), float(scale_a), float(scale_b), int(splits),
                             _ptr(workspace), ws_bytes, ctypes.c_void_p(_stream(stream)))
    _check("tmm_gemm_splitk", rc)
    return C


SPLITK_SCRATCH_BYTES = 32 << 20   # TMM_SPLITK_SCRATCH_BYTES


def tmm_gemm_splitk_noalloc(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                            bias: torch.Tensor | None = None, trans_b: bool = False, splits: int = 4,
                            scale_a: float = 1.0, scale_b: float = 1.0, stream=None):
    """tmm_gemm_splitk with the library's per-GPU scratch in place of a
    workspace (no allocation; calls that overlap on one GPU race)."""
    _on_gpu(A, B, C, bias)
    M, K = A.shape
    N = B.shape[0] if trans_b else B.shape[1]
    if (B.shape[1] if trans_b else B.shape[0]) != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same element type")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (N,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous float32 vector of N entries")
    rc = lib.tmm_gemm_splitk_noalloc(M, N, K, _dtype(A), _dtype(C), int(bool(trans_b)), _ptr(A), _ld(A),
                                     _ptr(B), _ld(B), _ptr(C), _ld(C), _ptr(bias), float(scale_a),
                                     float(scale_b), int(splits), ctypes.c_void_p(_stream(stream)))
    _check("tmm_gemm_splitk_noalloc", rc)
    return C


def tmm_gemm_strided_batched(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                             bias: torch.Tensor | None = None, trans_b: bool = False,
                             scale_a: float = 1.0, scale_b: float = 1.0, stream=None):
    """C[z] = scale_a*scale_b * A[z] . op(B[z]) (+ bias) for 3-D tensors (batch, rows, cols)."""
    _on_gpu(A, B, C, bias)
    Z, M, K = A.shape
    N = B.shape[1] if trans_b else B.shape[2]
    if B.shape[0] != Z or C.shape[0] != Z or tuple(C.shape[1:]) != (M, N) or \
            (B.shape[2] if trans_b else B.shape[1]) != K:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same element type")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (N,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous float32 vector of N entries")
    rc = lib.tmm_gemm_strided_batched(
        M, N, K, _dtype(A), _dtype(C), int(bool(trans_b)), _ptr(A), _ld(A), int(A.stride(0)),
        _ptr(B), _ld(B), int(B.stride(0)), _ptr(C), _ld(C), int(C.stride(0)), Z, _ptr(bias),
        float(scale_a), float(scale_b), ctypes.c_void_p(_stream(stream)))
    _check("tmm_gemm_strided_batched", rc)
    return C


def tmm_gemm_ex(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, bias: torch.Tensor | None = None,
                trans_a: bool = False, trans_b: bool = False, alpha: float = 1.0, beta: float = 0.0,
                relu: bool = False, stream=None):
    """C = act(alpha * op(A) . op(B) + bias + beta * C), act = ReLU when ``relu``.

    2-D tensors, or 3-D (batch, rows, cols) for a batch of problems.  A is
    (M, K), or (K, M) with ``trans_a``; B is (K, N), or (N, K) with ``trans_b``.
    """
    _on_gpu(A, B, C, bias)
    if A.dim() == 2:
        A, B, C = A.unsqueeze(0), B.unsqueeze(0), C.unsqueeze(0)
    Z = A.shape[0]
    M, K = (A.shape[2], A.shape[1]) if trans_a else (A.shape[1], A.shape[2])
    N, K2 = (B.shape[1], B.shape[2]) if trans_b else (B.shape[2], B.shape[1])
    if K2 != K or B.shape[0] != Z or tuple(C.shape) != (Z, M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same element type")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (N,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous float32 vector of N entries")
    rc = lib.tmm_gemm_ex(
        M, N, K, _dtype(A), _dtype(C), int(bool(trans_a)), int(bool(trans_b)), _ptr(A), _ld(A),
        int(A.stride(0)), _ptr(B), _ld(B), int(B.stride(0)), _ptr(C), _ld(C), int(C.stride(0)), Z,
        _ptr(bias), float(alpha), float(beta), 1 if relu else 0, ctypes.c_void_p(_stream(stream)))
    _check("tmm_gemm_ex", rc)
    return C


def tmm_gemv(W: torch.Tensor, x: torch.Tensor, y: torch.Tensor, bias: torch.Tensor | None = None,
             stream=None):
    """y = W . x (+ bias).  W (N, K) row-major, x (K,), y (N,)."""
    _on_gpu(W, x, y, bias)
    N, K = W.shape
    if tuple(x.shape) != (K,) or tuple(y.shape) != (N,):
        raise ValueError(f"shape mismatch: W {tuple(W.shape)}, x {tuple(x.shape)}, y {tuple(y.shape)}")
    if x.dtype != W.dtype:
        raise TypeError("W and x must have the same element type")
    if (K > 1 and x.stride(0) != 1) or (N > 1 and y.stride(0) != 1):
        raise ValueError("x and y must be contiguous")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (N,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous float32 vector of N entries")
    rc = lib.tmm_gemv(N, K, _dtype(W), _dtype(y), _ptr(W), _ld(W), _ptr(x), _ptr(y), _ptr(bias),
                      ctypes.c_void_p(_stream(stream)))
    _check("tmm_gemv", rc)
    return y


def tmm_attention_fwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, O: torch.Tensor,
                      scale: float | None = None, stream=None):
    """O[z] = softmax(scale * Q[z] . K[z]^T) . V[z] for 3-D tensors (batch, rows, D);
    scale defaults to 1/sqrt(D)."""
    _on_gpu(Q, K, V, O)
    Z, Nq, D = Q.shape
    Nk = K.shape[1]
    if tuple(K.shape) != (Z, Nk, D) or tuple(V.shape) != (Z, Nk, D) or tuple(O.shape) != (Z, Nq, D):
        raise ValueError(f"shape mismatch: Q {tuple(Q.shape)}, K {tuple(K.shape)}, "
                         f"V {tuple(V.shape)}, O {tuple(O.shape)}")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must have the same element type")
    if scale is None:
        scale = float(D) ** -0.5
    rc = lib.tmm_attention_fwd(Z, Nq, Nk, D, _dtype(Q), _dtype(O), _ptr(Q), _ld(Q), int(Q.stride(0)),
                               _ptr(K), _ld(K), int(K.stride(0)), _ptr(V), _ld(V), int(V.stride(0)),
                               _ptr(O), _ld(O), int(O.stride(0)), float(scale),
                               ctypes.c_void_p(_stream(stream)))
    _check("tmm_attention_fwd", rc)
    return O


def tmm_conv2d_fused(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor, pad: int,
                     scale: torch.Tensor | None = None, bias: torch.Tensor | None = None,
                     relu: bool = False, pool: int = 1, stream=None):
    """out = pool(act(conv(x, w) * scale + bias)), stride 1, NHWC.

    x (N, H, W, C), w (K, R, S, C), out (N, OH, OW, K), all contiguous;
    scale / bias float32 (K,) or None; pool 1 or 2 (2 x 2 max)."""
    _on_gpu(x, w, out, scale, bias)
    for t in (x, w, out):
        if not t.is_contiguous():
            raise ValueError("x, w and out must be contiguous")
    N, H, W, C = x.shape
    K, R, S, C2 = w.shape
    if C2 != C or w.dtype != x.dtype:
        raise ValueError("x and w disagree in channels or element type")
    P, Q = H + 2 * pad - R + 1, W + 2 * pad - S + 1
    if tuple(out.shape) != (N, P // pool, Q // pool, K):
        raise ValueError(f"out must be {(N, P // pool, Q // pool, K)}, got {tuple(out.shape)}")
    for v in (scale, bias):
        if v is not None and (v.dtype != torch.float32 or v.shape != (K,) or v.stride(0) != 1):
            raise ValueError("scale and bias must be contiguous float32 vectors of K entries")
    rc = lib.tmm_conv2d_fused(N, H, W, C, K, R, S, pad, _dtype(x), _dtype(out), _ptr(x), _ptr(w),
                              _ptr(scale), _ptr(bias), 1 if relu else 0, int(pool), _ptr(out),
                              ctypes.c_void_p(_stream(stream)))
    _check("tmm_conv2d_fused", rc)
    return out
