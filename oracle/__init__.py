"""The oracle: TEST INFRASTRUCTURE ONLY.

A plain fp64 CPU statement of C = s_a*s_b * A . op(B) (+ bias) over the
exactly decoded low-precision inputs, of one attention head
o = softmax(scale * Q . K^T) . V, plus the format decoders and the
round-to-nearest-even encoders they need (all in ``oracle.c``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP
library (``tiled_matrix_multiplication_amd``) and never imports it.

Every function here is pinned by ``tests/test_oracle.py`` and
``tests/test_oracle_attention.py`` against facts that do not come from the
oracle itself (brute force, closed forms, the block decomposition identity of
the "GEMM to FlashAttention" page's tiling figure, independent library
conversions for the codecs, an independent softmax routine and the
invariances of softmax for the attention).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# The oracle's own format codes (oracle.c numbering).
F32, BF16, F16, E4M3 = 0, 1, 2, 3
_NAMES = {"f32": F32, "bf16": BF16, "f16": F16, "e4m3": E4M3}
_BITS = {F32: np.uint32, BF16: np.uint16, F16: np.uint16, E4M3: np.uint8}


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain C, -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    lib.oracle_decode.argtypes = [ctypes.c_int, vp, vp, i64]
    lib.oracle_round.argtypes = [ctypes.c_int, vp, vp, i64]
    lib.oracle_gemm.argtypes = [i64, i64, i64, ctypes.c_int, vp, i64, vp, i64,
                                ctypes.c_int, vp, dp, dp, vp, i64, vp]
    lib.oracle_gemm_ex.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, i64,
                                   vp, i64, dp, dp, vp, vp, ctypes.c_int, vp, i64, vp]
    lib.oracle_conv2d.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp,
                                  ctypes.c_int, ctypes.c_int, vp, vp]
    lib.oracle_threads.argtypes = []
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_attention.argtypes = [i64, i64, i64, ctypes.c_int, vp, i64, vp, i64, vp, i64,
                                     ctypes.c_double, vp, i64, vp]
    for f in (lib.oracle_decode, lib.oracle_round, lib.oracle_gemm, lib.oracle_threads, lib.oracle_set_threads,
              lib.oracle_attention, lib.oracle_gemm_ex, lib.oracle_conv2d):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _fmt(fmt) -> int:
    return _NAMES[fmt] if isinstance(fmt, str) else int(fmt)


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(fmt, bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of an array of format bit patterns."""
    f = _fmt(fmt)
    bits = np.ascontiguousarray(bits, dtype=_BITS[f])
    out = np.empty(bits.shape, dtype=np.float64)
    rc = _load().oracle_decode(f, _ptr(bits), _ptr(out), bits.size)
    if rc:
        raise ValueError(f"oracle_decode failed ({rc})")
    return out


def round_to(fmt, x: np.ndarray) -> np.ndarray:
    """Bit patterns of the bf16/fp16 values nearest to x (ties to even)."""
    f = _fmt(fmt)
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    rc = _load().oracle_round(f, _ptr(x), _ptr(out), x.size)
    if rc:
        raise ValueError(f"oracle_round failed ({rc})")
    return out


def gemm(fmt, A: np.ndarray, B: np.ndarray, trans_b: bool = False,
         bias: np.ndarray | None = None, scale_a: float = 1.0,
         scale_b: float = 1.0, want_abs: bool = False):
    """o = s_a*s_b * A . op(B) (+ bias) in float64.

    A: (M, K) bit patterns of ``fmt``; B: (K, N) bit patterns, or (N, K) when
    ``trans_b``.  Row strides of the given arrays are honoured as leading
    dimensions.  Returns o (M, N) float64, and with ``want_abs`` also
    T = sum_k |a_ik b'_kj| (same shape).
    """
    f = _fmt(fmt)
    A = np.asarray(A)
    B = np.asarray(B)
    if A.dtype != _BITS[f] or B.dtype != _BITS[f]:
        raise TypeError("A and B must hold the format's bit patterns")
    if A.ndim != 2 or B.ndim != 2:
        raise ValueError("A and B must be 2-D")
    A = _rowmajor(A)
    B = _rowmajor(B)
    M, K = A.shape
    if trans_b:
        N, K2 = B.shape
    else:
        K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    lda = A.strides[0] // A.itemsize if M > 1 else max(K, 1)
    ldb = B.strides[0] // B.itemsize if B.shape[0] > 1 else max(B.shape[1], 1)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias must have N entries")
    C = np.empty((M, N), dtype=np.float64)
    T = np.empty((M, N), dtype=np.float64) if want_abs else None
    rc = _load().oracle_gemm(M, N, K, f, _ptr(A), lda, _ptr(B), ldb, int(bool(trans_b)),
                             _ptr(bias), float(scale_a), float(scale_b), _ptr(C),
                             max(N, 1), _ptr(T))
    if rc:
        raise ValueError(f"oracle_gemm failed ({rc})")
    return (C, T) if want_abs else C


def gemm_ex(fmt, A: np.ndarray, B: np.ndarray, trans_a: bool = False, trans_b: bool = False,
            alpha: float = 1.0, beta: float = 0.0, C_in: np.ndarray | None = None,
            bias: np.ndarray | None = None, relu: bool = False, want_abs: bool = False):
    """o = act(alpha * op(A) . op(B) + bias + beta * C_in) in float64.

    A: (M, K) bit patterns, or (K, M) when ``trans_a``; B: (K, N), or (N, K)
    when ``trans_b``; C_in: (M, N) values (float64; ignored when None);
    act = max(0, .) when ``relu``.  Returns o, and with ``want_abs`` also
    T = |alpha| sum_k |a'_ik b'_kj| + |bias_j| + |beta c_ij|.
    """
    f = _fmt(fmt)
    A = _rowmajor(np.asarray(A))
    B = _rowmajor(np.asarray(B))
    if A.dtype != _BITS[f] or B.dtype != _BITS[f] or A.ndim != 2 or B.ndim != 2:
        raise TypeError("A and B must be 2-D arrays of the format's bit patterns")
    M, K = (A.shape[1], A.shape[0]) if trans_a else A.shape
    N, K2 = B.shape if trans_b else (B.shape[1], B.shape[0])
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    lda = A.strides[0] // A.itemsize if A.shape[0] > 1 else max(A.shape[1], 1)
    ldb = B.strides[0] // B.itemsize if B.shape[0] > 1 else max(B.shape[1], 1)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias must have N entries")
    cin = None
    if C_in is not None:
        cin = np.ascontiguousarray(C_in, dtype=np.float64)
        if cin.shape != (M, N):
            raise ValueError("C_in must be M x N")
    C = np.empty((M, N), dtype=np.float64)
    T = np.empty((M, N), dtype=np.float64) if want_abs else None
    rc = _load().oracle_gemm_ex(M, N, K, f, int(bool(trans_a)), int(bool(trans_b)), _ptr(A), lda,
                                _ptr(B), ldb, float(alpha), float(beta), _ptr(cin), _ptr(bias),
                                1 if relu else 0, _ptr(C), max(N, 1), _ptr(T))
    if rc:
        raise ValueError(f"oracle_gemm_ex failed ({rc})")
    return (C, T) if want_abs else C


def conv2d(fmt, x: np.ndarray, w: np.ndarray, pad: int, scale: np.ndarray | None = None,
           bias: np.ndarray | None = None, relu: bool = False, pool: int = 1,
           want_abs: bool = False):
    """Fused stride-1 convolution in float64: act(conv(x, w) * scale + bias),
    max-pooled over 2 x 2 blocks when ``pool`` == 2.

    x: (N, H, W, C) bit patterns (NHWC); w: (K, R, S, C); zero padding ``pad``.
    Returns (N, OH, OW, K) float64, with ``want_abs`` also the |.| companion
    (the largest over each pooling window).
    """
    f = _fmt(fmt)
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    if x.dtype != _BITS[f] or w.dtype != _BITS[f] or x.ndim != 4 or w.ndim != 4:
        raise TypeError("x and w must be 4-D arrays of the format's bit patterns")
    N, H, W, C = x.shape
    K, R, S, C2 = w.shape
    if C2 != C:
        raise ValueError("channel counts differ")
    P, Q = H + 2 * pad - R + 1, W + 2 * pad - S + 1
    if P < 1 or Q < 1 or (pool == 2 and (P % 2 or Q % 2)):
        raise ValueError("output size not positive (or not even for pooling)")
    sc = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    bi = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((N, P // pool, Q // pool, K), dtype=np.float64)
    T = np.empty_like(out) if want_abs else None
    rc = _load().oracle_conv2d(N, H, W, C, K, R, S, pad, f, _ptr(x), _ptr(w), _ptr(sc), _ptr(bi),
                               1 if relu else 0, int(pool), _ptr(out), _ptr(T))
    if rc:
        raise ValueError(f"oracle_conv2d failed ({rc})")
    return (out, T) if want_abs else out


def attention(fmt, Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
              want_abs: bool = False):
    """o = softmax(scale * Q . K^T) . V in float64, one head.

    Q: (Nq, D), K and V: (Nk, D) bit patterns of ``fmt`` (row strides are
    honoured).  Returns o (Nq, D) float64, and with ``want_abs`` also
    T[i][c] = sum_j w_ij |v_jc| (same shape).
    """
    f = _fmt(fmt)
    arrs = [_rowmajor(np.asarray(X)) for X in (Q, K, V)]
    if any(X.dtype != _BITS[f] or X.ndim != 2 for X in arrs):
        raise TypeError("Q, K and V must be 2-D arrays of the format's bit patterns")
    Q, K, V = arrs
    Nq, D = Q.shape
    Nk = K.shape[0]
    if K.shape[1] != D or V.shape != (Nk, D):
        raise ValueError(f"shapes differ: Q {Q.shape}, K {K.shape}, V {V.shape}")
    ld = [X.strides[0] // X.itemsize if X.shape[0] > 1 else D for X in (Q, K, V)]
    O = np.empty((Nq, D), dtype=np.float64)
    T = np.empty((Nq, D), dtype=np.float64) if want_abs else None
    rc = _load().oracle_attention(Nq, Nk, D, f, _ptr(Q), ld[0], _ptr(K), ld[1], _ptr(V), ld[2],
                                  float(scale), _ptr(O), D, _ptr(T))
    if rc:
        raise ValueError(f"oracle_attention failed ({rc})")
    return (O, T) if want_abs else O


def threads() -> int:
    """Threads the oracle's product runs on (OpenMP, from OMP_NUM_THREADS)."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> int:
    """Run the oracle's loops on n threads from now on; returns the count in force."""
    return int(_load().oracle_set_threads(int(n)))


def _rowmajor(X: np.ndarray) -> np.ndarray:
    """A view whose elements along a row are adjacent (copy otherwise)."""
    if X.shape[1] <= 1 or X.strides[1] == X.itemsize:
        if X.strides[0] >= 0 and X.strides[0] % X.itemsize == 0:
            return X
    return np.ascontiguousarray(X)
