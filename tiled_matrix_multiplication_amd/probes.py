"""Binding of the measurement kernels (libtmm_probes.so, include/tmm_probes.h):
argument marshalling only, for bench.py and the tests."""
from __future__ import annotations

import ctypes
import os

import torch

from . import TmmError

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtmm_probes.so")
EXPORTS = ("tmmp_stream_read", "tmmp_mfma_loop")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python tiled_matrix_multiplication_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.tmmp_stream_read.argtypes = [vp, i64, i64, ci, vp, vp]
    lib.tmmp_mfma_loop.argtypes = [vp, i64, ci, i64, i64, vp, vp]
    lib.tmmp_stream_read.restype = ci
    lib.tmmp_mfma_loop.restype = ci
    return lib


lib = _load()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def stream_read(src: torch.Tensor, rows: int, row_bytes: int, waves_per_group: int, sink: torch.Tensor) -> None:
    """Read rows x row_bytes bytes of `src` with the GEMV's access pattern."""
    rc = lib.tmmp_stream_read(src.data_ptr(), rows, row_bytes, waves_per_group, sink.data_ptr(), _stream())
    if rc:
        raise TmmError("tmmp_stream_read", rc)


def mfma_loop(operands: torch.Tensor, shape: int, groups: int, iters: int, sink: torch.Tensor) -> None:
    """groups x 8 waves x iters rounds of 1 Mi flop of bf16 matrix instructions."""
    rc = lib.tmmp_mfma_loop(operands.data_ptr(), operands.numel() * operands.element_size(), shape, groups, iters,
                            sink.data_ptr(), _stream())
    if rc:
        raise TmmError("tmmp_mfma_loop", rc)
