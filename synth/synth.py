"""Seeded synthetic inputs (Python side of the input generator).

This module draws inputs only.  It contains none of the quantized sweep's
arithmetic: the CPU oracle (``oracle/``) and the GPU library
(``self_speculative_verify_amd``) both consume what it produces, and neither
imports the other.

The generator is Philox4x32-10 (Salmon et al., "Parallel random numbers: as
easy as 1, 2, 3", SC'11), counter-based, so any row of any matrix can be
regenerated on its own.  A normal variate is the Irwin-Hall sum of twelve
uniforms (mean 0, variance 1, support +-6); see ``philox_gen.c`` for the
exact bit-level definition shared with the device generator.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth.so")
GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

# Stream tags inside one seed.
STREAM_W = 0
STREAM_MASK = 1
STREAM_X = 2

_host = None
_gpu = None


def host_lib() -> ctypes.CDLL:
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_philox4x32_10.restype = None
        lib.synth_std_normal_f64.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64,
                                             ctypes.c_int64, ctypes.c_void_p]
        lib.synth_std_normal_f64.restype = None
        lib.synth_outlier_mask.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64,
                                           ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
        lib.synth_outlier_mask.restype = None
        lib.synth_weights_f32.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_double, ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_uint32, ctypes.c_double,
                                          ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
        lib.synth_weights_f32.restype = ctypes.c_int
        _host = lib
    return _host


def gpu_lib() -> ctypes.CDLL:
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB):
            raise RuntimeError(f"{GPU_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_LIB)
        lib.synth_weights_f32_gpu.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_double, ctypes.c_uint32,
                                              ctypes.c_uint32, ctypes.c_uint32, ctypes.c_double,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_weights_f32_gpu.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def default_threads() -> int:
    n = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return max(1, min(n, 16))


def philox_block(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    host_lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def std_normal(seed: int, stream: int, first: int, count: int) -> np.ndarray:
    """Standard-normal (Irwin-Hall-12) variates number first..first+count-1."""
    out = np.empty(count, dtype=np.float64)
    if count:
        host_lib().synth_std_normal_f64(seed, stream, first, count, out.ctypes.data)
    return out


def outlier_mask(seed: int, first: int, count: int, thresh: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint8)
    if count:
        host_lib().synth_outlier_mask(seed, STREAM_MASK, first, count, thresh, out.ctypes.data)
    return out


def weights(seed: int, K: int, row0: int, nrows: int, sigma: float,
            outlier_thresh: int = 0, outlier_mult: float = 20.0,
            nthreads: int | None = None) -> np.ndarray:
    """Rows [row0, row0+nrows) of the fp32 weight matrix drawn from ``seed``."""
    out = np.empty((nrows, K), dtype=np.float32)
    if nrows and K:
        rc = host_lib().synth_weights_f32(seed, K, row0, nrows, sigma, STREAM_W, STREAM_MASK,
                                          outlier_thresh, outlier_mult, out.ctypes.data, K,
                                          nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("synth_weights_f32 failed")
    return out


def weights_gpu(seed: int, K: int, row0: int, nrows: int, sigma: float, out_ptr: int,
                ldo: int, stream_ptr: int = 0, outlier_thresh: int = 0,
                outlier_mult: float = 20.0) -> None:
    """Same rows as :func:`weights`, generated on the device into ``out_ptr``."""
    rc = gpu_lib().synth_weights_f32_gpu(seed, K, row0, nrows, sigma, STREAM_W, STREAM_MASK,
                                         outlier_thresh, outlier_mult, out_ptr, ldo, stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synth_weights_f32_gpu failed ({rc})")


def x_fp16(seed: int, M: int, K: int) -> np.ndarray:
    """Activation panel X[M][K]: standard normals rounded (RNE) to fp16."""
    z = std_normal(seed, STREAM_X, 0, M * K).reshape(M, K)
    return z.astype(np.float16)
