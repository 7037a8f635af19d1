"""CPU oracle of the quantized weight sweep -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  It wraps ``liboracle.so`` (plain C built with gcc,
no SIMD intrinsics, no BLAS, no fast-math; see ``qg_oracle.c``), which shares
no source with the GPU library.

What it computes (the quantizer is the "Weights" item of the engine-internals
list on the Quasar/q27 wiki: symmetric groupwise codes with fp16 scales,
dequantized inside the weight-streaming product; group 32 and 4/5 bits):

* ``quantize``: per row n and group g of 32 consecutive k,
  ``s = fp16_RNE(double(max|w|) / Qmax)`` and
  ``q = clamp(RNE(double(w) / double(s)), -Qmax, Qmax)`` (q = 0 when s = 0).
* ``pack`` / ``unpack``: the tiled group-32 layout, written and read bit by bit.
* Format variants (a format code in place of ``bits``): ``Q4_G64`` (4-bit
  symmetric with one scale per 64 weights, the Quasar/q27 wiki's Q4_G64 byte
  accounting) and ``Q4_ZP`` (4-bit group-32 asymmetric with an integer zero
  point per group, the INT4 W4A16 weights of the qwen38 model notes):
  ``s = fp16_RNE((max(0, max w) - min(0, min w)) / 15)``,
  ``z = clamp(RNE(-min(0, min w) / s), 0, 15)``,
  ``u = clamp(RNE(w / s) + z, 0, 15)`` and ``w_hat = (u - z) * s``.  For
  ``Q4_ZP`` the quantizer and ``unpack`` return ``(u, scales, zeros)``.
* ``sweep``: ``Y[m, n] = sum_k X[m, k] * (q[n, k] * s[n, k//32])`` in fp64,
  ascending k, decoded from the packed bytes.
* ``compare``: the acceptance test -- relative L2 over a job's Y at most 1e-4
  and, per row m, ``max_n |Y - Yref| <= 1e-3 * ||X[m, :]||_2 * max(s)``.
* ``verify_head``: the greedy verify step after a sweep of an lm_head-class
  matrix.  Greedy speculative decoding leaves greedy output unchanged (Quasar/q27
  wiki, opening notes: greedy spec decode by default, greedy bitwise
  unchanged), so with a slot's panel rows r0 .. r0 + d (the states after the
  context and after each of its d drafted tokens), draft i + 1 stands only if
  it equals the argmax of row r0 + i; the accepted count is the longest such
  prefix, and the round's next token is the argmax of the first row that
  disagrees.  ``argmax_rows`` takes the lowest column among equal maxima.
* ``attn_verify``: the attention half of a verify round, per slot and layer:
  the W verify positions of a slot (the last W of its L cached positions)
  attend causally over the slot's keys and values, 6 query heads per KV head,
  4 KV heads, head dim 256 (the full-attention layers as the Quasar/q27 wiki
  sizes their KV bytes; GQA 6 in its fp8-KV note), all in fp64.
  ``e4m3_to_f64`` / ``f64_to_e4m3`` are the OCP E4M3 byte format of an fp8
  KV cache: a plain decode, and the saturating scale-free conversion the
  wiki's KV-cache item describes (nearest code, ties to even, clamp at 448).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

Q4, Q5, Q4_G64, Q4_ZP = 4, 5, 0x104, 0x204
FORMATS = (Q4, Q5, Q4_G64, Q4_ZP)

REL_L2_TOL = 1e-4
MAX_ABS_COEF = 1e-3

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f64_to_f16_array.argtypes = [vp, i64, vp]
        L.oracle_f64_to_f16_array.restype = None
        L.oracle_f16_to_f64_array.argtypes = [vp, i64, vp]
        L.oracle_f16_to_f64_array.restype = None
        L.oracle_packed_bytes.argtypes = [ci, i64, i64]
        L.oracle_packed_bytes.restype = i64
        L.oracle_quantize.argtypes = [vp, i64, i64, i64, ci, vp, vp, vp]
        L.oracle_quantize.restype = ci
        L.oracle_pack.argtypes = [vp, vp, vp, i64, i64, ci, vp]
        L.oracle_pack.restype = ci
        L.oracle_unpack.argtypes = [vp, i64, i64, ci, vp, vp, vp]
        L.oracle_unpack.restype = ci
        L.oracle_dequant.argtypes = [vp, i64, i64, ci, i64, i64, vp]
        L.oracle_dequant.restype = ci
        L.oracle_sweep_f64.argtypes = [vp, i64, i64, ci, vp, i64, ci, vp, i64, vp, i64, ci]
        L.oracle_sweep_f64.restype = ci
        _lib = L
    return _lib


def cpu_share() -> int:
    """Host cores this process may use: the CPUs it may run on, capped by its
    cgroup's CPU quota when one is set (a container can see every core of the
    machine but be entitled to fewer)."""
    try:
        c = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        c = os.cpu_count() or 1
    for path in ("/sys/fs/cgroup/cpu.max", "/sys/fs/cgroup/cpu/cpu.cfs_quota_us"):
        try:
            with open(path) as fh:
                parts = fh.read().split()
        except OSError:
            continue
        if path.endswith("cpu.max"):
            if parts and parts[0] != "max":
                c = min(c, max(1, -(-int(parts[0]) // int(parts[1]))))
        else:
            quota = int(parts[0]) if parts else -1
            if quota > 0:
                with open("/sys/fs/cgroup/cpu/cpu.cfs_period_us") as fh:
                    c = min(c, max(1, -(-quota // int(fh.read().split()[0]))))
        break
    return max(1, c)


def _threads(n):
    return int(n) if n else cpu_share()


class NonFiniteError(ValueError):
    pass


def f64_to_f16_bits(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64)).ravel()
    out = np.empty(a.size, dtype=np.uint16)
    lib().oracle_f64_to_f16_array(a.ctypes.data, a.size, out.ctypes.data)
    return out.reshape(np.shape(x))


def f16_bits_to_f64(h) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(h, dtype=np.uint16)).ravel()
    out = np.empty(a.size, dtype=np.float64)
    lib().oracle_f16_to_f64_array(a.ctypes.data, a.size, out.ctypes.data)
    return out.reshape(np.shape(h))


def group_size(fmt: int) -> int:
    return 64 if fmt == Q4_G64 else 32


def packed_bytes(fmt: int, N: int, K: int) -> int:
    return int(lib().oracle_packed_bytes(fmt, N, K))


def quantize(W: np.ndarray, fmt: int):
    """Codes q (int8, [N, K]) and scale bits (uint16, [N, K/group]); for
    ``Q4_ZP`` the codes are u (0..15) and the zero points (uint8, [N, K/32])
    come third."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    G = K // group_size(fmt)
    codes = np.empty((N, K), dtype=np.int8)
    scales = np.empty((N, G), dtype=np.uint16)
    zeros = np.empty((N, G), dtype=np.uint8) if fmt == Q4_ZP else None
    rc = lib().oracle_quantize(W.ctypes.data, K, N, K, fmt, codes.ctypes.data,
                               scales.ctypes.data, None if zeros is None else zeros.ctypes.data)
    if rc == 3:
        raise NonFiniteError("non-finite weight or fp16 scale overflow")
    if rc:
        raise ValueError(f"bad format {fmt:#x} or K {K}")
    return (codes, scales) if zeros is None else (codes, scales, zeros)


def pack(codes: np.ndarray, scales: np.ndarray, fmt: int, zeros: np.ndarray | None = None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    N, K = codes.shape
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    out = np.empty(packed_bytes(fmt, N, K), dtype=np.uint8)
    rc = lib().oracle_pack(codes.ctypes.data, scales.ctypes.data,
                           None if zeros is None else zeros.ctypes.data, N, K, fmt, out.ctypes.data)
    if rc:
        raise ValueError(f"bad format {fmt:#x}, K {K} or missing zero points")
    return out


def quantize_pack(W: np.ndarray, fmt: int) -> np.ndarray:
    q = quantize(W, fmt)
    return pack(q[0], q[1], fmt, q[2] if len(q) > 2 else None)


def unpack(packed: np.ndarray, N: int, K: int, fmt: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    G = K // group_size(fmt)
    codes = np.empty((N, K), dtype=np.int8)
    scales = np.empty((N, G), dtype=np.uint16)
    zeros = np.empty((N, G), dtype=np.uint8) if fmt == Q4_ZP else None
    rc = lib().oracle_unpack(packed.ctypes.data, N, K, fmt, codes.ctypes.data, scales.ctypes.data,
                             None if zeros is None else zeros.ctypes.data)
    if rc:
        raise ValueError(f"bad format {fmt:#x} or K {K}")
    return (codes, scales) if zeros is None else (codes, scales, zeros)


def dequant(packed: np.ndarray, N: int, K: int, fmt: int, row0: int = 0,
            nrows: int | None = None) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    nrows = N - row0 if nrows is None else nrows
    out = np.empty((nrows, K), dtype=np.float64)
    rc = lib().oracle_dequant(packed.ctypes.data, N, K, fmt, row0, nrows, out.ctypes.data)
    if rc:
        raise ValueError("bad format or row range out of bounds")
    return out


def sweep(packed: np.ndarray, N: int, K: int, fmt: int, X: np.ndarray, cols=None,
          nthreads: int | None = None) -> np.ndarray:
    """Yref [M, ncols] in fp64 for X fp16 [M, K]; cols = None means all N."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    Xb = np.ascontiguousarray(np.asarray(X, dtype=np.float16)).view(np.uint16)
    M = Xb.shape[0]
    assert Xb.shape[1] == K
    if cols is None:
        c_ptr, ncols = None, N
    else:
        cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
        c_ptr, ncols = cols.ctypes.data, cols.size
    Y = np.empty((M, ncols), dtype=np.float64)
    rc = lib().oracle_sweep_f64(packed.ctypes.data, N, K, fmt, Xb.ctypes.data, K, M,
                                Y.ctypes.data, ncols, c_ptr, ncols, _threads(nthreads))
    if rc:
        raise RuntimeError(f"oracle_sweep_f64 failed ({rc})")
    return Y


def compare(Y: np.ndarray, Yref: np.ndarray, X: np.ndarray, smax: float) -> dict:
    """The acceptance test for one job (Y, Yref: [M, ncols]; X fp16 [M, K])."""
    Y = np.asarray(Y, dtype=np.float64)
    Yref = np.asarray(Yref, dtype=np.float64)
    diff = Y - Yref
    den = np.linalg.norm(Yref)
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    xn = np.linalg.norm(np.asarray(X, dtype=np.float64), axis=1)
    bound = MAX_ABS_COEF * xn * smax
    rowmax = np.abs(diff).max(axis=1) if diff.size else np.zeros(Y.shape[0])
    finite = bool(np.isfinite(Y).all())
    ok_rows = rowmax <= bound
    return {
        "rel_l2": rel,
        "max_abs_ratio": float((rowmax / np.where(bound > 0, bound, 1)).max()) if rowmax.size else 0.0,
        "finite": finite,
        "ok": finite and rel <= REL_L2_TOL and bool(ok_rows.all()),
    }


def max_scale(packed: np.ndarray, N: int, K: int, fmt: int) -> float:
    s = unpack(packed, N, K, fmt)[1]
    return float(np.abs(f16_bits_to_f64(s)).max())


def argmax_rows(Y: np.ndarray) -> np.ndarray:
    """Per row, the column of the largest value, the lowest one among equal
    values (numpy's argmax returns the first occurrence)."""
    return np.argmax(np.asarray(Y), axis=1).astype(np.int64)


def accept(argmax, drafts, slots) -> list:
    """Accepted draft count per slot (row0, ndraft): leading rows i < ndraft
    with argmax[row0 + i] == drafts[row0 + i], counted until the first that
    differs."""
    out = []
    for row0, nd in slots:
        L = 0
        while L < nd and int(argmax[row0 + L]) == int(drafts[row0 + L]):
            L += 1
        out.append(L)
    return out


def verify_head(packed: np.ndarray, N: int, K: int, fmt: int, X: np.ndarray, drafts, slots,
                nthreads: int | None = None):
    """(argmax [M], max logit [M], accepted per slot, logits [M, N]) in fp64."""
    Y = sweep(packed, N, K, fmt, X, nthreads=nthreads)
    am = argmax_rows(Y)
    mx = Y[np.arange(Y.shape[0]), am]
    return am, mx, accept(am, drafts, slots), Y


def top2_gap(Y: np.ndarray) -> np.ndarray:
    """Per row, the largest value minus the second largest (0 on a tie)."""
    Y = np.asarray(Y, dtype=np.float64)
    part = np.partition(Y, Y.shape[1] - 2, axis=1)
    return part[:, -1] - part[:, -2]


# ---------------------------------------------------------------------------
# Shared-KV attention verify (the attention half of a verify round)
# ---------------------------------------------------------------------------
# Geometry of the full-attention layers on the Quasar/q27 wiki: 4 KV heads of
# head_dim 256 (long-context note on KV bytes per token) and 6 query heads per
# KV head (the fp8-KV note: GQA = 6).  A slot's cache holds L positions; the
# last W of them are the slot's verify positions (the accepted token and its
# drafts), and query w sits at position L - W + w and attends causally to
# positions 0 .. L - W + w.  All W * 6 queries of a KV head read that head's
# keys and values once: the "shared-KV verify".
ATTN_HKV, ATTN_GROUP, ATTN_D = 4, 6, 256
ATTN_HQ = ATTN_HKV * ATTN_GROUP
KV_FP16, KV_FP8 = 0, 1


def e4m3_to_f64(codes) -> np.ndarray:
    """OCP FP8 E4M3 bytes -> values: sign, 4 exponent bits (bias 7), 3
    mantissa bits; exponent 0 is subnormal (m / 8 * 2^-6); S.1111.111 is NaN
    and there are no infinities (largest finite 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8 * 2.0 ** -6, (1 + m / 8) * np.ldexp(1.0, e - 7))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def f64_to_e4m3(x) -> np.ndarray:
    """Saturating conversion to E4M3 (the KV cache's scale-free fp8 form on
    the Quasar/q27 wiki, KV-cache item: no per-row scale; values beyond the
    largest finite 448 clamp to it): the nearest code, ties to the even
    mantissa; NaN -> 0x7F.  Written as a search over the 127 finite
    non-negative codes."""
    x = np.asarray(x, dtype=np.float64)
    vals = e4m3_to_f64(np.arange(127, dtype=np.uint8))        # 0 .. 448 ascending
    a = np.minimum(np.abs(x), 448.0)
    idx = np.searchsorted(vals, a)                            # vals[idx-1] < a <= vals[idx]
    idx = np.clip(idx, 1, 126)
    lo, hi = vals[idx - 1], vals[idx]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & (idx % 2 == 0))
    code = np.where(a == 0, 0, np.where(pick_hi, idx, idx - 1))
    code = np.where(a <= vals[0], 0, code)
    out = (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), out).astype(np.uint8)


def attn_verify(Q, K, V, W: int, scale: float) -> np.ndarray:
    """One slot, one layer.  Q fp16 [W, 24, 256]; K, V values [L, 4, 256]
    (fp16 arrays, or fp64 values decoded from fp8); returns O [W, 24, 256] in
    fp64: for query head h (KV head h // 6) at position p = L - W + w,
    O = sum_j softmax_j(scale * q . k_j) v_j over j = 0 .. p, the softmax
    taken with its maximum subtracted (exact in fp64 up to rounding)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L = K.shape[0]
    assert Q.shape == (W, ATTN_HQ, ATTN_D) and K.shape == V.shape == (L, ATTN_HKV, ATTN_D) and 1 <= W <= L
    O = np.empty((W, ATTN_HQ, ATTN_D), dtype=np.float64)
    for w in range(W):
        p = L - W + w
        for h in range(ATTN_HQ):
            g = h // ATTN_GROUP
            s = scale * (K[:p + 1, g, :] @ Q[w, h, :])
            e = np.exp(s - s.max())
            O[w, h, :] = (e @ V[:p + 1, g, :]) / e.sum()
    return O
