"""Pins of the oracle's format variants (CPU only).

Q4_G64: 4-bit symmetric codes with one fp16 scale per 64 weights (the
Quasar/q27 wiki's group-64 byte accounting, "Batching & prefill notes").
Q4_ZP: 4-bit group-32 asymmetric codes with an integer zero point per group
(the INT4 W4A16 group-32 asymmetric weights of the qwen38 model notes,
"Path 1 -- vLLM" section).  Each test fixes the oracle to something it does
not compute itself: numpy re-derivations of the formulas, brute force over
every code, exact rational arithmetic, closed forms, a bound derived from the
rounding steps, raw byte offsets of the layout, or the pages' bpw figure.
"""
from fractions import Fraction
import os

import numpy as np
import pytest

from oracle import oracle
from synth import synth, workloads

HERE = os.path.dirname(os.path.abspath(__file__))
G64, ZP = oracle.Q4_G64, oracle.Q4_ZP


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _tiles(packed, N, K, tb):
    """Packed bytes as [row block, k tile, tile byte]."""
    return packed.reshape((N + 15) // 16, (K + 127) // 128, tb)


# --------------------------------------------------------------------------
# sizes: the group-64 format costs the pages' 4.25 bits per weight
# --------------------------------------------------------------------------
def test_packed_sizes():
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "bpw_accounting.txt"))
            if l.strip() and not l.startswith("#") and not l.startswith("ratio")]
    g64 = [float(r[3]) for r in rows if r[:3] == ["4", "64", "16"]][0]
    N, K = 34816, 5120
    assert oracle.packed_bytes(G64, N, K) * 8 == N * K * g64
    assert oracle.packed_bytes(ZP, N, K) * 8 == N * K * (4 + 16 / 32 + 4 / 32)
    assert oracle.packed_bytes(G64, 16, 96) == 0            # K not a multiple of 64
    assert oracle.packed_bytes(G64, 16, 192) == 2 * 1088
    assert oracle.packed_bytes(ZP, 17, 96) == 2 * 1184
    assert oracle.packed_bytes(0x304, 16, 128) == 0          # unknown format


# --------------------------------------------------------------------------
# Q4_G64 quantizer: scale formula (numpy) and brute-force nearest code
# --------------------------------------------------------------------------
def _brute_sym(W, s_rep, qmax):
    cand = np.arange(-qmax, qmax + 1, dtype=np.float64)
    err = np.abs(W.astype(np.float64)[..., None] - cand * s_rep[..., None])
    is_best = err == err.min(axis=-1, keepdims=True)
    first = cand[np.argmax(is_best, axis=-1)]
    tie = np.where(first % 2 == 0, first, first + 1)
    q = np.where(is_best.sum(axis=-1) == 2, tie, first)
    return np.where(s_rep == 0, 0, q).astype(np.int8)


def test_g64_quantizer_formula_and_brute_force():
    W = synth.weights(91, 384, 0, 48, 0.02, outlier_thresh=workloads.OUTLIER_THRESH * 20)
    W[5, 64:128] = 0.0                                         # amax = 0 group
    codes, sb = oracle.quantize(W, G64)
    amax = np.abs(W.reshape(48, 6, 64)).max(axis=2).astype(np.float64)
    assert np.array_equal(sb, (amax / 7).astype(np.float16).view(np.uint16))
    s_rep = np.repeat(_f16(sb), 64, axis=1)
    assert np.array_equal(codes, _brute_sym(W, s_rep, 7))
    assert sb[5, 1] == 0 and not codes[5, 64:128].any()


def test_g64_roundtrip_bound_and_statistics():
    W = synth.weights(92, 5120, 0, 256, workloads.SIGMA)
    packed = oracle.quantize_pack(W, G64)
    What = oracle.dequant(packed, 256, 5120, G64)
    s = np.repeat(_f16(oracle.unpack(packed, 256, 5120, G64)[1]), 64, axis=1)
    err = W.astype(np.float64) - What
    assert np.all(np.abs(err) <= s / 2)
    ratio = (err ** 2).mean() / ((s ** 2).mean() / 12)
    assert 0.9 < ratio < 1.05, ratio
    # a larger group has a larger amax: the error grows against group 32
    W32 = oracle.dequant(oracle.quantize_pack(W, oracle.Q4), 256, 5120, oracle.Q4)
    assert ((W - W32) ** 2).mean() < (err ** 2).mean()


# --------------------------------------------------------------------------
# Q4_G64 layout: code bytes as the 4-bit group-32 layout, scales at 1024 + 4r + 2h
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(16, 128), (37, 192), (5, 320)])
def test_g64_layout_raw_bytes(N, K):
    rng = _rng(N * K)
    codes = rng.integers(-8, 8, (N, K)).astype(np.int8)
    sb = rng.integers(1, 0x7C00, (N, K // 64)).astype(np.uint16)
    packed = oracle.pack(codes, sb, G64)
    assert packed.size == oracle.packed_bytes(G64, N, K)
    c2, s2 = oracle.unpack(packed, N, K, G64)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sb)
    # code region: byte for byte the group-32 4-bit layout (pinned elsewhere)
    ref = oracle.pack(codes, np.zeros((N, K // 32), np.uint16), oracle.Q4)
    t64, t32 = _tiles(packed, N, K, 1088), _tiles(ref, N, K, 1152)
    assert np.array_equal(t64[..., :1024], t32[..., :1024])
    # scale region read straight from the bytes
    for n in range(N):
        for g in range(K // 64):
            kt, h = divmod(g, 2)
            o = 1024 + 4 * (n % 16) + 2 * h
            word = int(t64[n // 16, kt, o]) | (int(t64[n // 16, kt, o + 1]) << 8)
            assert word == sb[n, g]
    # padding: rows past N and the half tile past K hold u = 8 and scale 0
    full = _tiles(packed, N, K, 1088)
    if K % 128:
        pad = oracle.unpack(packed, (N + 15) // 16 * 16, (K + 127) // 128 * 128, G64)
        assert not pad[1][:, K // 64:].any() and not pad[0][:, K:].any()
    assert full.shape[2] == 1088


# --------------------------------------------------------------------------
# Q4_ZP quantizer: parameters from numpy, codes by brute force
# --------------------------------------------------------------------------
def _zp_params(W):
    N, K = W.shape
    g = W.reshape(N, K // 32, 32).astype(np.float64)
    lo = np.minimum(g.min(axis=2), 0.0)
    hi = np.maximum(g.max(axis=2), 0.0)
    s = ((hi - lo) / 15).astype(np.float16)
    sf = s.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        z = np.where(sf > 0, np.clip(np.rint(-lo / sf), 0, 15), 0)
    return s.view(np.uint16), sf, z.astype(np.int64)


def _brute_zp(W, sf, z):
    N, K = W.shape
    s_rep = np.repeat(sf, 32, axis=1)
    z_rep = np.repeat(z, 32, axis=1)
    cand = np.arange(16, dtype=np.float64)
    # candidate u stands for q = u - z; nearest q * s, ties to the even q
    q = cand[None, None, :] - z_rep[..., None]
    err = np.abs(W.astype(np.float64)[..., None] - q * s_rep[..., None])
    is_best = err == err.min(axis=-1, keepdims=True)
    first = np.argmax(is_best, axis=-1)
    qf = first - z_rep
    u = np.where((is_best.sum(axis=-1) == 2) & (qf % 2 != 0), first + 1, first)
    return np.where(s_rep == 0, z_rep, u).astype(np.int8)


def test_zp_quantizer_params_and_brute_force():
    rng = _rng(93)
    W = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    W[1, :32] = np.abs(W[1, :32])          # all >= 0: lo = 0, z = 0
    W[2, 32:64] = -np.abs(W[2, 32:64])     # all <= 0: hi = 0, z = 15
    W[3, 64:96] = 0.0                      # s = 0
    W[4, 96:128] += 0.05                   # shifted group
    W[5, 128:160] = 1e-9                   # s underflows to 0
    u, sb, zs = oracle.quantize(W, ZP)
    s_want, sf, z_want = _zp_params(W)
    assert np.array_equal(sb, s_want)
    assert np.array_equal(zs, z_want)
    assert np.array_equal(u, _brute_zp(W, sf, z_want))
    assert zs[1, 0] == 0 and zs[2, 1] == 15
    assert sb[3, 2] == 0 and not u[3, 64:96].any() and zs[3, 2] == 0
    assert sb[5, 4] == 0


def test_zp_exact_ties_go_to_even():
    # s = 2^-6 exactly: hi - lo = 15 s with lo = -3 s, so z = 3; entries at
    # (k + 1/2) s round to the even k
    s = 2.0 ** -6
    vals = np.array([-3.0, 12.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 4.5] + [0.0] * 22) * s
    u, sb, zs = oracle.quantize(vals.astype(np.float32)[None, :], ZP)
    assert _f16(sb[0, 0]) == s and zs[0, 0] == 3
    q = u[0].astype(int) - 3
    assert list(q[:10]) == [-3, 12, 0, 2, 2, 0, -2, -2, 4, 4]


def test_zp_zero_exact_and_roundtrip_bound():
    W = synth.weights(94, 512, 0, 128, 0.02, outlier_thresh=workloads.OUTLIER_THRESH * 20)
    W[:, ::7] = 0.0
    packed = oracle.quantize_pack(W, ZP)
    What = oracle.dequant(packed, 128, 512, ZP)
    assert np.all(What[:, ::7] == 0.0)                       # zero is representable
    s = np.repeat(_f16(oracle.unpack(packed, 128, 512, ZP)[1]), 32, axis=1)
    err = np.abs(W.astype(np.float64) - What)
    # nearest-code rounding gives s/2; the fp16 rounding of s can shorten
    # the 15-step grid by at most 15 s 2^-11, which only the clamp at the top sees
    assert np.all(err <= s * (0.5 + 15 * 2.0 ** -11 * 1.01))
    assert np.mean(err <= s / 2) > 0.999


# --------------------------------------------------------------------------
# Q4_ZP layout: zero points at 1152 + 2r, bits 4j..4j+3
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(16, 128), (37, 96), (5, 416)])
def test_zp_layout_raw_bytes(N, K):
    rng = _rng(N + K)
    u = rng.integers(0, 16, (N, K)).astype(np.int8)
    sb = rng.integers(1, 0x7C00, (N, K // 32)).astype(np.uint16)
    zs = rng.integers(0, 16, (N, K // 32)).astype(np.uint8)
    packed = oracle.pack(u, sb, ZP, zs)
    assert packed.size == oracle.packed_bytes(ZP, N, K)
    u2, s2, z2 = oracle.unpack(packed, N, K, ZP)
    assert np.array_equal(u2, u) and np.array_equal(s2, sb) and np.array_equal(z2, zs)
    tz = _tiles(packed, N, K, 1184)
    # codes and scales: byte for byte the 4-bit symmetric layout of u - 8
    # (padding is u = 0 here, so compare on the full grid with it explicit)
    Nf, Kf = (N + 15) // 16 * 16, (K + 127) // 128 * 128
    uf = np.zeros((Nf, Kf), np.int64)
    uf[:N, :K] = u
    sf = np.zeros((Nf, Kf // 32), np.uint16)
    sf[:N, :K // 32] = sb
    ref = _tiles(oracle.pack((uf - 8).astype(np.int8), sf, oracle.Q4), Nf, Kf, 1152)
    assert np.array_equal(tz[..., :1152], ref)
    for n in range(N):
        for g in range(K // 32):
            kt, j = divmod(g, 4)
            o = 1152 + 2 * (n % 16)
            word = int(tz[n // 16, kt, o]) | (int(tz[n // 16, kt, o + 1]) << 8)
            assert (word >> (4 * j)) & 15 == zs[n, g]
    # padding groups and rows: all zero bytes in the zero-point area
    if K % 128 or N % 16:
        pad = oracle.unpack(packed, (N + 15) // 16 * 16, (K + 127) // 128 * 128, ZP)
        assert not pad[2][N:].any() and not pad[2][:, K // 32:].any() and not pad[0][N:].any()


def test_zp_every_zero_bit_used_once():
    N, K = 16, 128
    u = np.zeros((N, K), np.int8)
    sb = np.zeros((N, 4), np.uint16)
    seen = np.zeros(1184 * 8, dtype=np.int32)
    for n in range(N):
        for g in range(4):
            zs = np.zeros((N, 4), np.uint8)
            zs[n, g] = 15
            idx = np.flatnonzero(np.unpackbits(oracle.pack(u, sb, ZP, zs), bitorder="little"))
            assert idx.size == 4
            seen[idx] += 1
    used = np.flatnonzero(seen)
    assert np.all(seen[used] == 1) and used.size == 256
    assert used.min() == 1152 * 8 and used.max() == 1184 * 8 - 1


# --------------------------------------------------------------------------
# sweeps: closed forms, integer-exact sums, exact rational brute force
# --------------------------------------------------------------------------
def test_g64_all_ones_codes():
    N, K, M = 32, 256, 3
    s16 = np.float16(0.0372)
    tile = np.zeros(1088, dtype=np.uint8)
    tile[:1024] = 0x99                                           # u = 9: q = 1
    tile[1024:] = np.frombuffer(np.full(32, s16).tobytes(), dtype=np.uint8)
    packed = np.tile(tile, (N // 16) * (K // 128))
    X = _rng(95).integers(-4, 5, (M, K)).astype(np.float16)
    Y = oracle.sweep(packed, N, K, G64, X)
    want = float(s16) * X.astype(np.float64).sum(axis=1)
    assert np.array_equal(Y, np.repeat(want[:, None], N, axis=1))


def test_zp_constant_offset_closed_form():
    # u = 5 everywhere, z = 2 in every group: w_hat = 3 s, so Y = 3 s rowsum
    N, K, M = 32, 256, 2
    s16 = np.float16(0.125)
    tile = np.zeros(1184, dtype=np.uint8)
    tile[:1024] = 0x55
    tile[1024:1152] = np.frombuffer(np.full(64, s16).tobytes(), dtype=np.uint8)
    tile[1152:] = np.frombuffer(np.full(16, 0x2222, np.uint16).tobytes(), dtype=np.uint8)
    packed = np.tile(tile, (N // 16) * (K // 128))
    X = _rng(96).integers(-4, 5, (M, K)).astype(np.float16)
    Y = oracle.sweep(packed, N, K, ZP, X)
    want = 3 * float(s16) * X.astype(np.float64).sum(axis=1)
    assert np.array_equal(Y, np.repeat(want[:, None], N, axis=1))


@pytest.mark.parametrize("fmt", [G64, ZP])
def test_integer_exact_sweep(fmt):
    N, K, M = 24, 640, 4
    gs = oracle.group_size(fmt)
    rng = _rng(97 + fmt)
    e = rng.integers(-8, 3, (N, K // gs))
    sb = np.ldexp(1.0, e).astype(np.float16).view(np.uint16)
    X = rng.integers(-4, 5, (M, K)).astype(np.float16)
    if fmt == ZP:
        u = rng.integers(0, 16, (N, K)).astype(np.int8)
        zs = rng.integers(0, 16, (N, K // 32)).astype(np.uint8)
        packed = oracle.pack(u, sb, fmt, zs)
        q = u.astype(np.int64) - np.repeat(zs.astype(np.int64), 32, axis=1)
    else:
        q = rng.integers(-8, 8, (N, K)).astype(np.int8)
        packed = oracle.pack(q, sb, fmt)
        q = q.astype(np.int64)
    Y = oracle.sweep(packed, N, K, fmt, X)
    part = np.einsum("mgk,ngk->mng", X.astype(np.int64).reshape(M, K // gs, gs), q.reshape(N, K // gs, gs))
    assert np.array_equal(Y, (part * np.ldexp(1.0, e)[None]).sum(axis=2))


def _f16_rne_exact(x: Fraction) -> Fraction:
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= 2 ** (e + 1):
        e += 1
    while a < 2 ** e:
        e -= 1
    ulp = Fraction(2) ** (max(e, -14) - 10)
    q, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return sign * q * ulp


def _rne(r: Fraction) -> int:
    q = r.__floor__()
    f = r - q
    if f > Fraction(1, 2) or (f == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return int(q)


@pytest.mark.parametrize("fmt", [G64, ZP])
def test_tiny_brute_force_exact(fmt):
    N, K, M = 4, 128, 3
    W = synth.weights(98, K, 0, N, 0.3)
    X = synth.x_fp16(99, M, K)
    gs = oracle.group_size(fmt)
    what = [[None] * K for _ in range(N)]
    for n in range(N):
        for g in range(K // gs):
            grp = [Fraction(float(v)) for v in W[n, gs * g:gs * g + gs]]
            if fmt == G64:
                s = _f16_rne_exact(Fraction(float(max(abs(v) for v in grp) / 7)))
                for t, v in enumerate(grp):
                    q = 0 if s == 0 else max(-7, min(7, _rne(v / s)))
                    what[n][gs * g + t] = q * s
            else:
                lo, hi = min(min(grp), 0), max(max(grp), 0)
                s = _f16_rne_exact(Fraction(float((hi - lo) / 15)))   # fp64 quotient, then fp16
                z = 0 if s == 0 else max(0, min(15, _rne(-lo / s)))
                for t, v in enumerate(grp):
                    u = z if s == 0 else max(0, min(15, _rne(v / s) + z))
                    what[n][gs * g + t] = (u - z) * s
    Xf = [[Fraction(float(v)) for v in row] for row in X]
    want = np.array([[float(sum(Xf[m][k] * what[n][k] for k in range(K))) for n in range(N)]
                     for m in range(M)])
    Y = oracle.sweep(oracle.quantize_pack(W, fmt), N, K, fmt, X)
    assert np.allclose(Y, want, rtol=1e-15, atol=1e-300)


@pytest.mark.parametrize("fmt", [G64, ZP])
def test_one_hot_extracts_dequant(fmt):
    N, K = 33, 192
    W = synth.weights(100, K, 0, N, 0.02, outlier_thresh=workloads.OUTLIER_THRESH * 50)
    qz = oracle.quantize(W, fmt)
    gs = oracle.group_size(fmt)
    q = qz[0].astype(np.float64)
    if fmt == ZP:
        q = q - np.repeat(qz[2].astype(np.float64), 32, axis=1)
    what = q * np.repeat(_f16(qz[1]), gs, axis=1)
    Y = oracle.sweep(oracle.quantize_pack(W, fmt), N, K, fmt, np.eye(K, dtype=np.float16)[:80])
    assert np.array_equal(Y, what[:, :80].T)


def test_g64_sign_symmetry_and_zp_mirror():
    N, K, M = 20, 320, 2
    W = synth.weights(101, K, 0, N, 0.02)
    X = synth.x_fp16(102, M, K)
    c1, s1 = oracle.quantize(W, G64)
    c2, s2 = oracle.quantize(-W, G64)
    assert np.array_equal(s1, s2) and np.array_equal(c2, -c1)
    # mirroring W swaps lo and hi: same scale, z -> 15 - z and u -> 15 - u
    # wherever no rounding tie or clamp intervenes; the products stay mirrored
    u1, t1, z1 = oracle.quantize(W, ZP)
    u2, t2, z2 = oracle.quantize(-W, ZP)
    assert np.array_equal(t1, t2)
    Y1 = oracle.sweep(oracle.pack(u1, t1, ZP, z1), N, K, ZP, X)
    Y2 = oracle.sweep(oracle.pack(u2, t2, ZP, z2), N, K, ZP, X)
    rel = np.abs(Y1 + Y2).max() / np.abs(Y1).max()
    assert rel < 0.05


def test_zp_nonfinite_rejected():
    W = np.zeros((2, 64), dtype=np.float32)
    W[1, 5] = np.inf
    with pytest.raises(oracle.NonFiniteError):
        oracle.quantize(W, ZP)
    W[1, 5] = 8 * 65520.0
    W[1, 6] = -8 * 65520.0            # (hi - lo) / 15 above the largest fp16
    with pytest.raises(oracle.NonFiniteError):
        oracle.quantize(W, ZP)
    W[1, 6] = -7 * 65504.0
    W[1, 5] = 8 * 65504.0             # exactly 65504 * 15 / 15
    oracle.quantize(W, ZP)


def test_formats_reject_bad_group_size():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 96), np.float32), G64)
