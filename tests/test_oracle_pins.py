"""Pins of the CPU oracle against facts it does not compute itself (CPU only).

Each test fixes part of the oracle to something other than the oracle: a
library routine it reduces to, brute force, exact rational arithmetic, a
closed form, an invariant, or numbers printed on the pages.  A dropped term,
a wrong sign or index, or a transposed operand anywhere in quantize / pack /
unpack / sweep fails at least one of them.
"""
from fractions import Fraction
import os

import numpy as np
import pytest

from oracle import oracle
from synth import synth, workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# fp16 rounding reduces to numpy's binary64 -> binary16 conversion (RNE)
# --------------------------------------------------------------------------
def test_f64_to_f16_matches_numpy():
    rng = _rng(1)
    parts = [
        rng.standard_normal(50_000) * 10.0 ** rng.integers(-9, 6, 50_000),
        np.ldexp(rng.integers(1, 2048, 20_000).astype(np.float64) + 0.5,
                 rng.integers(-40, 6, 20_000)),          # exact halfway cases
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12),
                  np.inf, -np.inf]),
    ]
    x = np.concatenate(parts)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = oracle.f64_to_f16_bits(x)
    assert np.array_equal(got, want)
    back = oracle.f16_bits_to_f64(want)
    assert np.array_equal(back, want.view(np.float16).astype(np.float64))


# --------------------------------------------------------------------------
# P3: scale formula recomputed independently with numpy
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 5])
def test_scale_formula(bits):
    W = synth.weights(31, 256, 0, 40, 0.02, outlier_thresh=workloads.OUTLIER_THRESH * 20)
    _, s = oracle.quantize(W, bits)
    qmax = (1 << (bits - 1)) - 1
    amax = np.abs(W.reshape(40, 8, 32)).max(axis=2).astype(np.float64)
    want = (amax / qmax).astype(np.float16).view(np.uint16)
    assert np.array_equal(s, want)


# --------------------------------------------------------------------------
# P1: quantizer == brute-force nearest code (exact), ties to even
# --------------------------------------------------------------------------
def _brute_codes(W, scales_bits, bits):
    """argmin_q |w - q*s| over q in [-Qmax, Qmax], exact in fp64 (w fp32,
    q*s has <= 15 significant bits), ties to the even q."""
    qmax = (1 << (bits - 1)) - 1
    N, K = W.shape
    s = np.repeat(scales_bits.view(np.float16).astype(np.float64), 32, axis=1)
    cand = np.arange(-qmax, qmax + 1, dtype=np.float64)
    err = np.abs(W.astype(np.float64)[..., None] - cand * s[..., None])
    best = err.min(axis=-1, keepdims=True)
    is_best = err == best
    n_best = is_best.sum(axis=-1)
    first = cand[np.argmax(is_best, axis=-1)]
    # with two minimal candidates q and q+1 keep the even one
    tie_pick = np.where(first % 2 == 0, first, first + 1)
    q = np.where(n_best == 2, tie_pick, first)
    q = np.where(s == 0, 0, q)
    return q.astype(np.int8)


@pytest.mark.parametrize("bits", [4, 5])
def test_quantizer_brute_force_workload1(bits):
    wl = workloads.workload(1)
    m = wl.matrices[0]
    W = synth.weights(m.seed, m.K, 0, m.N, workloads.SIGMA)
    codes, scales = oracle.quantize(W, bits)
    assert np.array_equal(codes, _brute_codes(W, scales, bits))


def test_quantizer_exact_ties_go_to_even():
    # one group: amax = 7*s exactly, other entries (k+1/2)*s -> ties
    s = np.float64(np.float16(0.015625))           # 2^-6, exact
    halves = np.array([0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, -0.5, -1.5, -2.5, -3.5, -4.5,
                       -5.5, -6.5])
    vals = np.concatenate([[7.0], halves, np.zeros(32 - 15)]) * s
    W = vals.astype(np.float32)[None, :]
    codes, scales = oracle.quantize(W, 4)
    assert scales[0, 0] == np.float16(s).view(np.uint16)
    want = np.concatenate([[7], [0, 2, 2, 4, 4, 6, 6, 0, -2, -2, -4, -4, -6, -6],
                           np.zeros(17)])
    assert np.array_equal(codes[0], want.astype(np.int8))


def test_quantizer_random_groups_brute_force():
    rng = _rng(7)
    W = (rng.standard_normal((64, 128)) * 10.0 ** rng.integers(-6, 2, (64, 1))).astype(np.float32)
    W[3, :32] = 0.0                                  # amax = 0 group
    W[4, 32:64] = 1e-9                               # scale underflows to 0
    for bits in (4, 5):
        codes, scales = oracle.quantize(W, bits)
        assert np.array_equal(codes, _brute_codes(W, scales, bits))
        assert scales[3, 0] == 0 and np.all(codes[3, :32] == 0)
        assert scales[4, 1] == 0 and np.all(codes[4, 32:64] == 0)


# --------------------------------------------------------------------------
# P2 round-trip bound, P12 error statistics, P11 bits consistency
# --------------------------------------------------------------------------
def test_roundtrip_bound_and_error_statistics():
    m = workloads.workload(4, layers=1).matrices[0]
    rms = {}
    for outl in (m.thresh, 0):
        W = synth.weights(m.seed, m.K, 0, 512, workloads.SIGMA, outlier_thresh=outl)
        for bits in (4, 5):
            packed = oracle.quantize_pack(W, bits)
            What = oracle.dequant(packed, 512, m.K, bits)
            _, sb = oracle.unpack(packed, 512, m.K, bits)
            s = np.repeat(oracle.f16_bits_to_f64(sb), 32, axis=1)
            err = W.astype(np.float64) - What
            assert np.all(np.abs(err) <= s / 2)            # |w - w_hat| <= s/2
            if outl:
                continue
            # uniform rounding error: E[err^2] ~ E[s^2]/12 (without outliers;
            # an outlier group leaves most of its entries far below s/2)
            ratio = (err ** 2).mean() / ((s ** 2).mean() / 12)
            assert 0.9 < ratio < 1.05, ratio
            rms[bits] = np.sqrt((err ** 2).mean())
    assert abs(rms[5] / rms[4] - 7 / 15) < 0.03


# --------------------------------------------------------------------------
# layout: pack/unpack is a bijection on the padded tile grid
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("N,K", [(16, 128), (37, 96), (5, 416)])
def test_pack_unpack_roundtrip(bits, N, K):
    rng = _rng(N * K + bits)
    bias = 1 << (bits - 1)
    codes = rng.integers(-bias, bias, (N, K)).astype(np.int8)     # every u value
    scales = rng.integers(0, 0x7C00, (N, K // 32)).astype(np.uint16)
    packed = oracle.pack(codes, scales, bits)
    assert packed.size == oracle.packed_bytes(bits, N, K)
    c2, s2 = oracle.unpack(packed, N, K, bits)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


@pytest.mark.parametrize("bits", [4, 5])
def test_every_code_bit_used_once(bits):
    """One-hot codes: each element owns exactly `bits` distinct bits, and the
    elements of a full tile cover the code (and high-bit) region exactly."""
    N, K = 16, 128
    bias = 1 << (bits - 1)
    zero_u = np.full((N, K), -bias, dtype=np.int8)               # u = 0
    scales = np.zeros((N, K // 32), dtype=np.uint16)
    base = oracle.pack(zero_u, scales, bits)
    assert not base.any()
    seen = np.zeros(base.size * 8, dtype=np.int32)
    for n in range(N):
        for k in range(K):
            c = zero_u.copy()
            c[n, k] = bias - 1                                     # u = all ones
            bitsset = np.unpackbits(oracle.pack(c, scales, bits), bitorder="little")
            idx = np.flatnonzero(bitsset)
            assert idx.size == bits
            seen[idx] += 1
    code_region = 1024 * 8 + (256 * 8 if bits == 5 else 0)
    used = np.flatnonzero(seen)
    assert np.all(seen[used] == 1) and used.size == N * K * bits
    assert used.size == code_region


def test_lane_contract_of_layout():
    """A 16-byte slice 16*l of a tile holds chunk c = l//16 (8 consecutive k)
    of the four groups of row r = l % 16: the property the kernels load by."""
    N, K, bits = 16, 128, 4
    scales = np.zeros((N, 4), dtype=np.uint16)
    for n in (0, 5, 15):
        for k in (0, 9, 37, 127):
            c = np.full((N, K), -8, dtype=np.int8)
            c[n, k] = 7
            nz = np.flatnonzero(oracle.pack(c, scales, bits))
            lane = n + 16 * ((k % 32) // 8)
            assert np.all((nz >= 16 * lane) & (nz < 16 * lane + 16))


def test_packed_size_matches_page_bpw_accounting():
    """The tile layout stores bits + 16/32 bits per weight; the same formula
    reproduces the bits-per-weight figures printed on the Quasar wiki."""
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "bpw_accounting.txt"))
            if l.strip() and not l.startswith("#")]
    bpw = {}
    for r in rows:
        if r[0] == "ratio":
            ratio = float(r[1])
            continue
        cb, grp, sb, want = int(r[0]), int(r[1]), int(r[2]), float(r[3])
        got = cb + sb / grp
        assert got == want
        bpw[(grp, sb)] = got
    assert round(bpw[(16, 8)] / bpw[(64, 16)], 4) == ratio
    for bits in (4, 5):
        N, K = 34816, 5120
        assert oracle.packed_bytes(bits, N, K) * 8 == N * K * (bits + 16 / 32)
    # 100.27 MB for the 34816 x 5120 gate+up matrix at 4 bits
    assert round(oracle.packed_bytes(4, 34816, 5120) / 1e6, 2) == 100.27


# --------------------------------------------------------------------------
# P4: all-ones codes give scale x row sums
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 5])
def test_all_ones_codes(bits):
    N, K, M = 48, 384, 3
    TB = 1152 if bits == 4 else 1408
    ntiles = (N // 16) * (K // 128)
    s16 = np.float16(0.0372)
    tile = np.zeros(TB, dtype=np.uint8)
    # u = q + bias with q = 1: 4-bit u = 9 (0b1001), 5-bit u = 17 (0b10001)
    tile[:1024] = 0x99 if bits == 4 else 0x11
    tile[1024:1152] = np.frombuffer(np.full(64, s16).tobytes(), dtype=np.uint8)
    if bits == 5:
        tile[1152:] = 0xFF
    packed = np.tile(tile, ntiles)
    # integer-valued X: everything exact
    Xi = _rng(3).integers(-4, 5, (M, K)).astype(np.float16)
    Y = oracle.sweep(packed, N, K, bits, Xi)
    want = float(s16) * Xi.astype(np.float64).sum(axis=1)
    assert np.array_equal(Y, np.repeat(want[:, None], N, axis=1))
    # general fp16 X: closed form within fp64 rounding
    X = synth.x_fp16(4, M, K)
    Y = oracle.sweep(packed, N, K, bits, X)
    want = float(s16) * X.astype(np.float64).sum(axis=1)
    assert np.allclose(Y, want[:, None], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# P5 column independence, P6 row independence
# --------------------------------------------------------------------------
def test_column_and_row_independence():
    N, K, M, bits = 64, 256, 4, 5
    W = synth.weights(41, K, 0, N, 0.02)
    X = synth.x_fp16(42, M, K)
    packed = oracle.quantize_pack(W, bits)
    Yfull = oracle.sweep(packed, N, K, bits, X)
    S = np.array([0, 7, 16, 33, 63])
    assert np.array_equal(oracle.sweep(packed, N, K, bits, X, cols=S), Yfull[:, S])
    W2 = W.copy()
    others = np.setdiff1d(np.arange(N), S)
    W2[others] = synth.weights(43, K, 0, others.size, 0.5)
    Y2 = oracle.sweep(oracle.quantize_pack(W2, bits), N, K, bits, X)
    assert np.array_equal(Y2[:, S], Yfull[:, S])
    assert not np.array_equal(Y2[:, others], Yfull[:, others])
    # row m of Y depends on row m of X only
    Y1 = oracle.sweep(packed, N, K, bits, X[1:2])
    assert np.array_equal(Y1[0], Yfull[1])


# --------------------------------------------------------------------------
# P7 integer-exact sweep
# --------------------------------------------------------------------------
def test_integer_exact_sweep():
    N, K, M, bits = 40, 640, 5, 5
    rng = _rng(9)
    codes = rng.integers(-15, 16, (N, K)).astype(np.int8)
    e = rng.integers(-8, 3, (N, K // 32))
    scales = np.ldexp(1.0, e).astype(np.float16).view(np.uint16)
    packed = oracle.pack(codes, scales, bits)
    X = rng.integers(-4, 5, (M, K)).astype(np.float16)
    Y = oracle.sweep(packed, N, K, bits, X)
    # exact: integer partial sums per group times power-of-two scales
    part = np.einsum("mgk,ngk->mng", X.astype(np.int64).reshape(M, K // 32, 32),
                     codes.astype(np.int64).reshape(N, K // 32, 32))
    want = (part * np.ldexp(1.0, e)[None]).sum(axis=2)
    assert np.array_equal(Y, want)


# --------------------------------------------------------------------------
# P8 tiny brute force in exact rational arithmetic, from fp32 W to Y
# --------------------------------------------------------------------------
def _f16_rne_exact(x: Fraction) -> Fraction:
    """Nearest binary16 value to x (ties to even mantissa), exactly."""
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


@pytest.mark.parametrize("bits", [4, 5])
def test_tiny_brute_force_exact(bits):
    N, K, M = 5, 64, 3
    W = synth.weights(51, K, 0, N, 0.3)
    X = synth.x_fp16(52, M, K)
    qmax = (1 << (bits - 1)) - 1
    what = [[None] * K for _ in range(N)]
    for n in range(N):
        for g in range(K // 32):
            grp = [Fraction(float(v)) for v in W[n, 32 * g:32 * g + 32]]
            amax = max(abs(v) for v in grp)
            s = _f16_rne_exact(Fraction(float(amax / qmax)))   # fp64 quotient, then fp16
            for t, v in enumerate(grp):
                if s == 0:
                    q = 0
                else:
                    r = v / s
                    q = int(r.__floor__())
                    frac = r - q
                    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and q % 2 == 1):
                        q += 1
                    q = max(-qmax, min(qmax, q))
                what[n][32 * g + t] = q * s
    Xf = [[Fraction(float(v)) for v in row] for row in X]
    want = np.array([[float(sum(Xf[m][k] * what[n][k] for k in range(K))) for n in range(N)]
                     for m in range(M)])
    Y = oracle.sweep(oracle.quantize_pack(W, bits), N, K, bits, X)
    assert np.allclose(Y, want, rtol=1e-15, atol=1e-300)


# --------------------------------------------------------------------------
# P9 one-hot X extracts the dequantized weights; P10 sign symmetry
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 5])
def test_one_hot_extracts_dequant(bits):
    N, K = 33, 160
    W = synth.weights(61, K, 0, N, 0.02, outlier_thresh=workloads.OUTLIER_THRESH * 50)
    packed = oracle.quantize_pack(W, bits)
    codes, sb = oracle.quantize(W, bits)
    what = codes.astype(np.float64) * np.repeat(oracle.f16_bits_to_f64(sb), 32, axis=1)
    X = np.eye(K, dtype=np.float16)[:64]
    Y = oracle.sweep(packed, N, K, bits, X)
    assert np.array_equal(Y, what[:, :64].T)


@pytest.mark.parametrize("bits", [4, 5])
def test_sign_symmetry(bits):
    N, K, M = 20, 320, 2
    W = synth.weights(71, K, 0, N, 0.02)
    X = synth.x_fp16(72, M, K)
    c1, s1 = oracle.quantize(W, bits)
    c2, s2 = oracle.quantize(-W, bits)
    assert np.array_equal(s1, s2) and np.array_equal(c2, -c1)
    Y1 = oracle.sweep(oracle.pack(c1, s1, bits), N, K, bits, X)
    Y2 = oracle.sweep(oracle.pack(c2, s2, bits), N, K, bits, X)
    assert np.array_equal(Y2, -Y1)


# --------------------------------------------------------------------------
# non-finite inputs and the comparison rule itself
# --------------------------------------------------------------------------
def test_nonfinite_rejected():
    W = np.zeros((2, 64), dtype=np.float32)
    W[1, 5] = np.nan
    with pytest.raises(oracle.NonFiniteError):
        oracle.quantize(W, 4)
    W[1, 5] = 7 * 65520.0            # scale rounds to fp16 infinity
    with pytest.raises(oracle.NonFiniteError):
        oracle.quantize(W, 4)
    W[1, 5] = 7 * 65504.0            # largest finite scale is fine
    oracle.quantize(W, 4)


def test_compare_rule_rejects_planted_errors():
    N, K, M, bits = 64, 256, 3, 4
    W = synth.weights(81, K, 0, N, 0.02)
    X = synth.x_fp16(82, M, K)
    packed = oracle.quantize_pack(W, bits)
    Yref = oracle.sweep(packed, N, K, bits, X)
    smax = oracle.max_scale(packed, N, K, bits)
    assert oracle.compare(Yref.astype(np.float32), Yref, X, smax)["ok"]
    bad = Yref.copy()
    bad[1, 7] += 2e-3 * np.linalg.norm(X[1].astype(np.float64)) * smax   # one column off
    assert not oracle.compare(bad, Yref, X, smax)["ok"]
    bad = Yref * (1 + 3e-4)                                              # global drift
    assert not oracle.compare(bad, Yref, X, smax)["ok"]
    bad = Yref.copy()
    bad[0, 0] = np.nan
    assert not oracle.compare(bad, Yref, X, smax)["ok"]
