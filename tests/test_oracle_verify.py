"""Pins of the oracle's verify head (greedy acceptance) -- CPU only.

The argmax and the acceptance count are fixed to hand-worked cases, to a
quantization recomputed independently with numpy, and to exact rational
arithmetic on tiny inputs, never to the oracle itself.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle
from synth import synth


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_accept_hand_cases():
    # rows:        0  1  2  3   4  5 | 6  7 | 8 | 9 10 11
    argmax = np.array([7, 3, 9, 1, 4, 2, 5, 8, 6, 1, 1, 0])
    drafts = np.array([7, 3, 9, 2, 4, 0, 6, 0, 0, 1, 1, 0])
    slots = [(0, 5),   # rows 0..2 match, row 3 differs -> 3
             (6, 1),   # row 6: 5 != 6 -> 0
             (8, 0),   # no drafts -> 0
             (9, 2)]   # rows 9, 10 match, all drafts stand -> 2
    assert oracle.accept(argmax, drafts, slots) == [3, 0, 0, 2]
    # a mismatch ends the prefix even if later rows agree again
    assert oracle.accept(np.array([1, 2, 3, 4]), np.array([1, 9, 3, 4]), [(0, 3)]) == [1]


def test_argmax_lowest_column_on_ties():
    Y = np.array([[0.5, 2.0, 2.0, -1.0],
                  [-3.0, -3.0, -4.0, -3.0],
                  [1.0, 0.0, 0.0, 1.0 + 2 ** -40]])
    assert list(oracle.argmax_rows(Y)) == [1, 0, 3]
    assert list(oracle.top2_gap(Y)) == [0.0, 0.0, 2 ** -40]


def _numpy_dequant(W, bits):
    """Dequantized weights recomputed with numpy alone (not the oracle's C)."""
    N, K = W.shape
    qmax = (1 << (bits - 1)) - 1
    g = W.reshape(N, K // 32, 32).astype(np.float64)
    s = (np.abs(g).max(axis=2) / qmax).astype(np.float16).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s[:, :, None] > 0, np.clip(np.rint(g / s[:, :, None]), -qmax, qmax), 0.0)
    return (q * s[:, :, None]).reshape(N, K)


@pytest.mark.parametrize("bits", [4, 5])
def test_one_hot_row_picks_largest_dequantized_weight(bits):
    N, K = 200, 96
    W = synth.weights(77, K, 0, N, 0.02)
    k0 = 41
    # a planted clear winner and, in another column, an exact tie between
    # two identical weight rows
    W[123, :] = W[5, :]
    W[123, k0] = 0.5
    W[5, k0] = 0.5 * 0.6
    k1 = 70
    W[30, :] = W[150, :]
    W[30, k1] = W[150, k1] = 0.4
    packed = oracle.quantize_pack(W, bits)
    X = np.zeros((2, K), dtype=np.float16)
    X[0, k0] = 1.0
    X[1, k1] = 1.0
    drafts = np.array([123, 0])
    am, mx, acc, Y = oracle.verify_head(packed, N, K, bits, X, drafts, [(0, 1)])
    deq = _numpy_dequant(W, bits)
    assert am[0] == 123 == int(np.argmax(deq[:, k0]))
    assert am[1] == 30            # rows 30 and 150 tie; the lower wins
    assert deq[30, k1] == deq[150, k1] == mx[1]
    assert acc == [1]
    assert np.array_equal(Y[0], deq[:, k0])


@pytest.mark.parametrize("bits", [4, 5])
def test_tiny_exact_rational_argmax(bits):
    rng = _rng(5 + bits)
    N, K, M = 37, 64, 3
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    X = rng.standard_normal((M, K)).astype(np.float16)
    packed = oracle.quantize_pack(W, bits)
    codes, scales = oracle.unpack(packed, N, K, bits)
    s = oracle.f16_bits_to_f64(scales)
    exact = []
    for m in range(M):
        row = []
        for n in range(N):
            t = Fraction(0)
            for k in range(K):
                t += Fraction(float(X[m, k])) * Fraction(int(codes[n, k])) * Fraction(float(s[n, k // 32]))
            row.append(t)
        exact.append(row)
    want = [max(range(N), key=lambda n: (r[n], -n)) for r in exact]
    drafts = np.array([want[0], want[1], (want[2] + 1) % N])
    am, mx, acc, _ = oracle.verify_head(packed, N, K, bits, X, drafts, [(0, 2)])
    assert list(am) == want
    for m in range(M):
        assert mx[m] == float(exact[m][want[m]])
    assert acc == [2]
