"""Pins of the oracle's attention verify and its fp8 KV decode (CPU only).

E4M3 is fixed by its definition (every one of the 256 codes, a few printed
anchors of the format, nearest-code search with ties to even and saturation).
The attention is fixed by closed forms and invariants that a dropped term, a
wrong index or a transposed operand breaks: constant keys give the mean of
the visible values, one dominant key selects its value row, future positions
never matter (causality), context order does not matter, the six query heads
of a group share their KV head, the output is affine in V, and a tiny case
agrees with a 40-digit decimal evaluation.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import oracle

HQ, HKV, G, D = oracle.ATTN_HQ, oracle.ATTN_HKV, oracle.ATTN_GROUP, oracle.ATTN_D


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _qkv(seed, W, L, kscale=1.0):
    r = _rng(seed)
    Q = r.standard_normal((W, HQ, D)).astype(np.float16)
    K = (r.standard_normal((L, HKV, D)) * kscale).astype(np.float16)
    V = r.standard_normal((L, HKV, D)).astype(np.float16)
    return Q, K, V


# --------------------------------------------------------------------------
# E4M3
# --------------------------------------------------------------------------
def test_e4m3_every_code_from_the_definition():
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        v = oracle.e4m3_to_f64(np.uint8(c))
        if e == 15 and m == 7:
            assert np.isnan(v)
            continue
        want = s * (m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (8 + m) / 8)
        assert v == want, c
    anchors = {0x38: 1.0, 0x40: 2.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0xC0: -2.0, 0x00: 0.0}
    for c, v in anchors.items():
        assert oracle.e4m3_to_f64(np.uint8(c)) == v


def test_e4m3_encode_is_nearest_with_ties_to_even_and_saturates():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_to_f64(codes)
    assert np.array_equal(oracle.f64_to_e4m3(vals)[vals != 0], codes[vals != 0])
    r = _rng(3)
    x = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-4, 3, 20000),
                        [500.0, -1e6, 448.0, 464.0, 449.0, 0.0, -0.0]])
    got = oracle.f64_to_e4m3(x)
    gv = oracle.e4m3_to_f64(got)
    finite = oracle.e4m3_to_f64(np.arange(127, dtype=np.uint8))     # the non-negative finite codes
    for xi, g in zip(x, gv):
        a = min(abs(xi), 448.0)
        d = np.abs(np.abs(finite) - a)
        best = d.min()
        assert abs(abs(g) - a) == best
        if np.count_nonzero(d == best) > 1 and a != 0:           # a tie: the even code wins
            c = oracle.f64_to_e4m3(np.array([a]))[0]
            assert c % 2 == 0
        assert g == 0 or np.sign(g) == np.sign(xi)
    assert oracle.f64_to_e4m3(np.array([np.nan]))[0] == 0x7F
    # 464 is halfway between 448 and the (absent) 480: saturation, not rounding up
    assert oracle.e4m3_to_f64(oracle.f64_to_e4m3(np.array([464.0, 1e9])))[0] == 448.0


# --------------------------------------------------------------------------
# attention: closed forms
# --------------------------------------------------------------------------
def test_constant_keys_give_the_mean_of_visible_values():
    W, L = 3, 9
    Q, _, V = _qkv(1, W, L)
    K = np.zeros((L, HKV, D), np.float16)
    O = oracle.attn_verify(Q, K, V, W, 1 / 16)
    for w in range(W):
        p = L - W + w
        want = V[:p + 1].astype(np.float64).mean(axis=0)        # [HKV, D]
        for h in range(HQ):
            assert np.allclose(O[w, h], want[h // G], rtol=0, atol=1e-15)


def test_one_dominant_key_selects_its_value():
    W, L = 2, 7
    Q, K, V = _qkv(2, W, L, kscale=0.01)
    # key 3 of KV head 1 aligned with every query of that head, scaled up
    K[3, 1] = 0
    for h in range(G, 2 * G):
        K[3, 1] += (Q[:, h].astype(np.float32).sum(axis=0) * 4).astype(np.float16)
    O = oracle.attn_verify(Q, K, V, W, 1.0)
    for w in range(W):
        for h in range(G, 2 * G):
            assert np.allclose(O[w, h], V[3, 1].astype(np.float64), atol=1e-9)


def test_single_visible_position_copies_its_value():
    Q, K, V = _qkv(4, 1, 1)
    O = oracle.attn_verify(Q, K, V, 1, 0.3)
    for h in range(HQ):
        assert np.array_equal(O[0, h], V[0, h // G].astype(np.float64))


# --------------------------------------------------------------------------
# attention: invariants
# --------------------------------------------------------------------------
def test_causality_future_positions_do_not_matter():
    W, L = 5, 40
    Q, K, V = _qkv(5, W, L)
    O = oracle.attn_verify(Q, K, V, W, 1 / 16)
    for w in range(W):
        p = L - W + w
        K2, V2 = K.copy(), V.copy()
        K2[p + 1:] = 7
        V2[p + 1:] = -3
        O2 = oracle.attn_verify(Q, K2, V2, W, 1 / 16)
        assert np.array_equal(O2[w], O[w])
        if p + 1 < L:
            assert not np.array_equal(O2[W - 1], O[W - 1])


def test_context_order_does_not_matter():
    W, L = 4, 33
    Q, K, V = _qkv(6, W, L)
    perm = np.concatenate([_rng(7).permutation(L - W), np.arange(L - W, L)])
    O = oracle.attn_verify(Q, K, V, W, 1 / 16)
    Op = oracle.attn_verify(Q, K[perm], V[perm], W, 1 / 16)
    assert np.allclose(O, Op, rtol=1e-12, atol=1e-13)


def test_group_heads_share_their_kv_head_and_others_do_not():
    W, L = 2, 20
    Q, K, V = _qkv(8, W, L)
    Q[:, 1] = Q[:, 0]                     # heads 0, 1: same KV head 0
    Q[:, 6] = Q[:, 0]                     # head 6: KV head 1
    O = oracle.attn_verify(Q, K, V, W, 1 / 16)
    assert np.array_equal(O[:, 1], O[:, 0])
    assert not np.allclose(O[:, 6], O[:, 0])
    K[:, 0] = 0
    V[:, 0] = 0                           # KV head 0 silenced: only heads 0..5 change
    O2 = oracle.attn_verify(Q, K, V, W, 1 / 16)
    assert np.all(O2[:, :G] == 0) and np.array_equal(O2[:, G:], O[:, G:])


def test_affine_in_values():
    W, L = 3, 17
    Q, K, V = _qkv(9, W, L)
    V = (np.round(V.astype(np.float32) * 8) / 8).astype(np.float16)     # eighths: V + 1 stays exact
    O = oracle.attn_verify(Q, K, V, W, 1 / 16)
    O2 = oracle.attn_verify(Q, K, (V.astype(np.float32) * 2).astype(np.float16), W, 1 / 16)
    assert np.array_equal(O2, 2 * O)                                     # scaling by 2 is exact
    O3 = oracle.attn_verify(Q, K, (V.astype(np.float32) + 1).astype(np.float16), W, 1 / 16)
    assert np.allclose(O3, O + 1, rtol=0, atol=1e-12)


def test_tiny_case_against_decimal():
    getcontext().prec = 40
    W, L = 2, 5
    Q, K, V = _qkv(10, W, L)
    scale = 0.0625
    O = oracle.attn_verify(Q, K, V, W, scale)
    for w in range(W):
        p = L - W + w
        for h in (0, 7, 23):
            g = h // G
            s = [sum(Decimal(float(Q[w, h, d])) * Decimal(float(K[j, g, d])) for d in range(D)) * Decimal(scale)
                 for j in range(p + 1)]
            e = [x.exp() for x in s]
            tot = sum(e)
            for d in (0, 100, 255):
                want = sum(e[j] * Decimal(float(V[j, g, d])) for j in range(p + 1)) / tot
                assert abs(O[w, h, d] - float(want)) <= 1e-14 * max(1.0, abs(float(want)))


def test_fp8_values_flow_through_unchanged():
    """Decoded fp8 caches are ordinary values to the attention: the output
    from decoded codes equals the output from the same values as fp16."""
    W, L = 2, 12
    Q, K, V = _qkv(11, W, L)
    kc, vc = oracle.f64_to_e4m3(K.astype(np.float64)), oracle.f64_to_e4m3(V.astype(np.float64))
    Kd, Vd = oracle.e4m3_to_f64(kc), oracle.e4m3_to_f64(vc)
    assert np.array_equal(Kd.astype(np.float16).astype(np.float64), Kd)     # exact in fp16
    O1 = oracle.attn_verify(Q, Kd, Vd, W, 1 / 16)
    O2 = oracle.attn_verify(Q, Kd.astype(np.float16), Vd.astype(np.float16), W, 1 / 16)
    assert np.array_equal(O1, O2)
