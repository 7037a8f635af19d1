"""GPU parity of the shared-KV attention verify against the CPU oracle,
through the C boundary: fp16 and E4M3 caches, single and multi-chunk
positions, ragged W and L, several slots per call, repeat determinism, and
both workloads the benchmark times: one slot over 32768 positions (checked
on every query row of a sampled set of heads) and eight slots over 8192
each (checked on every row)."""
import numpy as np
import pytest

from oracle import oracle
from self_speculative_verify_amd import qgemm
from synth import synth

from gpu_util import device, say, to_dev

pytestmark = pytest.mark.gpu

HQ, HKV, D = qgemm.ATTN_HKV * qgemm.ATTN_GROUP, qgemm.ATTN_HKV, qgemm.ATTN_D
SCALE = 1 / 16


def _case(seed, W, L, kv, kscale=1.0):
    Q = synth.x_fp16(seed, W * HQ, D).reshape(W, HQ, D)
    K = (synth.x_fp16(seed + 1, L * HKV, D).astype(np.float32) * kscale).astype(np.float16).reshape(L, HKV, D)
    V = synth.x_fp16(seed + 2, L * HKV, D).reshape(L, HKV, D)
    if kv == qgemm.KV_FP8:
        Kc = oracle.f64_to_e4m3(K.astype(np.float64))
        Vc = oracle.f64_to_e4m3(V.astype(np.float64))
        return Q, Kc, Vc, oracle.e4m3_to_f64(Kc), oracle.e4m3_to_f64(Vc)
    return Q, K, V, K, V


def _check(O, Oref, Vvals, what):
    diff = O.astype(np.float64) - Oref
    rel = np.linalg.norm(diff) / np.linalg.norm(Oref)
    mx = np.abs(diff).max() / np.abs(Vvals).max()
    say(f"  {what}: rel_l2={rel:.2e} max_abs/max|V|={mx:.2e}")
    assert np.isfinite(O).all()
    assert rel <= 1e-3 and mx <= 2e-3, what


def _run(cases, kv):
    import torch

    dev = device()
    slots, keep = [], []
    for Q, Kc, Vc, _, _ in cases:
        W, L = Q.shape[0], Kc.shape[0]
        Qd, Kd, Vd = to_dev(Q), to_dev(Kc), to_dev(Vc)
        O = torch.full((W, HQ, D), float("nan"), dtype=torch.float32, device=dev)
        slots.append((Qd, Kd, Vd, O, L, W))
        keep.append(O)
    arr = qgemm.attn_slots(slots)
    ws = qgemm.Workspace(qgemm.attn_workspace_bytes(arr, kv), device=dev)
    qgemm.attn_verify(arr, kv, SCALE, ws)
    torch.cuda.synchronize()
    out = [O.cpu().numpy() for O in keep]
    return out, (arr, ws, slots, keep)


CASES = [(1, 1), (1, 2), (6, 6), (6, 37), (6, 1000), (16, 300), (12, 4097), (3, 65), (16, 16)]


@pytest.mark.parametrize("kv", [qgemm.KV_FP16, qgemm.KV_FP8])
@pytest.mark.parametrize("W,L", CASES)
def test_attn_single_slot(kv, W, L):
    say(f"attn kv={kv} W={W} L={L}")
    case = _case(10 * W + L, W, L, kv)
    (O,), _ = _run([case], kv)
    Q, _, _, Kv, Vv = case
    _check(O, oracle.attn_verify(Q, Kv, Vv, W, SCALE), Vv, f"W={W} L={L}")


@pytest.mark.parametrize("kv", [qgemm.KV_FP16, qgemm.KV_FP8])
def test_attn_many_slots_one_call_and_determinism(kv):
    import torch

    shapes = [(6, 500), (1, 3), (16, 2049), (8, 64), (5, 777)]
    cases = [_case(100 + i, W, L, kv, kscale=1.5) for i, (W, L) in enumerate(shapes)]
    outs, (arr, ws, slots, keep) = _run(cases, kv)
    for (W, L), case, O in zip(shapes, cases, outs):
        Q, _, _, Kv, Vv = case
        _check(O, oracle.attn_verify(Q, Kv, Vv, W, SCALE), Vv, f"slot W={W} L={L}")
    for O in keep:
        O.fill_(float("nan"))
    qgemm.attn_verify(arr, kv, SCALE, ws)
    torch.cuda.synchronize()
    for O, o1 in zip(keep, outs):
        assert np.array_equal(O.cpu().numpy(), o1)


def test_attn_peaked_scores():
    """Keys scaled up: near one-hot softmax rows, where the running maximum
    changes between chunks."""
    W, L = 6, 3000
    case = _case(7, W, L, qgemm.KV_FP16, kscale=8.0)
    (O,), _ = _run([case], qgemm.KV_FP16)
    Q, _, _, Kv, Vv = case
    _check(O, oracle.attn_verify(Q, Kv, Vv, W, SCALE), Vv, "peaked")


@pytest.mark.parametrize("kv", [qgemm.KV_FP16, qgemm.KV_FP8])
def test_attn_long_context_workload(kv):
    """The benchmark's shape: one slot, W = 6, L = 32768, as bench.py times it
    (checked on all rows of KV heads 0 and 3)."""
    W, L = 6, 32768
    case = _case(4242, W, L, kv)
    (O,), _ = _run([case], kv)
    Q, _, _, Kv, Vv = case
    assert np.isfinite(O).all()
    for g in (0, 3):
        hs = list(range(6 * g, 6 * g + 6))
        Qs = np.zeros_like(Q)
        Qs[:, hs] = Q[:, hs]
        Oref = oracle.attn_verify(Qs, Kv, Vv, W, SCALE)
        _check(O[:, hs], Oref[:, hs], Vv, f"L=32768 kv head {g}")


@pytest.mark.parametrize("kv", [qgemm.KV_FP16, qgemm.KV_FP8])
def test_attn_eight_slot_workload(kv):
    """The benchmark's many-slot shape: 8 slots of W = 6 over L = 8192 each,
    in one call, every slot checked on all its query rows."""
    W, L, n = 6, 8192, 8
    cases = [_case(5000 + 10 * i, W, L, kv) for i in range(n)]
    outs, _ = _run(cases, kv)
    for i, (case, O) in enumerate(zip(cases, outs)):
        Q, _, _, Kv, Vv = case
        _check(O, oracle.attn_verify(Q, Kv, Vv, W, SCALE), Vv, f"slot {i}")


@pytest.mark.parametrize("kv", [qgemm.KV_FP16, qgemm.KV_FP8])
def test_attn_single_position_returns_values_exactly(kv):
    """One visible position: the softmax weight is exactly 1, so O is the
    value row decoded from the cache, bit for bit.  The E4M3 row holds all
    256 codes (the NaN codes give NaN)."""
    import torch

    Q = synth.x_fp16(5, HQ, D).reshape(1, HQ, D)
    if kv == qgemm.KV_FP8:
        Kc = oracle.f64_to_e4m3(synth.x_fp16(6, HKV, D).astype(np.float64)).reshape(1, HKV, D)
        Vc = np.tile(np.arange(256, dtype=np.uint8), (HKV, 1))[None]
        Vv = oracle.e4m3_to_f64(Vc)
    else:
        Kc = synth.x_fp16(6, HKV, D).reshape(1, HKV, D)
        Vc = synth.x_fp16(7, HKV, D).reshape(1, HKV, D)
        Vv = Vc.astype(np.float64)
    (O,), _ = _run([(Q, Kc, Vc, None, None)], kv)
    for h in range(HQ):
        want = Vv[0, h // qgemm.ATTN_GROUP]
        got = O[0, h].astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(want))
        assert np.array_equal(got[~np.isnan(want)], want[~np.isnan(want)])
