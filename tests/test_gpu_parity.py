"""GPU parity: the HIP library against the CPU oracle through the C boundary.

Sizes here are the small and medium workloads in full (1: 1024 x 1024 4-bit
M=1; 2: 34816 x 5120 4-bit M=1; 3: that plus 5120 x 17408 5-bit at M=6) and
edge shapes that span several tiles and ragged tails.  The 64-layer stacks at
full size are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest

from oracle import oracle
from self_speculative_verify_amd import qgemm
from synth import synth, workloads

from gpu_util import Sweep, device, packed_dev, run_one, say, to_dev, x_dev, y_dev

pytestmark = pytest.mark.gpu


def _weights(seed, N, K, outliers=False, sigma=workloads.SIGMA):
    return synth.weights(seed, K, 0, N, sigma,
                         outlier_thresh=workloads.OUTLIER_THRESH if outliers else 0)


# --------------------------------------------------------------------------
# pack: bytes identical to the oracle's pack
# --------------------------------------------------------------------------
PACK_CASES = [
    (4, 1024, 1024, False), (4, 34816, 5120, False), (5, 5120, 17408, False),
    (4, 1, 32, False), (5, 17, 96, True), (4, 33, 416, True), (5, 100, 160, True),
    (5, 7168, 5120, True),
]


@pytest.mark.parametrize("bits,N,K,outl", PACK_CASES)
def test_pack_bytes_match_oracle(bits, N, K, outl):
    import torch

    say(f"pack bits={bits} N={N} K={K} outliers={outl}")
    W = _weights(1000 + N + K, N, K, outl)
    got = qgemm.pack(to_dev(W), bits)
    torch.cuda.synchronize()
    want = oracle.quantize_pack(W, bits)
    g = got.cpu().numpy()
    assert g.size == want.size
    if not np.array_equal(g, want):
        bad = np.flatnonzero(g != want)
        pytest.fail(f"{bad.size} bytes differ, first at {bad[:8]}")


def test_pack_strided_input_and_extremes():
    import torch

    say("pack strided + extremes")
    N, K, ldw = 40, 256, 300
    W = _weights(5, N, K, True, sigma=3.0)
    W[0, :32] = 0.0                                  # amax = 0
    W[1, 32:64] = 1e-9                               # scale underflows to 0
    W[2, 64:96] = 1e-6                               # fp16-subnormal scales
    W[3, :32] = 7 * 65504.0                          # largest finite scale
    buf = np.zeros((N, ldw), dtype=np.float32)
    buf[:, :K] = W
    dev = to_dev(buf)
    for bits in (4, 5):
        got = torch.empty(qgemm.packed_bytes(bits, N, K), dtype=torch.uint8, device=device())
        from ctypes import c_void_p
        st = qgemm.lib().qgemm_pack(dev.data_ptr(), ldw, N, K, bits, got.data_ptr(), None)
        assert st == qgemm.OK
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), oracle.quantize_pack(W, bits))


def test_pack_reports_nonfinite():
    say("pack non-finite")
    for bad in (np.nan, np.inf, 7 * 65520.0):
        W = _weights(6, 20, 64)
        W[3, 9] = bad
        with pytest.raises(qgemm.QgemmError) as e:
            qgemm.pack(to_dev(W), 4)
        assert e.value.status == qgemm.ERR_NONFINITE


# --------------------------------------------------------------------------
# sweeps of workloads 1-3 in full
# --------------------------------------------------------------------------
def _check(Y, Yref, X, smax, what):
    res = oracle.compare(Y, Yref, X, smax)
    say(f"  {what}: rel_l2={res['rel_l2']:.3e} max_abs/bound={res['max_abs_ratio']:.3f}")
    assert res["ok"], f"{what}: {res}"


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_workload_parity(cfg):
    import torch

    wl = workloads.workload(cfg)
    M = wl.Ms[0]
    say(f"workload {cfg}: {wl.name}")
    jobs, refs, keep = [], [], []
    Xs = {K: synth.x_fp16(wl.x_seed(K), M, K) for K in wl.distinct_K}
    Xd = {K: x_dev(X) for K, X in Xs.items()}
    for m in wl.matrices:
        W = _weights(m.seed, m.N, m.K, m.outliers)
        packed = qgemm.pack(to_dev(W), m.bits)
        ref_packed = oracle.quantize_pack(W, m.bits)
        assert np.array_equal(packed.cpu().numpy(), ref_packed), f"{m.name} pack bytes"
        Y = y_dev(M, m.N)
        jobs.append(qgemm.make_job(packed, m.bits, m.N, m.K, Xd[m.K], Y, M))
        keep.append((packed, Y))
        refs.append((m, ref_packed))
        del W
    paths = [qgemm.PATH_AUTO, qgemm.PATH_MFMA] + ([qgemm.PATH_GEMV] if M <= 8 else [])
    results = {}
    for path in paths:
        for _, Y in keep:
            Y.fill_(float("nan"))
        Sweep(jobs, path)()
        torch.cuda.synchronize()
        results[path] = [Y.cpu().numpy() for _, Y in keep]
    for i, (m, ref_packed) in enumerate(refs):
        Yref = oracle.sweep(ref_packed, m.N, m.K, m.bits, Xs[m.K])
        smax = oracle.max_scale(ref_packed, m.N, m.K, m.bits)
        for path in paths:
            _check(results[path][i], Yref, Xs[m.K], smax, f"{m.name} path={path}")
    if qgemm.auto_path(M) == qgemm.PATH_GEMV:
        assert all(np.array_equal(a, b) for a, b in zip(results[0], results[qgemm.PATH_GEMV]))
    else:
        assert all(np.array_equal(a, b) for a, b in zip(results[0], results[qgemm.PATH_MFMA]))


# --------------------------------------------------------------------------
# bit-exact checks: one-hot extraction, integer-exact sweeps
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("path,M", [(qgemm.PATH_GEMV, 8), (qgemm.PATH_MFMA, 64), (qgemm.PATH_MFMA, 5)])
def test_one_hot_extracts_dequant_bitwise(bits, path, M):
    say(f"one-hot bits={bits} path={path} M={M}")
    N, K = 80, 544
    W = _weights(77, N, K, True)
    ref_packed = oracle.quantize_pack(W, bits)
    what = oracle.dequant(ref_packed, N, K, bits)
    ks = np.random.Generator(np.random.PCG64(M)).choice(K, M, replace=False)
    X = np.zeros((M, K), dtype=np.float16)
    X[np.arange(M), ks] = 1.0
    Y = run_one(packed_dev(ref_packed), bits, N, K, X, M, path)
    assert np.array_equal(Y.astype(np.float64), what[:, ks].T)


@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("path,M", [(qgemm.PATH_GEMV, 1), (qgemm.PATH_GEMV, 3), (qgemm.PATH_GEMV, 8),
                                    (qgemm.PATH_MFMA, 1), (qgemm.PATH_MFMA, 16), (qgemm.PATH_MFMA, 40),
                                    (qgemm.PATH_MFMA, 64)])
def test_integer_exact_sweep_bitwise(bits, path, M):
    """Integer X and power-of-two scales: every partial sum is exact in fp32."""
    say(f"integer-exact bits={bits} path={path} M={M}")
    N, K = 300, 5120
    rng = np.random.Generator(np.random.PCG64(bits * 100 + M))
    qmax = (1 << (bits - 1)) - 1
    codes = rng.integers(-qmax, qmax + 1, (N, K)).astype(np.int8)
    e = rng.integers(-10, 2, (N, K // 32))
    scales = np.ldexp(1.0, e).astype(np.float16).view(np.uint16)
    ref_packed = oracle.pack(codes, scales, bits)
    X = rng.integers(-4, 5, (M, K)).astype(np.float16)
    Yref = oracle.sweep(ref_packed, N, K, bits, X)
    Y = run_one(packed_dev(ref_packed), bits, N, K, X, M, path)
    assert np.array_equal(Y.astype(np.float64), Yref)


# --------------------------------------------------------------------------
# M-invariance, repeatability, path agreement
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 5])
def test_m_invariance_bitwise(bits):
    """Row m is bitwise independent of M and of the other rows within a panel
    class (GEMV M <= 8; MFMA M <= 16; MFMA 17..64), and within tolerance
    across the two MFMA classes."""
    say(f"M-invariance bits={bits}")
    N, K = 257, 17408 if bits == 5 else 5120
    W = _weights(91, N, K, True)
    ref_packed = oracle.quantize_pack(W, bits)
    packed = packed_dev(ref_packed)
    X = synth.x_fp16(92, 64, K)
    classes = ((qgemm.PATH_MFMA, [64, 48, 33, 17]), (qgemm.PATH_MFMA, [16, 9, 5, 1]),
               (qgemm.PATH_GEMV, [8, 5, 4, 2, 1]))
    full = {}
    for path, Ms in classes:
        ref = run_one(packed, bits, N, K, X[:Ms[0]], Ms[0], path)
        full[(path, Ms[0])] = ref
        for M in Ms[1:]:
            part = run_one(packed, bits, N, K, X[:M], M, path)
            assert np.array_equal(part, ref[:M]), f"path={path} M={M}"
        # rows moved to other positions give the same bits
        rev = run_one(packed, bits, N, K, X[:Ms[0]][::-1].copy(), Ms[0], path)
        assert np.array_equal(rev[::-1], ref), f"path={path} permuted rows"
    a, b = full[(qgemm.PATH_MFMA, 64)][:16], full[(qgemm.PATH_MFMA, 16)]
    Yref = oracle.sweep(ref_packed, N, K, bits, X[:16])
    smax = oracle.max_scale(ref_packed, N, K, bits)
    _check(a, Yref, X[:16], smax, "group class")
    _check(b, Yref, X[:16], smax, "stream class")


def test_repeat_determinism_and_path_agreement():
    say("determinism")
    N, K, bits = 4099, 5120, 4
    W = _weights(93, N, K, True)
    ref_packed = oracle.quantize_pack(W, bits)
    packed = packed_dev(ref_packed)
    smax = oracle.max_scale(ref_packed, N, K, bits)
    for M in range(1, 9):
        X = synth.x_fp16(94 + M, M, K)
        g1 = run_one(packed, bits, N, K, X, M, qgemm.PATH_GEMV)
        g2 = run_one(packed, bits, N, K, X, M, qgemm.PATH_GEMV)
        m1 = run_one(packed, bits, N, K, X, M, qgemm.PATH_MFMA)
        m2 = run_one(packed, bits, N, K, X, M, qgemm.PATH_MFMA)
        assert np.array_equal(g1, g2) and np.array_equal(m1, m2)
        Yref = oracle.sweep(ref_packed, N, K, bits, X)
        _check(g1, Yref, X, smax, f"gemv M={M}")
        _check(m1, Yref, X, smax, f"mfma M={M}")


# --------------------------------------------------------------------------
# edge shapes: ragged N and K, strides, tiny K, many jobs in one sweep
# --------------------------------------------------------------------------
EDGE = [
    (4, 1, 32, 1), (5, 1, 32, 64), (4, 17, 96, 3), (5, 33, 416, 17), (4, 15, 160, 7),
    (5, 129, 4128, 2), (4, 1000, 1056, 33), (5, 31, 17408, 64), (4, 64, 128, 48),
]


@pytest.mark.parametrize("bits,N,K,M", EDGE)
def test_edge_shapes(bits, N, K, M):
    say(f"edge bits={bits} N={N} K={K} M={M}")
    W = _weights(N * 7 + K, N, K, True)
    ref_packed = oracle.quantize_pack(W, bits)
    packed = packed_dev(ref_packed)
    X = synth.x_fp16(N + K + M, M, K)
    Yref = oracle.sweep(ref_packed, N, K, bits, X)
    smax = oracle.max_scale(ref_packed, N, K, bits)
    paths = [qgemm.PATH_AUTO, qgemm.PATH_MFMA] + ([qgemm.PATH_GEMV] if M <= 8 else [])
    for path in paths:
        Y = run_one(packed, bits, N, K, X, M, path, ldx=K + 24, ldy=N + (4 - N % 4) % 4 + 8)
        _check(Y, Yref, X, smax, f"path={path}")


# A group-kernel launch of more than one round whose last round is partial
# and lies in its one job: that round is cut into units of 8 row blocks on a
# 256-workgroup grid.  At M = 17..48 (16-wave workgroups, 32 row blocks a
# unit) 9000 row blocks are 282 units, the last partial; at M = 49..64
# (8-wave workgroups, 16 row blocks) 4809 row blocks are 301.  N ragged,
# k-tile counts with and without the unit chaining.
RESLICE = [(4, 48, 9000 * 16 - 5, 256), (5, 32, 9000 * 16 - 11, 512), (4, 64, 4809 * 16 - 3, 160)]


@pytest.mark.parametrize("bits,M,N,K", RESLICE)
def test_group_last_round_resliced(bits, M, N, K):
    say(f"resliced last round bits={bits} M={M} N={N} K={K}")
    W = _weights(N + 3 * K + M, N, K, True)
    ref_packed = oracle.quantize_pack(W, bits)
    packed = packed_dev(ref_packed)
    X = synth.x_fp16(N + K + 2 * M, M, K)
    Yref = oracle.sweep(ref_packed, N, K, bits, X)
    smax = oracle.max_scale(ref_packed, N, K, bits)
    Y = run_one(packed, bits, N, K, X, M, qgemm.PATH_AUTO)
    _check(Y, Yref, X, smax, "auto")


def test_many_jobs_one_sweep():
    """More jobs than fit in the kernel arguments, mixed bits, M and shapes."""
    import torch

    say("many jobs")
    rng = np.random.Generator(np.random.PCG64(5))
    jobs, keep, refs = [], [], []
    for i in range(20):
        bits = 4 + i % 2
        N = int(rng.integers(1, 300))
        K = 32 * int(rng.integers(1, 60))
        M = [1, 2, 6, 16, 48, 64][i % 6]
        W = _weights(300 + i, N, K, True)
        ref_packed = oracle.quantize_pack(W, bits)
        X = synth.x_fp16(400 + i, M, K)
        packed, Xd, Y = packed_dev(ref_packed), x_dev(X), y_dev(M, N)
        jobs.append(qgemm.make_job(packed, bits, N, K, Xd, Y, M))
        keep.append((packed, Xd, Y))
        refs.append((ref_packed, bits, N, K, X))
    Sweep(jobs)()
    torch.cuda.synchronize()
    for (ref_packed, bits, N, K, X), (_, _, Y) in zip(refs, keep):
        Yref = oracle.sweep(ref_packed, N, K, bits, X)
        _check(Y[:, :N].cpu().numpy(), Yref, X, oracle.max_scale(ref_packed, N, K, bits),
               f"N={N} K={K}")


def test_workspace_slots_return_to_zero():
    """Every split-K slot a sweep writes is read and cleared by the same
    sweep: after each call the workspace of a one-matrix sweep (slots only)
    is all zero again, so it serves any later set of jobs without a refill."""
    import torch

    say("workspace reuse")
    N, K, bits, M = 34816, 5120, 4, 1
    W = _weights(2_000_000, N, K)
    ref_packed = oracle.quantize_pack(W, bits)
    packed = packed_dev(ref_packed)
    X = synth.x_fp16(7, M, K)
    Xd, Y = x_dev(X), y_dev(M, N)
    job_a = qgemm.make_job(packed, bits, N, K, Xd, Y, M)
    # a second set of different shapes, path and panel height
    N2, K2, bits2, M2 = 5120, 17408, 5, 6
    W2 = _weights(2_000_001, N2, K2)
    ref2 = oracle.quantize_pack(W2, bits2)
    packed2 = packed_dev(ref2)
    X2 = synth.x_fp16(8, M2, K2)
    Xd2, Y2 = x_dev(X2), y_dev(M2, N2)
    job_b = qgemm.make_job(packed2, bits2, N2, K2, Xd2, Y2, M2)
    ws = qgemm.Workspace(max(qgemm.workspace_bytes([job_a]), qgemm.workspace_bytes([job_b]),
                             qgemm.workspace_bytes([job_a], qgemm.PATH_GEMV)), device=device())
    outs = []
    for path in (qgemm.PATH_AUTO, qgemm.PATH_AUTO, qgemm.PATH_GEMV, qgemm.PATH_AUTO):
        Y.fill_(float("nan"))
        qgemm.sweep([job_a], ws, path)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws.buf)) == 0, "slots left non-zero"
        outs.append(Y.cpu().numpy())
        qgemm.sweep([job_b], ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws.buf)) == 0, "slots left non-zero"
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[3])
    Yref = oracle.sweep(ref_packed, N, K, bits, X)
    for o in outs:
        _check(o, Yref, X, oracle.max_scale(ref_packed, N, K, bits), "reuse")
    Yref2 = oracle.sweep(ref2, N2, K2, bits2, X2)
    _check(Y2[:, :N2].cpu().numpy(), Yref2, X2, oracle.max_scale(ref2, N2, K2, bits2), "reuse, second set")
