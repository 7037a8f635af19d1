"""GPU parity of the format variants (group-64 symmetric and group-32
zero-point 4-bit) against the CPU oracle, through the C boundary.

Pack bytes are bit-exact; one-hot and integer-exact sweeps are bitwise on
every path and panel class (stream GEMV, stream MFMA, group MFMA); sweeps of
random weights meet the same tolerance as the 4/5-bit formats; a sweep that
mixes all four formats in one launch matches the oracle job by job.
"""
import numpy as np
import pytest

from oracle import oracle
from self_speculative_verify_amd import qgemm
from synth import synth, workloads

from gpu_util import Sweep, device, packed_dev, run_one, say, to_dev, x_dev, y_dev

pytestmark = pytest.mark.gpu

G64, ZP = qgemm.FMT_Q4_G64, qgemm.FMT_Q4_ZP
FMTS = [G64, ZP]


def _weights(seed, N, K, outliers=False, sigma=workloads.SIGMA, shift=0.0):
    W = synth.weights(seed, K, 0, N, sigma, outlier_thresh=workloads.OUTLIER_THRESH if outliers else 0)
    return (W + np.float32(shift)) if shift else W


def _check(Y, Yref, X, smax, what):
    res = oracle.compare(Y, Yref, X, smax)
    say(f"  {what}: rel_l2={res['rel_l2']:.3e} max_abs/bound={res['max_abs_ratio']:.3f}")
    assert res["ok"], f"{what}: {res}"


PACK_CASES = [(1024, 1024, False, 0.0), (34816, 5120, False, 0.0), (5120, 17408, True, 0.0),
              (1, 64, False, 0.0), (17, 192, True, 0.0), (33, 448, True, 0.01), (100, 320, False, -0.02)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,outl,shift", PACK_CASES)
def test_pack_bytes_match_oracle(fmt, N, K, outl, shift):
    say(f"pack fmt={fmt:#x} N={N} K={K} outliers={outl} shift={shift}")
    W = _weights(7 * N + K, N, K, outl, shift=shift)
    got = qgemm.pack(to_dev(W), fmt).cpu().numpy()
    want = oracle.quantize_pack(W, fmt)
    assert got.size == want.size
    assert np.array_equal(got, want)


def test_pack_zero_point_extremes():
    # all-positive, all-negative, all-zero and tiny groups
    N, K = 16, 256
    rng = np.random.Generator(np.random.PCG64(5))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0] = np.abs(W[0])
    W[1] = -np.abs(W[1])
    W[2] = 0.0
    W[3] = 1e-9
    W[4, ::2] = 0.0
    got = qgemm.pack(to_dev(W), ZP).cpu().numpy()
    assert np.array_equal(got, oracle.quantize_pack(W, ZP))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path,M", [(qgemm.PATH_GEMV, 8), (qgemm.PATH_MFMA, 5), (qgemm.PATH_MFMA, 64)])
def test_one_hot_extracts_dequant_bitwise(fmt, path, M):
    say(f"one-hot fmt={fmt:#x} path={path} M={M}")
    N, K = 40, 384
    W = _weights(11 + fmt, N, K, True)
    ref_packed = oracle.quantize_pack(W, fmt)
    what = oracle.dequant(ref_packed, N, K, fmt)
    for k0 in range(0, K, M):
        X = np.zeros((M, K), dtype=np.float16)
        ks = np.arange(k0, min(K, k0 + M))
        X[np.arange(ks.size), ks] = 1.0
        Y = run_one(packed_dev(ref_packed), fmt, N, K, X, M, path)
        assert np.array_equal(Y[:ks.size], what[:, ks].T.astype(np.float32))


def _integer_case(fmt, N, K, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    gs = oracle.group_size(fmt)
    e = rng.integers(-8, 3, (N, K // gs))
    sb = np.ldexp(1.0, e).astype(np.float16).view(np.uint16)
    if fmt == ZP:
        u = rng.integers(0, 16, (N, K)).astype(np.int8)
        zs = rng.integers(0, 16, (N, K // 32)).astype(np.uint8)
        return oracle.pack(u, sb, fmt, zs)
    return oracle.pack(rng.integers(-8, 8, (N, K)).astype(np.int8), sb, fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path,M", [(qgemm.PATH_GEMV, 1), (qgemm.PATH_GEMV, 3), (qgemm.PATH_GEMV, 8),
                                    (qgemm.PATH_MFMA, 1), (qgemm.PATH_MFMA, 6), (qgemm.PATH_MFMA, 16),
                                    (qgemm.PATH_MFMA, 17), (qgemm.PATH_MFMA, 48), (qgemm.PATH_MFMA, 64)])
def test_integer_exact_sweep_bitwise(fmt, path, M):
    say(f"integer-exact fmt={fmt:#x} path={path} M={M}")
    N, K = 300, 1344 if fmt == G64 else 1312
    ref_packed = _integer_case(fmt, N, K, fmt + M)
    X = np.random.Generator(np.random.PCG64(M)).integers(-4, 5, (M, K)).astype(np.float16)
    Yref = oracle.sweep(ref_packed, N, K, fmt, X)
    Y = run_one(packed_dev(ref_packed), fmt, N, K, X, M, path)
    assert np.array_equal(Y, Yref.astype(np.float32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 6, 48])
def test_random_weights_parity(fmt, M):
    """Gate+up-sized rows over a ragged N, every path that takes M."""
    import torch

    say(f"random fmt={fmt:#x} M={M}")
    N, K = 4099, 5120
    W = _weights(21 + M, N, K, True)
    packed = qgemm.pack(to_dev(W), fmt)
    ref_packed = oracle.quantize_pack(W, fmt)
    assert np.array_equal(packed.cpu().numpy(), ref_packed)
    X = synth.x_fp16(22 + M, M, K)
    Yref = oracle.sweep(ref_packed, N, K, fmt, X)
    smax = oracle.max_scale(ref_packed, N, K, fmt)
    paths = [qgemm.PATH_AUTO] + ([qgemm.PATH_GEMV] if M <= qgemm.GEMV_MAX_M else [])
    for path in paths:
        Y = run_one(packed, fmt, N, K, X, M, path)
        _check(Y, Yref, X, smax, f"fmt={fmt:#x} M={M} path={path}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", FMTS)
def test_m_invariance_bitwise(fmt):
    say(f"M-invariance fmt={fmt:#x}")
    N, K = 257, 5120
    W = _weights(31, N, K)
    packed = packed_dev(oracle.quantize_pack(W, fmt))
    X = synth.x_fp16(32, 64, K)
    for Ms in ([16, 1, 2, 5, 8], [64, 17, 33, 48]):
        ref = run_one(packed, fmt, N, K, X[:Ms[0]], Ms[0], qgemm.PATH_MFMA)
        for M in Ms[1:]:
            assert np.array_equal(run_one(packed, fmt, N, K, X[:M], M, qgemm.PATH_MFMA), ref[:M])
        rev = run_one(packed, fmt, N, K, X[:Ms[0]][::-1].copy(), Ms[0], qgemm.PATH_MFMA)
        assert np.array_equal(rev, ref[::-1])


@pytest.mark.parametrize("M,njobs", [(1, 4), (6, 4), (40, 4), (6, 14), (40, 14)])
def test_mixed_formats_one_launch(M, njobs):
    """All four formats in one sweep (inline jobs, and a job table)."""
    import torch

    say(f"mixed formats M={M} njobs={njobs}")
    fmts = [qgemm.FMT_Q4, G64, ZP, qgemm.FMT_Q5]
    shapes = [(700, 1024), (300, 2048), (1100, 640), (129, 1536)]
    jobs, keep, refs = [], [], []
    for i in range(njobs):
        fmt = fmts[i % 4]
        N, K = shapes[(i // 4 + i) % 4]
        W = _weights(100 + i, N, K, i % 3 == 0)
        ref_packed = oracle.quantize_pack(W, fmt)
        X = synth.x_fp16(200 + i, M, K)
        packed, Xd, Y = packed_dev(ref_packed), x_dev(X), y_dev(M, N)
        jobs.append(qgemm.make_job(packed, fmt, N, K, Xd, Y, M))
        keep.append((packed, Xd, Y))
        refs.append((ref_packed, fmt, N, K, X))
    Sweep(jobs)()
    torch.cuda.synchronize()
    for (ref_packed, fmt, N, K, X), (_, _, Y) in zip(refs, keep):
        Yref = oracle.sweep(ref_packed, N, K, fmt, X)
        _check(Y[:, :N].cpu().numpy(), Yref, X, oracle.max_scale(ref_packed, N, K, fmt), f"fmt={fmt:#x} {N}x{K}")


def test_classic_rows_unchanged_by_a_variant_job():
    """A 4-bit job's rows are bitwise the same whether its launch partner is
    another 4-bit job or a zero-point job of the same shape (equal step
    weights, so the same K split; the second launch takes the all-format
    kernel)."""
    import torch

    N, K, M = 2000, 5120, 6
    W = _weights(41, N, K)
    X = synth.x_fp16(42, M, K)
    p4 = packed_dev(oracle.quantize_pack(W, qgemm.FMT_Q4))
    pz = packed_dev(oracle.quantize_pack(W, ZP))
    Xd = x_dev(X)
    Ya, Yb, Yc, Yz = (y_dev(M, N) for _ in range(4))
    Sweep([qgemm.make_job(p4, qgemm.FMT_Q4, N, K, Xd, Ya, M), qgemm.make_job(p4, qgemm.FMT_Q4, N, K, Xd, Yb, M)])()
    Sweep([qgemm.make_job(p4, qgemm.FMT_Q4, N, K, Xd, Yc, M), qgemm.make_job(pz, ZP, N, K, Xd, Yz, M)])()
    torch.cuda.synchronize()
    assert np.array_equal(Ya.cpu().numpy(), Yc.cpu().numpy())
    assert np.isfinite(Ya.cpu().numpy()[:, :N]).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_verify_head_on_variant(fmt):
    import torch

    say(f"verify head fmt={fmt:#x}")
    N, K, M = 3001, 1024, 12
    W = _weights(51, N, K, sigma=0.05)
    ref_packed = oracle.quantize_pack(W, fmt)
    X = synth.x_fp16(52, M, K)
    Yref = oracle.sweep(ref_packed, N, K, fmt, X)
    am_ref = oracle.argmax_rows(Yref)
    drafts = np.array(am_ref, dtype=np.int32)
    drafts[3] += 1            # slot 0 rejects its fourth draft
    slots = [(0, 5), (6, 5)]
    packed, Xd = packed_dev(ref_packed), x_dev(X)
    Y = y_dev(M, N)
    head = qgemm.make_head_job(packed, fmt, N, K, Xd, M, Y=Y)
    ws = qgemm.Workspace(qgemm.verify_workspace_bytes(head), device=device())
    am = torch.empty(M, dtype=torch.int32, device=device())
    acc = torch.empty(len(slots), dtype=torch.int32, device=device())
    qgemm.verify_head(head, to_dev(drafts), slots, am, acc, ws)
    torch.cuda.synchronize()
    Yg = Y[:, :N].cpu().numpy()
    _check(Yg, Yref, X, oracle.max_scale(ref_packed, N, K, fmt), "logits")
    assert np.array_equal(am.cpu().numpy(), oracle.argmax_rows(Yg))
    assert acc.cpu().numpy().tolist() == oracle.accept(am.cpu().numpy(), drafts, slots)


EDGE = [
    (G64, 1, 64, 1), (G64, 1, 64, 64), (G64, 17, 192, 3), (G64, 33, 448, 17), (G64, 129, 4160, 2),
    (G64, 1000, 1088, 33), (ZP, 1, 32, 1), (ZP, 1, 32, 64), (ZP, 17, 96, 3), (ZP, 33, 416, 17),
    (ZP, 15, 160, 7), (ZP, 31, 17408, 64), (ZP, 64, 128, 48),
]


@pytest.mark.parametrize("fmt,N,K,M", EDGE)
def test_edge_shapes(fmt, N, K, M):
    """Single rows and groups, ragged tiles and padded strides on every path."""
    say(f"edge fmt={fmt:#x} N={N} K={K} M={M}")
    W = _weights(N * 7 + K + fmt, N, K, True, shift=0.005)
    ref_packed = oracle.quantize_pack(W, fmt)
    packed = packed_dev(ref_packed)
    X = synth.x_fp16(N + K + M, M, K)
    Yref = oracle.sweep(ref_packed, N, K, fmt, X)
    smax = oracle.max_scale(ref_packed, N, K, fmt)
    paths = [qgemm.PATH_AUTO, qgemm.PATH_MFMA] + ([qgemm.PATH_GEMV] if M <= 8 else [])
    for path in paths:
        Y = run_one(packed, fmt, N, K, X, M, path, ldx=K + 24, ldy=N + (4 - N % 4) % 4 + 8)
        _check(Y, Yref, X, smax, f"path={path}")
