"""Seeded random shapes through the sweep, against the oracle (GPU).

Each single-job case draws, from its own seed, a format, N (mostly not a
multiple of 16), K (one group up to 2048), M (1..64), padded row strides and
a path the panel height allows; the sweep must meet the stated tolerance on
every column.  Each multi-job case draws a whole launch (up to 20 jobs of
mixed formats, shapes and panel heights, some sharing one X) and checks
every job.  The draws are printed before each GPU step."""
import numpy as np
import pytest

from oracle import oracle
from self_speculative_verify_amd import qgemm
from synth import synth, workloads

from gpu_util import Sweep, device, packed_dev, say, x_dev, y_dev

pytestmark = pytest.mark.gpu

FMTS = [qgemm.FMT_Q4, qgemm.FMT_Q5, qgemm.FMT_Q4_G64, qgemm.FMT_Q4_ZP]
MAX_WORK = 60e6  # N * K * M per job, so the oracle stays quick


def _draw_job(rng, M=None):
    while True:
        fmt = FMTS[int(rng.integers(0, 4))]
        g = 64 if fmt == qgemm.FMT_Q4_G64 else 32
        N = int(rng.integers(1, 2500))
        K = g * int(rng.integers(1, 2048 // g + 1))
        m = int(rng.integers(1, 65)) if M is None else M
        if N * K * m <= MAX_WORK:
            return fmt, N, K, m


def _job(seed, fmt, N, K, M, X=None, ldx=None, ldy=None):
    W = synth.weights(seed, K, 0, N, workloads.SIGMA, outlier_thresh=workloads.OUTLIER_THRESH)
    ref = oracle.quantize_pack(W, fmt)
    p = packed_dev(ref)
    if X is None:
        Xh = synth.x_fp16(seed + 1, M, K)
        X = (Xh, x_dev(Xh, ldx))
    Y = y_dev(M, N, ldy)
    return dict(ref=ref, p=p, fmt=fmt, N=N, K=K, M=M, X=X, Y=Y,
                job=qgemm.make_job(p, fmt, N, K, X[1], Y, M))


def _check(j, what):
    Y = j["Y"][:, :j["N"]].cpu().numpy()
    Xh = j["X"][0]
    Yref = oracle.sweep(j["ref"], j["N"], j["K"], j["fmt"], Xh)
    res = oracle.compare(Y, Yref, Xh, oracle.max_scale(j["ref"], j["N"], j["K"], j["fmt"]))
    assert res["ok"], (what, res)


@pytest.mark.parametrize("seed", range(40))
def test_random_single_job(seed):
    import torch

    rng = np.random.Generator(np.random.PCG64(7000 + seed))
    fmt, N, K, M = _draw_job(rng)
    paths = [qgemm.PATH_AUTO, qgemm.PATH_MFMA] + ([qgemm.PATH_GEMV] if M <= qgemm.GEMV_MAX_M else [])
    path = paths[int(rng.integers(0, len(paths)))]
    ldx = K + 8 * int(rng.integers(0, 3))
    ldy = (N + 3) // 4 * 4 + 4 * int(rng.integers(0, 3))
    what = f"seed={seed} fmt={fmt:#x} N={N} K={K} M={M} path={path} ldx={ldx} ldy={ldy}"
    say(what)
    j = _job(9000 + seed, fmt, N, K, M, ldx=ldx, ldy=ldy)
    Sweep([j["job"]], path)()
    torch.cuda.synchronize()
    _check(j, what)


@pytest.mark.parametrize("seed", range(6))
def test_random_launch(seed):
    import torch

    rng = np.random.Generator(np.random.PCG64(8000 + seed))
    njobs = int(rng.integers(2, 21))
    jobs = []
    shared = {}
    for i in range(njobs):
        fmt, N, K, M = _draw_job(rng)
        if rng.integers(0, 3) == 0 and shared:
            # reuse an X panel of a previous job (inputs may be shared)
            (K, M), X = next(iter(shared.items()))
            g = 64 if fmt == qgemm.FMT_Q4_G64 else 32
            if K % g:
                fmt = qgemm.FMT_Q4
            N = max(1, min(N, int(MAX_WORK // (K * M))))
            jobs.append(_job(100 * seed + i, fmt, N, K, M, X=X))
        else:
            jobs.append(_job(100 * seed + i, fmt, N, K, M))
            shared.setdefault((K, M), jobs[-1]["X"])
    desc = [(hex(j["fmt"]), j["N"], j["K"], j["M"]) for j in jobs]
    say(f"launch seed={seed} jobs={desc}")
    Sweep([j["job"] for j in jobs], qgemm.PATH_AUTO)()
    torch.cuda.synchronize()
    for i, j in enumerate(jobs):
        _check(j, f"launch seed={seed} job {i} {desc[i]}")
