"""The allocation-free sweep (qgemm_sweep_noalloc) on the GPU, through the C
boundary: on calls in a row that share the library's static scratch, its
outputs are bitwise those of qgemm_sweep_path with a workspace of its own --
a set with a launch of more than 12 jobs (its job table copied into the
scratch), then a smaller set, then the first again."""
import numpy as np
import pytest

from self_speculative_verify_amd import qgemm
from synth import synth

from gpu_util import Sweep, device, say, to_dev, x_dev, y_dev

pytestmark = pytest.mark.gpu


def _jobs(specs, seed):
    """specs: (format, N, K, M) per job -> (jobs, Y) twice over the same
    weights and X: one set of outputs per entry point."""
    out = ([], [], [], [])
    keep = []
    for i, (fmt, N, K, M) in enumerate(specs):
        W = synth.weights(seed + i, K, 0, N, 0.02)
        packed = qgemm.pack(to_dev(W), fmt)
        X = x_dev(synth.x_fp16(seed + 100 + i, M, K))
        keep += [packed, X]
        for jobs, ys in ((out[0], out[1]), (out[2], out[3])):
            Y = y_dev(M, N)
            ys.append(Y)
            jobs.append(qgemm.make_job(packed, fmt, N, K, X, Y, M))
    return out, keep


def _check(specs, seed, path=qgemm.PATH_AUTO):
    import torch

    device()
    (jobs_a, ys_a, jobs_b, ys_b), _keep = _jobs(specs, seed)
    say(f"noalloc: {len(specs)} jobs, workspace {qgemm.workspace_bytes(jobs_a, path)} bytes")
    assert qgemm.workspace_bytes(jobs_a, path) <= qgemm.NOALLOC_SCRATCH_BYTES
    qgemm.sweep_noalloc(jobs_a, path)
    Sweep(jobs_b, path)()
    torch.cuda.synchronize()
    for (fmt, N, K, M), ya, yb in zip(specs, ys_a, ys_b):
        a = ya[:, :N].cpu().numpy()
        b = yb[:, :N].cpu().numpy()
        assert np.isfinite(b).all(), (fmt, N, K, M)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (fmt, N, K, M)


# 13 verify panels of one class share a stream launch (more than 12 jobs: a
# job table), two 48-row panels a group launch
BIG_SET = ([(4 if i % 2 else 5, 160 + 48 * i, 640 + 128 * (i % 5), 6) for i in range(13)]
           + [(4, 700, 1536, 48), (5, 300, 1312, 48)])
SMALL_SET = [(4, 300, 1312, 1)]


def test_noalloc_matches_workspace_sweep_on_calls_in_a_row():
    _check(BIG_SET, 1)
    _check(SMALL_SET, 2)
    _check(BIG_SET, 3)


def test_noalloc_gemv_path_and_oversize():
    _check([(5, 513, 2080, 3), (4, 97, 4096, 8)], 4, qgemm.PATH_GEMV)
    _check(SMALL_SET, 5, qgemm.PATH_GEMV)
    # a set whose workspace exceeds the scratch is refused, nothing launched
    N, K = 120000, 65536
    jobs = [qgemm.Job((2 + 2 * i) << 32, (20 + i) << 32, (30 + i) << 32, N, K, K, N, M, 4)
            for i, M in enumerate((1, 2, 4, 8, 16))]
    with pytest.raises(qgemm.QgemmError):
        qgemm.sweep_noalloc(jobs, qgemm.PATH_MFMA)
