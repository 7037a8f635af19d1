"""Helpers shared by the GPU tests (device buffers through torch, sweeps
through the C boundary).  Nothing here computes expected values."""
import sys

import numpy as np
import pytest

from self_speculative_verify_amd import qgemm


def device():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def x_dev(X: np.ndarray, ldx: int | None = None):
    """fp16 [M, K] host panel -> device fp16 tensor with row stride ldx."""
    import torch

    M, K = X.shape
    ldx = ldx or K
    buf = torch.zeros((M, ldx), dtype=torch.float16, device=device())
    buf[:, :K] = torch.from_numpy(np.ascontiguousarray(X)).to(device())
    return buf


def y_dev(M: int, N: int, ldy: int | None = None):
    """fp32 [M, ldy] output poisoned with NaN, so a kernel that did not run fails."""
    import torch

    return torch.full((M, ldy or (N + 3) // 4 * 4), float("nan"), dtype=torch.float32,
                      device=device())


def packed_dev(packed_host: np.ndarray):
    return to_dev(packed_host)


class Sweep:
    """A set of jobs with its workspace, run through qgemm_sweep_path."""

    def __init__(self, jobs, path=qgemm.PATH_AUTO):
        self.jobs = jobs
        self.path = path
        self.ws = qgemm.Workspace(qgemm.workspace_bytes(jobs, path), device=device())

    def __call__(self):
        qgemm.sweep(self.jobs, self.ws, self.path)


def run_one(packed, bits, N, K, X, M, path=qgemm.PATH_AUTO, ldx=None, ldy=None):
    import torch

    Xd = x_dev(X, ldx)
    Y = y_dev(M, N, ldy or (N + 3) // 4 * 4)
    job = qgemm.make_job(packed, bits, N, K, Xd, Y, M)
    Sweep([job], path)()
    torch.cuda.synchronize()
    return Y[:, :N].cpu().numpy()
