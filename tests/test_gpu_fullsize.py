"""GPU parity at full size: the 64-layer 27B-class stacks (workload 4: 4-bit,
M = 48; workload 5: 5-bit, M swept over 1..64; workloads 7 and 8: the
group-64 and zero-point 4-bit formats at M = 1, 8, 48), swept in one call over
all 256 matrices exactly as the benchmark launches them.

The weights are generated on the device (Philox twin of the host generator),
packed on the device, and checked on samples the oracle computes one by one:
64 seeded rows of every matrix plus its first and last row (column
independence makes a sampled column exact), packed bytes of the first and
last 16-row block of every matrix, and finiteness of every output.
"""
import numpy as np
import pytest

from oracle import oracle
from self_speculative_verify_amd import qgemm
from synth import synth, workloads

from gpu_util import Sweep, device, say, x_dev, y_dev

pytestmark = pytest.mark.gpu

SAMPLES = 64


class Stack:
    def __init__(self, cfg):
        import torch

        self.wl = workloads.workload(cfg)
        self.packed = []
        self._ref = {}
        maxel = max(m.N * m.K for m in self.wl.matrices)
        tmp = torch.empty(maxel, dtype=torch.float32, device=device())
        for i, m in enumerate(self.wl.matrices):
            w = tmp[: m.N * m.K].view(m.N, m.K)
            synth.weights_gpu(m.seed, m.K, 0, m.N, workloads.SIGMA, w.data_ptr(), m.K,
                              torch.cuda.current_stream().cuda_stream, outlier_thresh=m.thresh,
                              outlier_mult=workloads.OUTLIER_MULT)
            self.packed.append(qgemm.pack(w, m.bits))
            if i % 64 == 63:
                say(f"  packed {i + 1} matrices")
        del tmp
        torch.cuda.synchronize()

    def rows(self, i):
        m = self.wl.matrices[i]
        rng = np.random.Generator(np.random.PCG64(m.seed))
        r = rng.choice(np.arange(1, m.N - 1), SAMPLES, replace=False)
        return np.sort(np.concatenate([[0, m.N - 1], r]))

    def sample_ref(self, i):
        """(rows, oracle-packed sampled rows) of matrix i, cached."""
        if i not in self._ref:
            m = self.wl.matrices[i]
            rows = self.rows(i)
            self._ref[i] = (rows, oracle.quantize_pack(self.host_rows(i, rows), m.bits))
        return self._ref[i]

    def host_rows(self, i, rows):
        m = self.wl.matrices[i]
        return np.concatenate([synth.weights(m.seed, m.K, int(n), 1, workloads.SIGMA,
                                             outlier_thresh=m.thresh,
                                             outlier_mult=workloads.OUTLIER_MULT) for n in rows])


_stacks = {}


def stack(cfg):
    if cfg not in _stacks:
        _stacks.clear()
        say(f"building stack {cfg}")
        _stacks[cfg] = Stack(cfg)
    return _stacks[cfg]


def _sweep_all(st, M, path=qgemm.PATH_AUTO):
    import torch

    X = {K: synth.x_fp16(st.wl.x_seed(K), M, K) for K in st.wl.distinct_K}
    Xd = {K: x_dev(v) for K, v in X.items()}
    Ys, jobs = [], []
    for m, p in zip(st.wl.matrices, st.packed):
        Y = y_dev(M, m.N)
        Ys.append(Y)
        jobs.append(qgemm.make_job(p, m.bits, m.N, m.K, Xd[m.K], Y, M))
    Sweep(jobs, path)()
    torch.cuda.synchronize()
    return X, Ys


def _check_samples(st, M, X, Ys):
    worst = 0.0
    for i, m in enumerate(st.wl.matrices):
        Y = Ys[i]
        assert bool(torch_isfinite_all(Y)), f"{m.name}: non-finite output"
        rows, ref_packed = st.sample_ref(i)
        Yref = oracle.sweep(ref_packed, rows.size, m.K, m.bits, X[m.K])
        import torch

        got = Y[:, torch.from_numpy(rows).to(Y.device)].cpu().numpy()
        res = oracle.compare(got, Yref, X[m.K], oracle.max_scale(ref_packed, rows.size, m.K, m.bits))
        worst = max(worst, res["rel_l2"])
        assert res["ok"], f"{m.name} M={M}: {res}"
    say(f"  M={M}: worst sampled rel_l2 {worst:.3e}")


def torch_isfinite_all(Y):
    import torch

    return torch.isfinite(Y).all().item()


def _check_pack_blocks(st):
    tb = oracle.packed_bytes(st.wl.matrices[0].bits, 16, 128)
    for i, m in enumerate(st.wl.matrices):
        nkt = (m.K + 127) // 128
        nrb = (m.N + 15) // 16
        for rb in (0, nrb - 1):
            W = st.host_rows(i, range(16 * rb, 16 * rb + 16))
            want = oracle.quantize_pack(W, m.bits)
            got = st.packed[i][rb * nkt * tb:(rb + 1) * nkt * tb].cpu().numpy()
            assert np.array_equal(got, want), f"{m.name} row block {rb}"


def test_fullsize_workload4_pack_blocks():
    _check_pack_blocks(stack(4))


def test_fullsize_workload4_m48():
    st = stack(4)
    X, Ys = _sweep_all(st, 48)
    _check_samples(st, 48, X, Ys)


def test_fullsize_workload5_pack_blocks():
    _check_pack_blocks(stack(5))


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 32, 48, 64])
def test_fullsize_workload5(M):
    import torch

    st = stack(5)
    slots = workloads.ragged_slots(M)
    say(f"workload 5 M={M} slots={slots}")
    X, Ys = _sweep_all(st, M)
    _check_samples(st, M, X, Ys)
    if M <= 8:
        # the other path over every column: within twice the tolerance of each other
        other = qgemm.PATH_MFMA if qgemm.auto_path(M) == qgemm.PATH_GEMV else qgemm.PATH_GEMV
        _, Yo = _sweep_all(st, M, other)
        for i, m in enumerate(st.wl.matrices):
            a, b = Ys[i].double(), Yo[i].double()
            rel = (torch.linalg.norm(a - b) / torch.linalg.norm(a)).item()
            assert rel <= 2 * oracle.REL_L2_TOL, f"{m.name}: paths differ rel {rel}"


@pytest.mark.parametrize("cfg", [7, 8])
def test_fullsize_format_stack_pack_blocks(cfg):
    _check_pack_blocks(stack(cfg))


@pytest.mark.parametrize("cfg,M", [(7, 1), (7, 8), (7, 48), (8, 1), (8, 8), (8, 48)])
def test_fullsize_format_stack(cfg, M):
    st = stack(cfg)
    say(f"workload {cfg} M={M}")
    X, Ys = _sweep_all(st, M)
    _check_samples(st, M, X, Ys)
