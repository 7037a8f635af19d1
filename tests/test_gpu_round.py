"""Round replay through the C boundary: a recorded round (per-matrix sweeps in
order, a many-job sweep that needs a job table, then the verify head) is
replayed several times, with fresh panels and eager calls of the same sweeps
and synchronizations between replays; every replay must equal the eager
results bitwise, and the last one also the oracle within the sweep's bound.
"""
import numpy as np
import pytest

from oracle import oracle
from self_speculative_verify_amd import qgemm
from synth import synth, workloads

from gpu_util import device, packed_dev, say, to_dev, x_dev, y_dev

pytestmark = pytest.mark.gpu

FMTS = [qgemm.FMT_Q4, qgemm.FMT_Q5, qgemm.FMT_Q4_G64, qgemm.FMT_Q4_ZP]
LAYER = [("qkv", 704, 512), ("o", 512, 512), ("gate_up", 1504, 512), ("down", 512, 1536)]


class RoundCase:
    def __init__(self, M, layers=3, table_jobs=14):
        import torch

        self.M = M
        self.X = {}
        for K in (512, 1536, 640):
            self.X[K] = x_dev(np.zeros((M, K), np.float16))
        self.mats, self.sweeps, self.keep = [], [], []
        i = 0
        for L in range(layers):
            for name, N, K in LAYER:
                fmt = FMTS[i % 4]
                W = synth.weights(300 + i, K, 0, N, workloads.SIGMA, outlier_thresh=workloads.OUTLIER_THRESH)
                ref = oracle.quantize_pack(W, fmt)
                p, Y = packed_dev(ref), y_dev(M, N)
                job = qgemm.make_job(p, fmt, N, K, self.X[K], Y, M)
                self.sweeps.append(([job], qgemm.PATH_AUTO))
                self.mats.append((f"L{L}.{name}", ref, fmt, N, K, Y))
                self.keep.append(p)
                i += 1
        # one sweep of many small jobs: its job table lives in the workspace
        jobs = []
        for t in range(table_jobs):
            fmt = FMTS[t % 4]
            N, K = 96 + 37 * t, 640
            W = synth.weights(400 + t, K, 0, N, workloads.SIGMA)
            ref = oracle.quantize_pack(W, fmt)
            p, Y = packed_dev(ref), y_dev(M, N)
            jobs.append(qgemm.make_job(p, fmt, N, K, self.X[K], Y, M))
            self.mats.append((f"T{t}", ref, fmt, N, K, Y))
            self.keep.append(p)
        self.sweeps.append((jobs, qgemm.PATH_AUTO))
        # verify head over the last layer's hidden size
        self.NH, self.KH = 3001, 512
        Wh = synth.weights(500, self.KH, 0, self.NH, 0.05)
        self.head_ref = oracle.quantize_pack(Wh, qgemm.FMT_Q4)
        self.head_p = packed_dev(self.head_ref)
        self.head_Y = y_dev(M, self.NH)
        self.head = qgemm.make_head_job(self.head_p, qgemm.FMT_Q4, self.NH, self.KH, self.X[512], M, Y=self.head_Y)
        self.slots = [(6 * s, 5) for s in range(M // 6)]
        self.drafts = torch.zeros(M, dtype=torch.int32, device=device())
        self.argmax = torch.empty(M, dtype=torch.int32, device=device())
        self.accepted = torch.empty(len(self.slots), dtype=torch.int32, device=device())
        # eager workspaces: one per sweep (a workspace's layout follows its jobs)
        self.ws = [qgemm.Workspace(qgemm.workspace_bytes(j, p), device=device()) for j, p in self.sweeps]
        self.vws = qgemm.Workspace(qgemm.verify_workspace_bytes(self.head), device=device())

    def fill(self, seed):
        import torch

        for K, buf in self.X.items():
            buf.copy_(torch.from_numpy(synth.x_fp16(seed + K, self.M, K)).to(device()))
        rng = np.random.Generator(np.random.PCG64(seed))
        d = rng.integers(0, self.NH, self.M).astype(np.int32)
        self.drafts.copy_(torch.from_numpy(d).to(device()))

    def outputs(self):
        import torch

        torch.cuda.synchronize()
        # the columns each job writes (Y rows are padded to a multiple of 4)
        return ([Y[:, :N].cpu().numpy().copy() for _, _, _, N, _, Y in self.mats] +
                [self.head_Y[:, :self.NH].cpu().numpy().copy()],
                self.argmax.cpu().numpy().copy(), self.accepted.cpu().numpy().copy())

    def poison(self):
        for *_, Y in self.mats:
            Y.fill_(float("nan"))
        self.head_Y.fill_(float("nan"))
        self.argmax.fill_(-7)
        self.accepted.fill_(-7)

    def eager(self):
        for (jobs, path), ws in zip(self.sweeps, self.ws):
            qgemm.sweep(jobs, ws, path)
        qgemm.verify_head(self.head, self.drafts, self.slots, self.argmax, self.accepted, self.vws)


@pytest.mark.parametrize("M", [6, 40])
def test_round_replay_matches_eager_and_oracle(M):
    import torch

    say(f"round M={M}")
    c = RoundCase(M)
    sweeps = qgemm.round_sweeps(c.sweeps)
    ws = qgemm.Workspace(qgemm.round_workspace_bytes(sweeps, c.head), device=device())
    r = qgemm.Round(sweeps, ws, c.head, c.drafts, c.slots, c.argmax, c.accepted)
    try:
        # kernels per replay: one per sweep (single class each), two for the head
        assert r.kernels == len(c.sweeps) + 2
        for rep in range(3):
            c.fill(1000 * rep + M)
            c.poison()
            c.eager()
            want = c.outputs()
            c.poison()
            r.launch()
            got = c.outputs()
            say(f"  replay {rep}: accepted {got[2].tolist()}")
            for a, b in zip(got[0], want[0]):
                assert np.isfinite(b).all() and np.array_equal(a, b)
            assert np.array_equal(got[1], want[1]) and np.array_equal(got[2], want[2])
        # the last replay against the oracle
        for idx in range(0, len(c.mats), 5):
            name, ref, fmt, N, K, _ = c.mats[idx]
            X = c.X[K].cpu().numpy()
            Yref = oracle.sweep(ref, N, K, fmt, X)
            res = oracle.compare(got[0][idx], Yref, X, oracle.max_scale(ref, N, K, fmt))
            assert res["ok"], (name, res)
        Yh = got[0][-1]
        assert np.array_equal(got[1], oracle.argmax_rows(Yh))
        assert got[2].tolist() == oracle.accept(got[1], c.drafts.cpu().numpy(), c.slots)
    finally:
        torch.cuda.synchronize()
        r.destroy()


def test_round_without_head_and_two_rounds_share_nothing():
    import torch

    c = RoundCase(8, layers=1, table_jobs=13)
    sw1 = qgemm.round_sweeps(c.sweeps[:2])
    sw2 = qgemm.round_sweeps(c.sweeps[2:])
    w1 = qgemm.Workspace(qgemm.round_workspace_bytes(sw1), device=device())
    w2 = qgemm.Workspace(qgemm.round_workspace_bytes(sw2), device=device())
    r1, r2 = qgemm.Round(sw1, w1), qgemm.Round(sw2, w2)
    try:
        c.fill(77)
        c.poison()
        c.eager()
        want = c.outputs()
        c.poison()
        r1.launch()
        r2.launch()
        r1.launch()
        got = c.outputs()
        for a, b, (name, *_) in zip(got[0][:-1], want[0][:-1], c.mats):
            assert np.array_equal(a, b), name
    finally:
        torch.cuda.synchronize()
        r1.destroy()
        r2.destroy()


def test_round_cache_replays_records_and_evicts():
    """Three round descriptions through a cache of two: the first two layer
    sweeps, the rest, and the whole round with the verify head.  Every run,
    hit or miss, must equal the eager calls of the same sweeps bitwise on
    fresh panels; hits, misses and least-recently-used evictions follow the
    sequence."""
    import torch

    c = RoundCase(6, layers=1, table_jobs=13)
    keys = [c.sweeps[:2], c.sweeps[2:], c.sweeps]
    nm = len(c.mats)
    mats_of = [range(0, 2), range(2, nm), range(0, nm)]
    cache = qgemm.RoundCache(2)
    seq = [0, 0, 1, 0, 2, 1, 0, 2, 2]
    want_hit = [False, True, False, True, False, False, False, False, True]
    try:
        for t, (k, wh) in enumerate(zip(seq, want_hit)):
            c.fill(500 + 7 * t)
            c.poison()
            c.eager()
            want = c.outputs()
            c.poison()
            head = k == 2
            hit = cache.run(keys[k], c.head if head else None, c.drafts if head else None, c.slots if head else (),
                            c.argmax if head else None, c.accepted if head else None)
            got = c.outputs()
            say(f"  run {t}: key {k} hit={hit}")
            assert hit == wh, (t, k, hit)
            for i in mats_of[k]:
                assert np.isfinite(want[0][i]).all() and np.array_equal(got[0][i], want[0][i]), (t, c.mats[i][0])
            if head:
                assert np.array_equal(got[0][-1], want[0][-1])
                assert np.array_equal(got[1], want[1]) and np.array_equal(got[2], want[2])
        st = cache.stats()
        assert st == {"size": 2, "hits": 3, "misses": 6, "evictions": 4}, st
    finally:
        torch.cuda.synchronize()
        cache.destroy()
