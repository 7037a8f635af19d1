"""Benchmark of the fused quantized weight sweep on one MI355X.

A step is one qgemm_sweep call over the whole workload (every matrix of it,
one launch), with weights, activations and outputs already resident in HBM.
The headline line is the gate+up projection (34816 x 5120, 4-bit group-32,
M = 1, single-stream decode); the same run times every other workload and
reports it in the same JSON line: the 1024 x 1024 layer (latency), the M = 6
verify workload (gate+up 4-bit + down 5-bit), the 64-layer 27B-class 4-bit
stack at M = 48 (8 slots x 6 tokens) and the 5-bit stack at every M of its
sweep, each with its roofline time (the larger of the HBM and the MFMA
term).  Workloads 2 and 3 also get the read ceiling of their launch (the
same loads with the same geometry and nothing else, libqgemm_ceiling) and
the sweep's fraction of it.  Then the CPU oracle on the same workloads.

Weight GB/s counts code and scale bytes (bits/8 per weight + 2 bytes per 32);
tokens/s per sweep is M / step time.  The workloads that fit in the 256 MB
last-level cache rotate over enough packed copies (>= 1 GB) that every step
streams its weights from HBM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only 1|2|3|4|5|6|7|8|9|10]
       [--no-cpu] [--stack-layers L] [--ceiling] [--timeline]
       python bench.py --copy-calib MIB   (a plain device copy of MIB MiB, the
       reference for scaling the HBM byte counters)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 MFMA, MI355X
PATHS = {"auto": 0, "gemv": 1, "mfma": 2}

# HBM bytes per launch of the headline sweep kernel, from rocprofv3 FETCH_SIZE
# and WRITE_SIZE runs scaled by the same counters on a plain copy (profiles/
# has the commands and raw figures).  Valid only for the kernel sources they
# were taken on: keyed by the SHA-256 of those sources, else reported as null.
TRAFFIC = {
    # FETCH_SIZE 50380.0 KiB x 1.9999 (a 1 GiB device copy reads 524305 KiB)
    # + WRITE_SIZE 4018 KiB x 1.0 (the copy writes 1048576 KiB)
    "42f71eff0fb17887": {"workload": "gate+up 5120->34816 4-bit M=1", "bytes": 107289400},
}
KERNEL_SOURCES = ("self_speculative_verify_amd/csrc/qgemm_kernels.hip",
                  "self_speculative_verify_amd/csrc/qgemm_internal.h",
                  "self_speculative_verify_amd/csrc/qgemm_host.cpp",
                  "self_speculative_verify_amd/csrc/sweep_device.h",
                  "self_speculative_verify_amd/csrc/stream_plan.h",
                  "self_speculative_verify_amd/csrc/stream_impl.h",
                  "self_speculative_verify_amd/csrc/stream_q4.hip")


def kernel_sha():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]
METRIC = "weight GB/s (% of HBM peak) + verify tokens/s per sweep at M=1,6,48"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Bench:
    def __init__(self, cfg, layers=None, rotate_bytes=1 << 30, M=None):
        import torch

        from self_speculative_verify_amd import qgemm
        from synth import synth, workloads

        self.qgemm = qgemm
        self.path = qgemm.PATH_AUTO
        self.wl = workloads.workload(cfg, layers) if layers else workloads.workload(cfg)
        self.M = M if M is not None else self.wl.Ms[0]
        dev = torch.device("cuda:0")
        stream = torch.cuda.current_stream()
        maxel = max(m.N * m.K for m in self.wl.matrices)
        tmp = torch.empty(maxel, dtype=torch.float32, device=dev)
        packed = []
        for m in self.wl.matrices:
            w = tmp[: m.N * m.K].view(m.N, m.K)
            synth.weights_gpu(m.seed, m.K, 0, m.N, workloads.SIGMA, w.data_ptr(), m.K,
                              stream.cuda_stream, outlier_thresh=m.thresh,
                              outlier_mult=workloads.OUTLIER_MULT)
            packed.append(qgemm.pack(w, m.bits))
        del tmp
        self.weight_bytes = sum(workloads.weight_bytes(m.bits, m.N, m.K) for m in self.wl.matrices)
        self.packed_bytes = sum(p.numel() for p in packed)
        copies = max(1, -(-rotate_bytes // self.packed_bytes)) if self.packed_bytes < rotate_bytes else 1
        self.copies = [packed] + [[p.clone() for p in packed] for _ in range(copies - 1)]
        M = self.M
        self.X = {}
        for K in self.wl.distinct_K:
            x = synth.x_fp16(self.wl.x_seed(K), M, K)
            self.X[K] = torch.from_numpy(x).to(dev)
        self.Y = [torch.empty((M, m.N), dtype=torch.float32, device=dev) for m in self.wl.matrices]
        self.jobsets = []
        for cp in self.copies:
            self.jobsets.append([qgemm.make_job(p, m.bits, m.N, m.K, self.X[m.K], y, M)
                                 for p, m, y in zip(cp, self.wl.matrices, self.Y)])
        ws = max(qgemm.workspace_bytes(js) for js in self.jobsets)
        self.ws = qgemm.Workspace(ws, device=dev)
        # the job arrays are marshalled once; each step is one C call
        self.arrays = [qgemm.job_array(js) for js in self.jobsets]
        self.xbytes = sum(2 * M * K for K in self.wl.distinct_K)
        self.ybytes = sum(4 * M * m.N for m in self.wl.matrices)
        torch.cuda.synchronize()

    def set_M(self, M):
        """Re-point every job at fresh X / Y panels of M rows (same weights)."""
        import torch

        from synth import synth

        q = self.qgemm
        dev = torch.device("cuda:0")
        self.M = M
        self.X = {K: torch.from_numpy(synth.x_fp16(self.wl.x_seed(K), M, K)).to(dev)
                  for K in self.wl.distinct_K}
        self.Y = [torch.empty((M, m.N), dtype=torch.float32, device=dev) for m in self.wl.matrices]
        self.jobsets = [[q.make_job(p, m.bits, m.N, m.K, self.X[m.K], y, M)
                         for p, m, y in zip(cp, self.wl.matrices, self.Y)] for cp in self.copies]
        ws = max(q.workspace_bytes(js, self.path) for js in self.jobsets)
        self.ws = q.Workspace(ws, device=dev)
        self.arrays = [q.job_array(js) for js in self.jobsets]
        self.xbytes = sum(2 * M * K for K in self.wl.distinct_K)
        self.ybytes = sum(4 * M * m.N for m in self.wl.matrices)
        torch.cuda.synchronize()

    def set_verify(self, M):
        """Time the verify head instead: the single matrix swept with the
        argmax epilogue (no logits written) and M / 6 slots of five drafts."""
        import torch

        q = self.qgemm
        dev = torch.device("cuda:0")
        self.set_M(M)
        m = self.wl.matrices[0]
        self.heads = [q.make_head_job(cp[0], m.bits, m.N, m.K, self.X[m.K], M) for cp in self.copies]
        self.vslots = q.slot_array([(6 * i, 5) for i in range(M // 6)])
        self.drafts = torch.zeros(M, dtype=torch.int32, device=dev)
        self.am = torch.empty(M, dtype=torch.int32, device=dev)
        self.acc = torch.empty(len(self.vslots), dtype=torch.int32, device=dev)
        self.ws = q.Workspace(q.verify_workspace_bytes(self.heads[0]), device=dev)
        self.ybytes = 0
        self.verify = True
        torch.cuda.synchronize()

    def step(self, i):
        q = self.qgemm
        if getattr(self, "verify", False):
            import ctypes

            st = q.lib().qgemm_verify_head(ctypes.byref(self.heads[i % len(self.heads)]), self.drafts.data_ptr(),
                                           self.vslots, len(self.vslots), self.am.data_ptr(), None,
                                           self.acc.data_ptr(), self.ws.ptr, self.ws.nbytes, self.stream)
            if st != q.OK:
                raise q.QgemmError(st, "qgemm_verify_head")
            return
        arr = self.arrays[i % len(self.arrays)]
        st = q.lib().qgemm_sweep_path(arr, len(arr), self.path, self.ws.ptr, self.ws.nbytes, self.stream)
        if st != q.OK:
            raise q.QgemmError(st, "qgemm_sweep_path")

    def run(self, steps, warmup):
        import torch

        self.stream = torch.cuda.current_stream().cuda_stream
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            self.step(warmup + i)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = e0.elapsed_time(e1) / steps
        return ms, wall

    def run_calls(self, calls, warmup):
        """Per-call event times (us): an event pair on the stream around
        each call; p10, median and p90 over the calls."""
        import numpy as np
        import torch

        self.stream = torch.cuda.current_stream().cuda_stream
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for i, (e0, e1) in enumerate(ev):
            e0.record()
            self.step(warmup + i)
            e1.record()
        torch.cuda.synchronize()
        us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
        p10, med, p90 = (round(float(x), 3) for x in np.percentile(us, [10, 50, 90]))
        return {"calls": calls, "p10": p10, "median": med, "p90": p90}

    def run_graph(self, sweeps, reps, warmup):
        """GPU time per sweep with no host gaps: `sweeps` consecutive sweeps
        (rotating over the weight copies) recorded as one round and replayed
        `reps` times; returns us per sweep."""
        import torch

        q = self.qgemm
        rsw = q.round_sweeps([(self.jobsets[i % len(self.jobsets)], self.path) for i in range(sweeps)])
        ws = q.Workspace(q.round_workspace_bytes(rsw), device=torch.device("cuda:0"))
        r = q.Round(rsw, ws)
        try:
            for _ in range(warmup):
                r.launch()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                r.launch()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (reps * sweeps)
        finally:
            torch.cuda.synchronize()
            r.destroy()

    def report(self, ms):
        s = ms / 1e3
        gbps = self.weight_bytes / s / 1e9
        alg = self.weight_bytes + self.xbytes + self.ybytes
        # roofline time: the larger of the HBM term (algorithmic bytes) and
        # the dense fp16 MFMA term (2 M N K flops)
        flops = sum(2 * self.M * m.N * m.K for m in self.wl.matrices)
        t_hbm, t_mfma = alg / (HBM_PEAK_GBPS * 1e9), flops / (MFMA_F16_PEAK_TFLOPS * 1e12)
        return {
            "workload": self.wl.name,
            "M": self.M,
            "matrices": len(self.wl.matrices),
            "ms_per_sweep": round(ms, 5),
            "weight_GBps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "tokens_per_s": round(self.M / s, 1),
            "alg_bytes": alg,
            "alg_GBps": round(alg / s / 1e9, 1),
            "weight_bytes": self.weight_bytes,
            "rotated_copies": len(self.copies),
            "roofline": {"bound": "hbm" if t_hbm >= t_mfma else "mfma",
                         "ms": round(max(t_hbm, t_mfma) * 1e3, 5),
                         "frac": round(max(t_hbm, t_mfma) / s, 4)},
        }


def ceiling(b, steps, warmup):
    """The read ceiling of the sweep launch of Bench b (a stream-kernel launch,
    M <= 16): libqgemm_ceiling's kernel over the same rotated weight copies and
    X panels, with the sweep's wave count.  Returns its time per launch."""
    import ctypes

    import torch

    import __graft_entry__

    __graft_entry__.ensure_built("qgemm_ceiling")
    L = ctypes.CDLL(__graft_entry__.LIBS["qgemm_ceiling"])

    class CJob(ctypes.Structure):
        _fields_ = [("packed", ctypes.c_void_p), ("X", ctypes.c_void_p), ("N", ctypes.c_int64),
                    ("K", ctypes.c_int64), ("ldx", ctypes.c_int64), ("bits", ctypes.c_int32)]

    L.qgemm_read_ceiling.argtypes = [ctypes.POINTER(CJob), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    L.qgemm_read_ceiling.restype = ctypes.c_int
    mats = b.wl.matrices
    units = sum(-(-(-(-m.N // 16)) // 4) * (m.K // 128) * (11 if m.bits == 5 else 9) for m in mats)
    nwaves = max(1, min(2048, units // 11))   # the stream kernels' wave count for these units
    arrays = [(CJob * len(mats))(*[CJob(p.data_ptr(), b.X[m.K].data_ptr(), m.N, m.K, m.K, m.bits)
                                   for p, m in zip(cp, mats)]) for cp in b.copies]
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream

    def launch(i):
        a = arrays[i % len(arrays)]
        if L.qgemm_read_ceiling(a, len(mats), nwaves, b.M, sink.data_ptr(), sp) != 0:
            raise RuntimeError("qgemm_read_ceiling failed")

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        launch(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"us": round(ms * 1e3, 3), "weight_GBps": round(b.weight_bytes / (ms / 1e3) / 1e9, 1),
            "waves": nwaves}


def round_bench(args):
    """Round replay: the 4-bit 64-layer stack as one sweep per matrix in layer
    order (256 launches, as an engine that interleaves other work between
    layers issues them), then the verify head over the lm_head-class matrix,
    at M = 6 (one slot, five drafts).  Times a round issued call by call
    against the same round replayed as one graph (directly, and through the
    keyed round cache), and the host time to issue each; one JSON line."""
    import ctypes

    import torch

    from self_speculative_verify_amd import qgemm as q
    from synth import workloads

    M = 6
    b = Bench(4, layers=args.stack_layers, rotate_bytes=0)
    b.set_M(M)
    h = Bench(6, rotate_bytes=0)
    dev = torch.device("cuda:0")
    jobs = b.jobsets[0]
    mh = h.wl.matrices[0]
    head = q.make_head_job(h.copies[0][0], mh.bits, mh.N, mh.K, b.X[mh.K], M)
    slots = [(0, M - 1)]
    drafts = torch.zeros(M, dtype=torch.int32, device=dev)
    am = torch.empty(M, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    sweeps = [([j], q.PATH_AUTO) for j in jobs]
    # call by call: one workspace per sweep (a workspace's layout follows its jobs)
    wss = [q.Workspace(q.workspace_bytes(j, p), device=dev) for j, p in sweeps]
    arrs = [q.job_array(j) for j, _ in sweeps]
    vws = q.Workspace(q.verify_workspace_bytes(head), device=dev)
    slot_arr = q.slot_array(slots)
    L = q.lib()
    st = torch.cuda.current_stream()
    sp = st.cuda_stream

    def eager():
        for a, ws in zip(arrs, wss):
            L.qgemm_sweep(a, 1, ws.ptr, ws.nbytes, sp)
        L.qgemm_verify_head(ctypes.byref(head), drafts.data_ptr(), slot_arr, 1, am.data_ptr(), None,
                            acc.data_ptr(), vws.ptr, vws.nbytes, sp)

    rsw = q.round_sweeps(sweeps)
    rws = q.Workspace(q.round_workspace_bytes(rsw, head), device=dev)
    rnd = q.Round(rsw, rws, head, drafts, slots, am, acc)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        host = (time.perf_counter() - t0) / steps
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, host * 1e3

    # the fused alternative: every matrix in one launch, then the head
    fused_arr = q.job_array(jobs)
    fws = q.Workspace(q.workspace_bytes(jobs), device=dev)

    def fused():
        L.qgemm_sweep(fused_arr, len(jobs), fws.ptr, fws.nbytes, sp)
        L.qgemm_verify_head(ctypes.byref(head), drafts.data_ptr(), slot_arr, 1, am.data_ptr(), None,
                            acc.data_ptr(), vws.ptr, vws.nbytes, sp)

    # the same round through the keyed cache: recorded on the first call,
    # replayed on every later one (the key is rebuilt and looked up per call)
    cache = q.RoundCache(64)

    def cached():
        cache.run(rsw, head, drafts, slots, am, acc)

    eager_ms, eager_host = timed(eager, args.steps, args.warmup)
    graph_ms, graph_host = timed(rnd.launch, args.steps, args.warmup)
    cached()
    cache_ms, cache_host = timed(cached, args.steps, args.warmup)
    fused_ms, fused_host = timed(fused, args.steps, args.warmup)
    torch.cuda.synchronize()
    cache_stats = cache.stats()
    cache.destroy()
    rnd.destroy()
    wb = b.weight_bytes + workloads.weight_bytes(mh.bits, mh.N, mh.K)
    print(json.dumps({
        "workload": f"round: {len(jobs)} one-matrix sweeps of the {args.stack_layers}-layer 4-bit stack + verify head, M={M}",
        "kernels_per_round": rnd.kernels if rnd.handle else len(jobs) + 2,
        "eager_ms": round(eager_ms, 4), "eager_host_ms": round(eager_host, 4),
        "graph_ms": round(graph_ms, 4), "graph_host_ms": round(graph_host, 4),
        "cache_hit_ms": round(cache_ms, 4), "cache_hit_host_ms": round(cache_host, 4), "cache": cache_stats,
        "fused_launch_ms": round(fused_ms, 4),
        "graph_speedup": round(eager_ms / graph_ms, 3),
        "graph_weight_GBps": round(wb / (graph_ms / 1e3) / 1e9, 1),
        "weight_bytes": wb,
    }), flush=True)


def attn_bench(args):
    """Attention verify over the 16 full-attention layers of a round: per
    layer one call for every slot (W = 6 verify positions each), caches of
    distinct layers in distinct buffers (2 GB and more, so they stream from
    HBM).  One JSON line per (cache format, slots, L)."""
    import torch

    from self_speculative_verify_amd import qgemm as q
    from synth import synth

    dev = torch.device("cuda:0")
    layers, W, HQ, HKV, D = 16, 6, 24, 4, 256
    for kv in (q.KV_FP16, q.KV_FP8):
        for nslots, L in ((1, 32768), (8, 8192)):
            esz = 2 if kv == q.KV_FP16 else 1
            # values: standard normals (fp16) or random finite E4M3 bytes of
            # the same spread (|v| < 4); the timing does not depend on them
            base = torch.from_numpy(synth.x_fp16(77, 64, HKV * D)).to(dev)
            per_layer = []
            for li in range(layers):
                slots = []
                for si in range(nslots):
                    Qt = base[:W * HQ * D // (HKV * D)].reshape(W, HQ, D).contiguous()
                    if kv == q.KV_FP16:
                        Kt = base[0].repeat(L).reshape(L, HKV, D).contiguous()
                        Vt = base[1].repeat(L).reshape(L, HKV, D).contiguous()
                    else:
                        g = torch.Generator(device=dev)
                        g.manual_seed(li * 100 + si)
                        Kt = torch.randint(0, 0x4C, (L, HKV, D), dtype=torch.uint8, device=dev, generator=g)
                        Vt = torch.randint(0, 0x4C, (L, HKV, D), dtype=torch.uint8, device=dev, generator=g)
                        Kt |= torch.randint(0, 2, (L, HKV, D), dtype=torch.uint8, device=dev, generator=g) << 7
                    Ot = torch.empty((W, HQ, D), dtype=torch.float32, device=dev)
                    slots.append((Qt, Kt, Vt, Ot, L, W))
                arr = q.attn_slots(slots)
                per_layer.append((arr, slots))
            ws = q.Workspace(q.attn_workspace_bytes(per_layer[0][0], kv), device=dev)
            L_ = q.lib()
            sp = torch.cuda.current_stream().cuda_stream

            def step():
                for arr, _ in per_layer:
                    L_.qgemm_attn_verify(arr, len(arr), kv, 0.0625, ws.ptr, ws.nbytes, sp)

            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                step()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            kv_bytes = layers * nslots * L * HKV * D * 2 * esz
            io_bytes = layers * nslots * W * HQ * D * (2 + 4)
            print(json.dumps({
                "workload": f"attention verify, {layers} layers, {nslots} slot(s) x L={L}, W={W}, "
                            f"{'fp16' if kv == q.KV_FP16 else 'e4m3'} KV",
                "ms_per_round": round(ms, 4), "us_per_layer": round(ms * 1e3 / layers, 2),
                "kv_GBps": round(kv_bytes / (ms / 1e3) / 1e9, 1),
                "hbm_frac": round((kv_bytes + io_bytes) / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                "kv_bytes": kv_bytes,
            }), flush=True)
            del per_layer, ws
            torch.cuda.empty_cache()


def timeline(args):
    """Per-wave timeline of the stream kernel (a build of the library with
    s_memrealtime stamps): workloads 2 (M = 1) and 3 (M = 6), the last of
    `steps` back-to-back sweeps.  Prints one JSON line per workload with
    percentiles (us) of each wave's start (after the first wave's), first
    step computed, streaming span and end."""
    import ctypes

    import numpy as np
    import torch

    import __graft_entry__
    from self_speculative_verify_amd import qgemm

    __graft_entry__.ensure_built("qgemm_timeline")
    qgemm.LIB_PATH = __graft_entry__.LIBS["qgemm_timeline"]
    L = qgemm.lib()
    L.qgemm_timeline_set.argtypes = [ctypes.c_void_p]
    L.qgemm_timeline_set.restype = None
    words = 8
    tr = torch.zeros(4096 * words, dtype=torch.int64, device="cuda")
    L.qgemm_timeline_set(tr.data_ptr())
    for cfg in (2, 3):
        b = Bench(cfg)
        tr.zero_()
        ms, _ = b.run(args.steps, args.warmup)
        torch.cuda.synchronize()
        t = tr.cpu().numpy().reshape(-1, words)
        t = t[t[:, 0] > 0]
        base = t[:, 0].min()
        us = lambda a: (a / 100.0)  # 100 MHz
        pct = lambda a: [round(float(x), 2) for x in np.percentile(a, [0, 10, 50, 90, 100])]
        readers = (t[:, 5] & 8) != 0
        out = {
            "workload": b.wl.name, "M": b.M, "waves": int(len(t)), "ms_per_sweep": round(ms, 5),
            "percentiles": [0, 10, 50, 90, 100],
            "start_us": pct(us(t[:, 0] - base)),
            "first_step_us": pct(us(t[:, 1] - t[:, 0])),
            "stream_span_us": pct(us(t[:, 2] - t[:, 1])),
            "after_last_step_us": pct(us(t[:, 3] - t[:, 2])),
            "end_us": pct(us(t[:, 3] - base)),
            "kernel_span_us": round(float(us(t[:, 3].max() - base)), 2),
            "readers": int(readers.sum()),
            "wait_us": pct(us(t[:, 4])),
            "compute_us": pct(us(t[:, 7])),
            "plan_us": pct(us(t[:, 6] - t[:, 0])),
        }
        print(json.dumps(out), flush=True)
        if args.timeline_dump:
            os.makedirs(args.timeline_dump, exist_ok=True)
            np.save(os.path.join(args.timeline_dump, f"timeline_cfg{cfg}.npy"), t)
        del b
        torch.cuda.empty_cache()
    L.qgemm_timeline_set(None)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def _timed(fn, min_s=0.5, max_reps=50):
    """Seconds per call of fn: one call, repeated while under min_s in total."""
    t0 = time.perf_counter()
    fn()
    reps = 1
    while time.perf_counter() - t0 < min_s and reps < max_reps:
        fn()
        reps += 1
    return (time.perf_counter() - t0) / reps


def _sampled_rows(m, step):
    """Every step-th 16-row block of matrix m (generation is seeded per row, so
    the rows are the matrix's own); returns (W rows, number of blocks)."""
    import numpy as np

    from synth import synth, workloads

    nrb = -(-m.N // 16)
    blocks = list(range(0, nrb, step))
    W = np.concatenate([synth.weights(m.seed, m.K, 16 * b, min(16, m.N - 16 * b), workloads.SIGMA,
                                      outlier_thresh=m.thresh, outlier_mult=workloads.OUTLIER_MULT)
                        for b in blocks])
    return W, len(blocks), nrb


def cpu_baseline():
    """The oracle (oracle.sweep: plain C, fp64, scalar decode from the packed
    bytes), untuned, on the host cores this process may use; generation and
    packing untimed.  Workloads 1-3 in full on every core, plus one thread
    (workload 1 in full, 2 and 3 on a 1/4 and 1/16 sample of row blocks);
    the 64-layer stacks (workloads 4 and 5) on a 1/16 sample of the row
    blocks of layer 0's four matrices, at M = 1 and at every M the GPU line
    reports, scaled by 16 x 64: the sweep is independent per output column,
    so its work is linear in the rows swept and the same in every layer."""
    import numpy as np

    from oracle import oracle
    from synth import synth, workloads

    threads = oracle.cpu_share()
    per = {}

    def entry(wl, M, t, scale, sample, one=None):
        wb = sum(workloads.weight_bytes(m.bits, m.N, m.K) for m in wl.matrices)
        full_s = t * scale
        e = {"workload": wl.name, "M": M, "s_per_sweep": round(full_s, 4),
             "weight_GBps": round(wb / full_s / 1e9, 4), "tokens_per_s": round(M / full_s, 3),
             "threads": threads, "sample": sample}
        if one is not None:
            e["one_thread"] = one
        return e

    def x_of(wl, K, M):
        return synth.x_fp16(wl.x_seed(K), M, K)

    # workloads 1-3: every matrix in full on every core; one thread on a sample
    for cfg, one_step in ((1, 1), (2, 4), (3, 16)):
        wl = workloads.workload(cfg)
        M = wl.Ms[0]
        mats = []
        for m in wl.matrices:
            W = synth.weights(m.seed, m.K, 0, m.N, workloads.SIGMA)
            mats.append((m, oracle.quantize_pack(W, m.bits), x_of(wl, m.K, M)))
            del W
        t_all = _timed(lambda: [oracle.sweep(p, m.N, m.K, m.bits, X, nthreads=threads) for m, p, X in mats])
        samples = []
        for m, p, X in mats:
            nrb = -(-m.N // 16)
            cols = np.concatenate([np.arange(16 * b, min(16 * b + 16, m.N)) for b in range(0, nrb, one_step)])
            samples.append((m, p, X, cols, m.N / cols.size))
        t_one = _timed(lambda: [oracle.sweep(p, m.N, m.K, m.bits, X, cols=c, nthreads=1)
                                for m, p, X, c, _ in samples])
        scale_one = samples[0][4]   # the same row-block fraction of every matrix
        wb = sum(workloads.weight_bytes(m.bits, m.N, m.K) for m in wl.matrices)
        one = {"s_per_sweep": round(t_one * scale_one, 4),
               "weight_GBps": round(wb / (t_one * scale_one) / 1e9, 4),
               "sample": "full" if one_step == 1 else f"every {one_step}th 16-row block, scaled x{scale_one:.2f}"}
        per[str(cfg)] = entry(wl, M, t_all, 1.0, "full", one)
        log(f"[bench] cpu baseline workload {cfg}: {json.dumps(per[str(cfg)])}")
        del mats, samples

    # the stacks: a 1/16 row-block sample of layer 0, scaled to 64 layers
    for cfg, Ms in ((4, [1, 48]), (5, workloads.workload(5).Ms)):
        wl = workloads.workload(cfg)
        layer0 = wl.matrices[:4]
        mats, scale = [], None
        for m in layer0:
            W, nb, nrb = _sampled_rows(m, 16)
            mats.append((m, oracle.quantize_pack(W, m.bits), W.shape[0]))
            scale = nrb / nb
            del W
        res = {}
        for M in Ms:
            Xs = {K: x_of(wl, K, M) for K in wl.distinct_K}
            t = _timed(lambda: [oracle.sweep(p, n, m.K, m.bits, Xs[m.K], nthreads=threads) for m, p, n in mats],
                       min_s=0.0, max_reps=1)
            res[str(M)] = entry(wl, M, t, scale * (len(wl.matrices) // 4),
                                f"every 16th 16-row block of layer 0's 4 matrices, scaled x{scale:.2f} x "
                                f"{len(wl.matrices) // 4} layers")
            log(f"[bench] cpu baseline workload {cfg} M={M}: {json.dumps(res[str(M)])}")
        per[str(cfg)] = res

    head = per["2"]
    return {"value": head["weight_GBps"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "workload 2 (34816x5120 4-bit, M=1) swept in full on every core; per_config: "
                      "workloads 1-3 in full plus one-thread figures, the 64-layer stacks on a 1/16 "
                      "row-block sample of layer 0 scaled to the stack",
            "cpu_model": cpu_model(), "one_thread": head["one_thread"], "per_config": per}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", type=int, default=0,
                    help="time one workload (1, 2, 3 or 4) only; 5 times the 5-bit stack at every M of its "
                         "sweep; 6 times the verify head; 7 and 8 the group-64 and zero-point 4-bit "
                         "stacks at M = 1, 8, 48; 9 a round of per-matrix sweeps plus the verify head, "
                         "issued call by call and replayed as one graph; 10 the attention verify")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--path", choices=sorted(PATHS), default="auto",
                    help="with --only 1-5, 7, 8: the sweep path (gemv: panels of at most 8 rows)")
    ap.add_argument("--Ms", default="", help="with --only 1-5, 7, 8: comma-separated panel heights to time")
    ap.add_argument("--stack-layers", type=int, default=64)
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB")
    ap.add_argument("--timeline-dump", default="", metavar="DIR",
                    help="with --timeline: also save the raw stamps (numpy) under DIR")
    ap.add_argument("--ceiling", action="store_true",
                    help="the read ceiling of the sweep launches of workloads 2 and 3 (same geometry, "
                         "loads only) beside their sweep times")
    ap.add_argument("--timeline", action="store_true",
                    help="per-wave stamps of the stream kernel on workloads 2 and 3 (diagnostic build)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the sweep shards "
              "along N with no collective, so one GPU's share at its real shape is what it times",
              file=sys.stderr)
        sys.exit(2)

    import __graft_entry__

    __graft_entry__.ensure_built()
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calib:
        # one device-to-device copy kernel per step: reads and writes exactly
        # n bytes each, the yardstick for the byte counters
        n = args.copy_calib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)
        return

    if args.timeline:
        timeline(args)
        return

    if args.only == 6:
        # the verify head (lm_head-class sweep + argmax + acceptance) at each
        # M of workload 6; one JSON line per M, no headline
        b = Bench(6)
        for M in b.wl.Ms:
            b.verify = False
            b.set_M(M)
            ms_sweep, _ = b.run(args.steps, args.warmup)     # the same matrix, logits written
            b.set_verify(M)
            ms, wall = b.run(args.steps, args.warmup)
            r = b.report(ms)
            r["wall_s"] = round(wall, 4)
            r["slots"] = M // 6
            r["rounds_per_s"] = round(1e3 / ms, 1)
            r["plain_sweep_ms"] = round(ms_sweep, 5)
            print(json.dumps(r), flush=True)
        return

    if args.only == 9:
        round_bench(args)
        return

    if args.only == 10:
        attn_bench(args)
        return

    if args.only in (5, 7, 8):
        # a stack (5-bit; 7: 4-bit group-64; 8: 4-bit zero-point) at each M
        # of its sweep (same weights, fresh panels); one JSON line per M, no
        # headline
        b = Bench(args.only, layers=args.stack_layers)
        b.path = PATHS[args.path]
        for M in ([int(m) for m in args.Ms.split(",")] if args.Ms else b.wl.Ms):
            b.set_M(M)
            ms, wall = b.run(args.steps, args.warmup)
            r = b.report(ms)
            r["wall_s"] = round(wall, 4)
            print(json.dumps(r), flush=True)
        return

    if args.ceiling:
        for cfg in (2, 3):
            b = Bench(cfg)
            ms_sweep, _ = b.run(args.steps, args.warmup)
            c = ceiling(b, args.steps, args.warmup)
            c.update({"workload": b.wl.name, "M": b.M, "sweep_us": round(ms_sweep * 1e3, 3),
                      "sweep_frac_of_ceiling": round(c["us"] / (ms_sweep * 1e3), 4)})
            print(json.dumps(c), flush=True)
            del b
            torch.cuda.empty_cache()
        return

    if args.only in (1, 2, 3, 4):
        b = Bench(args.only, layers=args.stack_layers if args.only == 4 else None)
        b.path = PATHS[args.path]
        for M in ([int(m) for m in args.Ms.split(",")] if args.Ms else [b.M]):
            b.set_M(M)
            ms, wall = b.run(args.steps, args.warmup)
            r = b.report(ms)
            r["wall_s"] = round(wall, 4)
            r["path"] = args.path
            print(json.dumps(r), flush=True)
        return

    # the default line: every workload (1: latency; 2, 3: with their read
    # ceiling; 4 at M = 48; 5 at every M of its sweep), then the oracle
    configs = {}
    for cfg in (2, 3, 1, 4, 5):
        log(f"[bench] workload {cfg}: building")
        b = Bench(cfg, layers=args.stack_layers if cfg in (4, 5) else None)
        log(f"[bench] workload {cfg}: {len(b.wl.matrices)} matrices, {b.packed_bytes / 1e6:.1f} MB "
            f"packed x {len(b.copies)} copies; timing {args.steps} steps")
        if cfg == 5:
            configs["5"] = {}
            for M in b.wl.Ms:
                b.set_M(M)
                ms, wall = b.run(args.steps, args.warmup)
                configs["5"][str(M)] = b.report(ms)
                log(f"[bench] workload 5 M={M}: {json.dumps(configs['5'][str(M)])}")
        else:
            ms, wall = b.run(args.steps, args.warmup)
            r = b.report(ms)
            r["wall_s"] = round(wall, 4)
            if cfg in (2, 3):
                c = ceiling(b, args.steps, args.warmup)
                c["sweep_frac_of_ceiling"] = round(c["us"] / (ms * 1e3), 4)
                r["read_ceiling"] = c
            if cfg == 1:
                r["us_per_sweep"] = round(ms * 1e3, 3)
                # a sweep this short is issued from the host about as fast as it
                # runs: the same sweeps replayed as one graph give the GPU time
                r["graph_us_per_sweep"] = round(b.run_graph(50, 20, 2), 3)
            # per call (an event pair around each): the spread behind the mean
            if cfg in (1, 2, 3):
                r["per_call_us"] = b.run_calls(50, 10)
            configs[str(cfg)] = r
            log(f"[bench] workload {cfg}: {json.dumps(r)}")
        del b
        torch.cuda.empty_cache()

    head = configs["2"]
    # dominant kernel: the headline sweep is one stream-kernel launch per
    # step, timed with events on the stream it is launched on, so the event
    # time per step is the kernel's average duration (launch gaps included)
    roof = {
        "bound": "hbm",
        "achieved": head["alg_GBps"],
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(head["alg_GBps"] / HBM_PEAK_GBPS, 4),
        "traffic": None,
    }
    tr = TRAFFIC.get(kernel_sha())
    if tr and head["workload"] == tr["workload"]:
        roof["traffic"] = tr["bytes"]
    line = {
        "metric": METRIC,
        "value": head["weight_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_sweep"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "M": head["M"], "matrices": head["matrices"]},
        "hbm_frac": head["hbm_frac"],
        "read_ceiling_frac": head["read_ceiling"]["sweep_frac_of_ceiling"],
        "tokens_per_s": head["tokens_per_s"],
        "configs": configs,
        "roofline": roof,
    }
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
