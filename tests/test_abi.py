"""The C boundary on the CPU: the library loads, exports what the header
declares, and validates arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import __graft_entry__
from oracle import oracle
from self_speculative_verify_amd import qgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _lib_built():
    __graft_entry__.ensure_built("qgemm")


def _header_functions():
    text = open(os.path.join(ROOT, "include", "qgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(qgemm_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_match_header():
    names = _header_functions()
    assert names == sorted(qgemm.EXPORTS)
    L = ctypes.CDLL(qgemm.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_ceiling_library_loads_and_rejects_bad_arguments():
    """The read-ceiling measurement library (bench.py) exports its one entry
    point and refuses bad arguments before any HIP call."""
    __graft_entry__.ensure_built("qgemm_ceiling")
    L = ctypes.CDLL(__graft_entry__.LIBS["qgemm_ceiling"])
    fn = L.qgemm_read_ceiling
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int

    class CJob(ctypes.Structure):
        _fields_ = [("packed", ctypes.c_void_p), ("X", ctypes.c_void_p), ("N", ctypes.c_int64),
                    ("K", ctypes.c_int64), ("ldx", ctypes.c_int64), ("bits", ctypes.c_int32)]

    ok = dict(packed=0x100000, X=0x200000, N=34816, K=5120, ldx=5120, bits=4)
    for kw in (dict(bits=3), dict(K=5120 - 32), dict(ldx=4096), dict(packed=0), dict(N=0)):
        j = CJob(**{**ok, **kw})
        assert fn(ctypes.byref(j), 1, 2048, 1, 0x300000, None) == 1, kw
    j = CJob(**ok)
    assert fn(ctypes.byref(j), 1, 2048, 1, None, None) == 1           # no sink
    assert fn(ctypes.byref(j), 1, 2048, 17, 0x300000, None) == 1      # more than 16 rows
    assert fn(ctypes.byref(j), 0, 2048, 1, 0x300000, None) == 1       # no job
    small = CJob(**{**ok, "N": 64, "K": 128, "ldx": 128})
    assert fn(ctypes.byref(small), 1, 2048, 1, 0x300000, None) == 1   # under 11 units per wave


def test_packed_bytes_agrees_with_oracle():
    for bits in (4, 5):
        for N, K in [(1, 32), (15, 96), (16, 128), (1024, 1024), (34816, 5120), (5120, 17408),
                     (7168, 5120), (33, 416)]:
            assert qgemm.packed_bytes(bits, N, K) == oracle.packed_bytes(bits, N, K) > 0
    for fmt in (qgemm.FMT_Q4_G64, qgemm.FMT_Q4_ZP):
        for N, K in [(1, 64), (15, 192), (16, 128), (34816, 5120), (5120, 17408), (33, 448)]:
            assert qgemm.packed_bytes(fmt, N, K) == oracle.packed_bytes(fmt, N, K) > 0
    assert qgemm.packed_bytes(qgemm.FMT_Q4_ZP, 3, 96) == oracle.packed_bytes(qgemm.FMT_Q4_ZP, 3, 96) > 0
    assert qgemm.packed_bytes(qgemm.FMT_Q4_G64, 16, 96) == 0          # K % 64
    assert qgemm.packed_bytes(qgemm.FMT_Q4_G64, 16, 32) == 0
    assert qgemm.packed_bytes(0x304, 16, 128) == 0
    assert qgemm.packed_bytes(3, 16, 128) == 0
    assert qgemm.packed_bytes(4, 16, 100) == 0
    assert qgemm.packed_bytes(4, 0, 128) == 0
    assert qgemm.packed_bytes(4, 16, 0) == 0


def test_auto_path_table():
    for M in range(1, 65):
        assert qgemm.auto_path(M) == qgemm.PATH_MFMA
    assert qgemm.auto_path(0) == -1 and qgemm.auto_path(65) == -1


def _job(**kw):
    base = dict(packed=0x100000, X=0x200000, Y=0x10000000, N=64, K=256, ldx=256, ldy=64, M=4, bits=4)
    base.update(kw)
    return qgemm.Job(base["packed"], base["X"], base["Y"], base["N"], base["K"], base["ldx"],
                     base["ldy"], base["M"], base["bits"])


BAD = [
    dict(M=0), dict(M=65), dict(bits=3), dict(bits=8), dict(K=100), dict(K=0), dict(N=0),
    dict(bits=0x104, K=96, ldx=96), dict(bits=0x304), dict(bits=0x105),
    dict(packed=0), dict(X=0), dict(Y=0), dict(packed=0x100080), dict(X=0x200008),
    dict(Y=0x10000004), dict(ldx=255), dict(ldx=260), dict(ldy=63), dict(ldy=66),
    dict(Y=0x200000),                      # Y overlaps X
    dict(Y=0x100000 + 256),                # Y inside the packed weights
]


@pytest.mark.parametrize("kw", BAD)
def test_validation_rejects(kw):
    jobs = [_job(**kw)]
    assert qgemm.validate(jobs, qgemm.PATH_AUTO, 0x40000000, 1 << 30) == qgemm.ERR_INVALID_ARG
    assert qgemm.workspace_bytes(jobs) == 0


def test_validation_rejects_overlaps_across_jobs():
    a = _job()
    cases = [
        [a, _job(Y=0x10000000 + 128)],                  # two outputs overlap
        [a, _job(Y=0x20000000, X=0x10000000 + 64)],     # a job reads another's output
        [a, _job(Y=0x20000000, packed=0x10000000)],     # weights under another's output
    ]
    for jobs in cases:
        assert qgemm.validate(jobs, qgemm.PATH_AUTO, 0x40000000, 1 << 30) == qgemm.ERR_INVALID_ARG
    # shared inputs are fine
    ok = [a, _job(Y=0x20000000)]
    assert qgemm.validate(ok, qgemm.PATH_AUTO, 0x40000000, 1 << 30) == qgemm.OK


def test_validation_accepts_and_sizes_workspace():
    jobs = [_job(), _job(Y=0x20000000, M=33, bits=5, N=17, K=416, ldx=416, ldy=20),
            _job(Y=0x30000000, bits=0x104, K=448, ldx=448), _job(Y=0x38000000, bits=0x204, M=20)]
    ws = qgemm.workspace_bytes(jobs)
    assert ws > 0 and ws % 256 == 0
    assert qgemm.validate(jobs, qgemm.PATH_AUTO, 0x40000000, ws) == qgemm.OK
    assert qgemm.validate(jobs, qgemm.PATH_AUTO, 0x40000000, ws - 256) == qgemm.ERR_INVALID_ARG
    assert qgemm.validate(jobs, qgemm.PATH_AUTO, 0x40000001, ws) == qgemm.ERR_INVALID_ARG
    assert qgemm.validate(jobs, qgemm.PATH_AUTO, 0, ws) == qgemm.ERR_INVALID_ARG
    # GEMV is limited to M <= 8
    assert qgemm.validate(jobs, qgemm.PATH_GEMV, 0x40000000, 1 << 30) == qgemm.ERR_INVALID_ARG
    assert qgemm.validate(jobs[:1], qgemm.PATH_GEMV, 0x40000000, 1 << 30) == qgemm.OK
    assert qgemm.validate(jobs, 7, 0x40000000, 1 << 30) == qgemm.ERR_INVALID_ARG
    assert qgemm.validate([], qgemm.PATH_AUTO, 0x40000000, 1 << 30) == qgemm.ERR_INVALID_ARG


def test_workspace_sized_by_accumulators():
    """The split-K slots hold each lane's accumulators: one per row block up to
    four panel rows on the MFMA path (M = 1..4 share a size), more above; the
    K split itself depends on the shapes only."""
    def ws(M, path=qgemm.PATH_AUTO):
        return qgemm.workspace_bytes([_job(N=34816, K=5120, M=M, Y=0x100000000, ldy=34816,
                                           packed=0x200000000, X=0x300000000, ldx=5120)], path)
    assert ws(1) == ws(4) > 0
    assert ws(8) == ws(5) > ws(4)
    assert ws(16) > ws(8)
    assert ws(2, qgemm.PATH_GEMV) > ws(1, qgemm.PATH_GEMV) > 0


def test_noalloc_rejects_before_any_hip_call():
    """The allocation-free sweep refuses argument errors and job sets whose
    workspace exceeds its static scratch on the host, before any HIP call
    (this runs without a GPU)."""
    L = qgemm.lib()
    bad = qgemm.job_array([_job(M=0)])
    assert L.qgemm_sweep_noalloc(bad, 1, qgemm.PATH_AUTO, None) == qgemm.ERR_INVALID_ARG
    # five launches of at least 4 GiB of weights each (classes 1..16): their
    # slots alone exceed the scratch
    N, K = 120000, 65536
    jobs = [_job(packed=(2 + 2 * i) << 32, X=(20 + i) << 32, Y=(30 + i) << 32, N=N, K=K, ldx=K,
                 ldy=N, M=M) for i, M in enumerate((1, 2, 4, 8, 16))]
    assert qgemm.packed_bytes(4, N, K) >= 4 << 30
    assert qgemm.workspace_bytes(jobs, qgemm.PATH_MFMA) > qgemm.NOALLOC_SCRATCH_BYTES
    assert L.qgemm_sweep_noalloc(qgemm.job_array(jobs), 5, qgemm.PATH_MFMA, None) == qgemm.ERR_INVALID_ARG


def test_validation_rejects_workspace_overlap():
    """The workspace is written: it may overlap no job's X, weights or Y."""
    a = _job()
    for w in (0x100000, 0x200000 - 256, 0x10000000):     # packed, X (its start inside), Y
        assert qgemm.validate([a], qgemm.PATH_AUTO, w, 1 << 20) == qgemm.ERR_INVALID_ARG, hex(w)
    assert qgemm.validate([a], qgemm.PATH_AUTO, 0x40000000, 1 << 20) == qgemm.OK


def test_status_strings():
    for s in range(5):
        assert qgemm.status_string(s)
    assert "non-finite" in qgemm.status_string(qgemm.ERR_NONFINITE)


def test_no_cpu_fallback_in_product_path():
    """The package never imports the oracle and never computes on the host."""
    pkg = os.path.join(ROOT, "self_speculative_verify_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "from oracle" not in text and "import oracle" not in text, f
                assert "qg_oracle" not in text, f


def test_verify_head_validation_rejects_before_any_launch():
    L = qgemm.lib()
    head = _job(M=6, Y=0)                      # logits not written: allowed
    ws = qgemm.verify_workspace_bytes(head)
    assert ws > 0 and ws % 8 == 0
    assert qgemm.verify_workspace_bytes(_job(M=0, Y=0)) == 0
    good = qgemm.slot_array([(0, 5)])
    drafts, am, acc, mx, wsp = 0x50000000, 0x50001000, 0x50002000, 0x50003000, 0x40000000

    def call(h=head, d=drafts, slots=good, n=None, a=am, c=acc, w=wsp, nb=ws):
        return L.qgemm_verify_head(ctypes.byref(h), d, slots, len(slots) if n is None else n, a, mx, c, w, nb, None)

    assert call(h=_job(M=0, Y=0)) == qgemm.ERR_INVALID_ARG
    assert call(n=0) == qgemm.ERR_INVALID_ARG
    assert call(slots=qgemm.slot_array([(0, 0)] * 65)) == qgemm.ERR_INVALID_ARG
    for bad in ([(-1, 2)], [(0, -1)], [(0, 6)], [(3, 3)], [(0, 5), (6, 0)]):
        assert call(slots=qgemm.slot_array(bad)) == qgemm.ERR_INVALID_ARG, bad
    assert call(d=None) == qgemm.ERR_INVALID_ARG           # drafts needed when a slot drafts
    assert call(a=None) == qgemm.ERR_INVALID_ARG
    assert call(c=None) == qgemm.ERR_INVALID_ARG
    assert call(w=0) == qgemm.ERR_INVALID_ARG
    assert call(w=wsp + 8) == qgemm.ERR_INVALID_ARG
    assert call(nb=ws - 8) == qgemm.ERR_INVALID_ARG
    # outputs and workspace are written: no overlap among them or with the job
    assert call(a=acc) == qgemm.ERR_INVALID_ARG             # argmax over accepted
    assert call(a=mx + 8) == qgemm.ERR_INVALID_ARG          # argmax over maxlogit
    assert call(c=wsp + 256) == qgemm.ERR_INVALID_ARG       # accepted inside the workspace
    assert call(a=0x200000) == qgemm.ERR_INVALID_ARG        # argmax over the head's X
    assert call(w=0x100000) == qgemm.ERR_INVALID_ARG        # workspace over the weights


def test_round_validation_rejects_before_any_launch():
    L = qgemm.lib()
    a = [_job()]
    b = [_job(Y=0x20000000, M=40, N=300, ldy=300)]
    sweeps = qgemm.round_sweeps([(a, qgemm.PATH_AUTO), (b, qgemm.PATH_MFMA)])
    ws = qgemm.round_workspace_bytes(sweeps)
    assert ws > 0 and ws % 256 == 0
    head = _job(M=6, Y=0)
    wsh = qgemm.round_workspace_bytes(sweeps, head)
    assert wsh >= ws + 16 * 64 * 8
    # invalid sweeps or head: size 0
    assert qgemm.round_workspace_bytes(qgemm.round_sweeps([([_job(M=0)], 0)])) == 0
    assert qgemm.round_workspace_bytes(qgemm.round_sweeps([(a, 9)])) == 0
    assert qgemm.round_workspace_bytes(sweeps, _job(M=65, Y=0)) == 0
    assert L.qgemm_round_workspace_bytes(None, 0, None) == 0
    out = ctypes.c_void_p()
    good = qgemm.slot_array([(0, 5)])

    def create(sw=sweeps, n=None, h=None, slots=None, w=0x40000000, nb=wsh, o=ctypes.byref(out), d=0x50000000,
               am=0x50001000, acc=0x50002000):
        return L.qgemm_round_create(sw, len(sw) if n is None else n, ctypes.byref(h) if h is not None else None,
                                    d, slots, len(slots) if slots else 0, am, None, acc, w, nb, None, o)

    assert create(o=None) == qgemm.ERR_INVALID_ARG
    assert create(w=0) == qgemm.ERR_INVALID_ARG
    assert create(w=0x40000008) == qgemm.ERR_INVALID_ARG
    assert create(nb=ws - 256) == qgemm.ERR_INVALID_ARG
    assert create(n=-1) == qgemm.ERR_INVALID_ARG
    assert create(sw=qgemm.round_sweeps([([_job(K=100)], 0)])) == qgemm.ERR_INVALID_ARG
    assert create(h=head, slots=qgemm.slot_array([(0, 6)])) == qgemm.ERR_INVALID_ARG
    assert create(h=head, slots=good, am=None) == qgemm.ERR_INVALID_ARG
    assert create(h=head, slots=good, d=None) == qgemm.ERR_INVALID_ARG
    assert create(h=head, slots=good, nb=wsh - 256) == qgemm.ERR_INVALID_ARG
    assert L.qgemm_round_create(None, 0, None, None, None, 0, None, None, None, 0x40000000, 1 << 20, None,
                                ctypes.byref(out)) == qgemm.ERR_INVALID_ARG
    assert out.value is None
    assert L.qgemm_round_launch(None, None) == qgemm.ERR_INVALID_ARG
    assert L.qgemm_round_kernels(None) == 0
    L.qgemm_round_destroy(None)


def test_round_cache_rejects_before_any_hip_call():
    """Creation, bad arguments and every invalid miss return before any HIP
    call, and leave the cache as it was."""
    L = qgemm.lib()
    out = ctypes.c_void_p()
    assert L.qgemm_round_cache_create(0, ctypes.byref(out)) == qgemm.ERR_INVALID_ARG
    assert L.qgemm_round_cache_create(qgemm.ROUND_CACHE_MAX + 1, ctypes.byref(out)) == qgemm.ERR_INVALID_ARG
    assert L.qgemm_round_cache_create(4, None) == qgemm.ERR_INVALID_ARG
    assert out.value is None
    cache = qgemm.RoundCache(4)
    try:
        hit = ctypes.c_int(7)
        sw = qgemm.round_sweeps([([_job()], qgemm.PATH_AUTO)])

        def run(c=cache.handle, sweeps=sw, n=None, h=None, slots=None, h_out=ctypes.byref(hit), am=0x50001000,
                acc=0x50002000, d=0x50000000):
            return L.qgemm_round_cache_run(c, sweeps, len(sweeps) if n is None else n,
                                           ctypes.byref(h) if h is not None else None, d, slots,
                                           len(slots) if slots else 0, am, None, acc, None, h_out)

        assert run(c=None) == qgemm.ERR_INVALID_ARG
        assert hit.value == 0
        assert run(h_out=None) == qgemm.ERR_INVALID_ARG
        assert run(n=-1) == qgemm.ERR_INVALID_ARG
        assert run(sweeps=None, n=0) == qgemm.ERR_INVALID_ARG            # no sweeps and no head
        assert run(sweeps=qgemm.round_sweeps([([_job(K=100)], 0)])) == qgemm.ERR_INVALID_ARG
        assert run(sweeps=qgemm.round_sweeps([([_job(M=0)], 0)])) == qgemm.ERR_INVALID_ARG
        assert run(sweeps=qgemm.round_sweeps([([_job()], 9)])) == qgemm.ERR_INVALID_ARG
        head = _job(M=6, Y=0)
        good = qgemm.slot_array([(0, 5)])
        assert run(h=head, slots=qgemm.slot_array([(0, 6)])) == qgemm.ERR_INVALID_ARG
        assert run(h=head, slots=good, am=None) == qgemm.ERR_INVALID_ARG
        assert run(h=head, slots=good, d=None) == qgemm.ERR_INVALID_ARG
        assert run(h=head, slots=None) == qgemm.ERR_INVALID_ARG
        assert cache.stats() == {"size": 0, "hits": 0, "misses": 0, "evictions": 0}
        assert L.qgemm_round_cache_stats(None, None, None, None, None) == qgemm.ERR_INVALID_ARG
    finally:
        cache.destroy()
    L.qgemm_round_cache_destroy(None)


def test_attn_validation_rejects_before_any_launch():
    L = qgemm.lib()

    def slot(Q=0x100000, K=0x200000, V=0x300000, O=0x40000000, Ln=100, W=6):
        return qgemm.AttnSlot(Q, K, V, O, Ln, W)

    def arr(*ss):
        return (qgemm.AttnSlot * len(ss))(*ss)

    good = arr(slot())
    ws = qgemm.attn_workspace_bytes(good, qgemm.KV_FP16)
    assert ws > 0 and ws % 256 == 0
    assert qgemm.attn_workspace_bytes(good, qgemm.KV_FP8) == ws        # layout from positions only
    bad = [slot(W=0), slot(W=17), slot(Ln=5), slot(Ln=(1 << 24) + 1), slot(Q=0), slot(O=0x40000008),
           slot(K=0x200004), slot(O=0x100000), slot(O=0x300000 + 64)]
    for b in bad:
        assert qgemm.attn_workspace_bytes(arr(b), qgemm.KV_FP16) == 0
        assert L.qgemm_attn_verify(arr(b), 1, qgemm.KV_FP16, 0.0625, 0x50000000, 1 << 30, None) == qgemm.ERR_INVALID_ARG
    assert qgemm.attn_workspace_bytes(good, 2) == 0
    assert L.qgemm_attn_verify(good, 0, 0, 0.0625, 0x50000000, 1 << 30, None) == qgemm.ERR_INVALID_ARG
    assert L.qgemm_attn_verify(arr(*[slot(O=0x40000000 + (1 << 20) * i) for i in range(17)]), 17, 0, 0.0625,
                               0x50000000, 1 << 30, None) == qgemm.ERR_INVALID_ARG
    two = arr(slot(), slot(O=0x40000000 + 1024))                     # outputs overlap
    assert L.qgemm_attn_verify(two, 2, 0, 0.0625, 0x50000000, 1 << 30, None) == qgemm.ERR_INVALID_ARG
    cross = arr(slot(), slot(Q=0x40000000 + 4096, O=0x48000000))        # an output over another slot's Q
    assert L.qgemm_attn_verify(cross, 2, 0, 0.0625, 0x50000000, 1 << 30, None) == qgemm.ERR_INVALID_ARG
    ok2 = arr(slot(), slot(O=0x48000000))
    assert qgemm.attn_workspace_bytes(ok2, qgemm.KV_FP16) > 0
    assert L.qgemm_attn_verify(good, 1, 0, float("nan"), 0x50000000, 1 << 30, None) == qgemm.ERR_INVALID_ARG
    assert L.qgemm_attn_verify(good, 1, 0, 0.0625, 0x50000008, 1 << 30, None) == qgemm.ERR_INVALID_ARG
    assert L.qgemm_attn_verify(good, 1, 0, 0.0625, 0x50000000, ws - 256, None) == qgemm.ERR_INVALID_ARG
