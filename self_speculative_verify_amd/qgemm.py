"""Python binding of ``libqgemm.so`` (argument marshalling only).

Every step of the sweep runs in the HIP library; this module turns torch
device tensors into the plain pointers and sizes of the C boundary
(``include/qgemm.h``) and raises on a non-OK status.  There is no fallback:
if the library is missing or a call fails, it raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NONFINITE, ERR_HIP = 0, 1, 2, 3, 4
PATH_AUTO, PATH_GEMV, PATH_MFMA = 0, 1, 2
MAX_M = 64
GEMV_MAX_M = 8
FMT_Q4, FMT_Q5, FMT_Q4_G64, FMT_Q4_ZP = 4, 5, 0x104, 0x204

# every symbol the boundary header declares
EXPORTS = (
    "qgemm_packed_bytes", "qgemm_pack", "qgemm_workspace_bytes", "qgemm_workspace_init",
    "qgemm_sweep", "qgemm_sweep_path", "qgemm_validate", "qgemm_auto_path",
    "qgemm_status_string", "qgemm_verify_workspace_bytes", "qgemm_verify_head",
    "qgemm_round_workspace_bytes", "qgemm_round_create", "qgemm_round_launch", "qgemm_round_kernels",
    "qgemm_round_destroy", "qgemm_attn_workspace_bytes", "qgemm_attn_verify", "qgemm_sweep_noalloc",
    "qgemm_round_cache_create", "qgemm_round_cache_run", "qgemm_round_cache_stats", "qgemm_round_cache_destroy",
)
ROUND_CACHE_MAX = 4096
NOALLOC_SCRATCH_BYTES = 64 << 20
KV_FP16, KV_FP8 = 0, 1
ATTN_HKV, ATTN_GROUP, ATTN_D, ATTN_MAX_W, ATTN_MAX_SLOTS = 4, 6, 256, 16, 16
MAX_SLOTS = 64


class QgemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class Job(ctypes.Structure):
    """Mirror of ``qgemm_job``."""
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("X", ctypes.c_void_p),
        ("Y", ctypes.c_void_p),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("ldx", ctypes.c_int64),
        ("ldy", ctypes.c_int64),
        ("M", ctypes.c_int32),
        ("bits", ctypes.c_int32),
    ]


class Slot(ctypes.Structure):
    """Mirror of ``qgemm_slot``: panel rows row0 .. row0 + ndraft."""
    _fields_ = [("row0", ctypes.c_int32), ("ndraft", ctypes.c_int32)]


class AttnSlot(ctypes.Structure):
    """Mirror of ``qgemm_attn_slot``."""
    _fields_ = [("Q", ctypes.c_void_p), ("K", ctypes.c_void_p), ("V", ctypes.c_void_p), ("O", ctypes.c_void_p),
                ("L", ctypes.c_int32), ("W", ctypes.c_int32)]


class RoundSweep(ctypes.Structure):
    """Mirror of ``qgemm_round_sweep``."""
    _fields_ = [("jobs", ctypes.POINTER(Job)), ("njobs", ctypes.c_int32), ("path", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        jp = ctypes.POINTER(Job)
        L.qgemm_packed_bytes.argtypes = [ci, i64, i64]
        L.qgemm_packed_bytes.restype = sz
        L.qgemm_pack.argtypes = [vp, i64, i64, i64, ci, vp, vp]
        L.qgemm_pack.restype = ci
        L.qgemm_workspace_bytes.argtypes = [jp, ci, ci]
        L.qgemm_workspace_bytes.restype = sz
        L.qgemm_workspace_init.argtypes = [vp, sz, vp]
        L.qgemm_workspace_init.restype = ci
        L.qgemm_sweep.argtypes = [jp, ci, vp, sz, vp]
        L.qgemm_sweep.restype = ci
        L.qgemm_sweep_path.argtypes = [jp, ci, ci, vp, sz, vp]
        L.qgemm_sweep_path.restype = ci
        L.qgemm_sweep_noalloc.argtypes = [jp, ci, ci, vp]
        L.qgemm_sweep_noalloc.restype = ci
        L.qgemm_validate.argtypes = [jp, ci, ci, vp, sz]
        L.qgemm_validate.restype = ci
        L.qgemm_auto_path.argtypes = [ci]
        L.qgemm_auto_path.restype = ci
        L.qgemm_status_string.argtypes = [ci]
        L.qgemm_status_string.restype = ctypes.c_char_p
        L.qgemm_verify_workspace_bytes.argtypes = [jp]
        L.qgemm_verify_workspace_bytes.restype = sz
        L.qgemm_verify_head.argtypes = [jp, vp, ctypes.POINTER(Slot), ci, vp, vp, vp, vp, sz, vp]
        L.qgemm_verify_head.restype = ci
        rp = ctypes.POINTER(RoundSweep)
        L.qgemm_round_workspace_bytes.argtypes = [rp, ci, jp]
        L.qgemm_round_workspace_bytes.restype = sz
        L.qgemm_round_create.argtypes = [rp, ci, jp, vp, ctypes.POINTER(Slot), ci, vp, vp, vp, vp, sz, vp,
                                         ctypes.POINTER(vp)]
        L.qgemm_round_create.restype = ci
        L.qgemm_round_launch.argtypes = [vp, vp]
        L.qgemm_round_launch.restype = ci
        L.qgemm_round_kernels.argtypes = [vp]
        L.qgemm_round_kernels.restype = ci
        L.qgemm_round_destroy.argtypes = [vp]
        L.qgemm_round_destroy.restype = None
        L.qgemm_round_cache_create.argtypes = [ci, ctypes.POINTER(vp)]
        L.qgemm_round_cache_create.restype = ci
        L.qgemm_round_cache_run.argtypes = [vp, rp, ci, jp, vp, ctypes.POINTER(Slot), ci, vp, vp, vp, vp,
                                            ctypes.POINTER(ci)]
        L.qgemm_round_cache_run.restype = ci
        u64p = ctypes.POINTER(ctypes.c_uint64)
        L.qgemm_round_cache_stats.argtypes = [vp, ctypes.POINTER(ci), u64p, u64p, u64p]
        L.qgemm_round_cache_stats.restype = ci
        L.qgemm_round_cache_destroy.argtypes = [vp]
        L.qgemm_round_cache_destroy.restype = None
        ap = ctypes.POINTER(AttnSlot)
        L.qgemm_attn_workspace_bytes.argtypes = [ap, ci, ci]
        L.qgemm_attn_workspace_bytes.restype = sz
        L.qgemm_attn_verify.argtypes = [ap, ci, ci, ctypes.c_float, vp, sz, vp]
        L.qgemm_attn_verify.restype = ci
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qgemm_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise QgemmError(status, what)


def _stream_ptr(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def packed_bytes(bits: int, N: int, K: int) -> int:
    return int(lib().qgemm_packed_bytes(bits, N, K))


def auto_path(M: int) -> int:
    return int(lib().qgemm_auto_path(M))


def pack(W, bits: int, out=None, stream=None):
    """Quantize and pack a CUDA fp32 [N, K] tensor; returns the uint8 buffer."""
    import torch

    assert W.is_cuda and W.dtype == torch.float32 and W.dim() == 2 and W.stride(1) == 1
    N, K = W.shape
    nbytes = packed_bytes(bits, N, K)
    if nbytes == 0:
        raise QgemmError(ERR_INVALID_ARG, "qgemm_packed_bytes")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    assert out.numel() >= nbytes and out.is_cuda
    _check(lib().qgemm_pack(W.data_ptr(), W.stride(0), N, K, bits, out.data_ptr(),
                            _stream_ptr(stream)), "qgemm_pack")
    return out


def make_job(packed, bits: int, N: int, K: int, X, Y, M: int) -> Job:
    """Job for packed [N, K] weights, X fp16 [>=M, K] and Y fp32 [>=M, N] tensors."""
    return Job(packed.data_ptr(), X.data_ptr(), Y.data_ptr(), N, K, X.stride(0), Y.stride(0), M, bits)


def job_array(jobs):
    arr = (Job * len(jobs))(*jobs)
    return arr


def workspace_bytes(jobs, path: int = PATH_AUTO) -> int:
    arr = job_array(jobs)
    return int(lib().qgemm_workspace_bytes(arr, len(jobs), path))


class Workspace:
    """A zero-initialised device workspace large enough for a set of sweeps."""

    def __init__(self, nbytes: int, device="cuda", stream=None):
        import torch

        nbytes = max(256, (int(nbytes) + 255) // 256 * 256)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _check(lib().qgemm_workspace_init(self.buf.data_ptr(), nbytes, _stream_ptr(stream)),
               "qgemm_workspace_init")

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    @property
    def nbytes(self) -> int:
        return self.buf.numel()


def sweep(jobs, workspace: Workspace, path: int = PATH_AUTO, stream=None) -> None:
    arr = job_array(jobs)
    _check(lib().qgemm_sweep_path(arr, len(jobs), path, workspace.ptr, workspace.nbytes,
                                  _stream_ptr(stream)), "qgemm_sweep_path")


def sweep_noalloc(jobs, path: int = PATH_AUTO, stream=None) -> None:
    """As ``sweep`` on the library's static per-device scratch (no workspace,
    no device allocation); job sets needing more than NOALLOC_SCRATCH_BYTES
    are refused."""
    arr = job_array(jobs)
    st = lib().qgemm_sweep_noalloc(arr, len(jobs), path, _stream_ptr(stream))
    if st == ERR_INVALID_ARG:
        need = workspace_bytes(jobs, path)
        if need > NOALLOC_SCRATCH_BYTES:
            raise QgemmError(st, f"qgemm_sweep_noalloc (the jobs need {need} bytes of scratch, more "
                                 f"than the {NOALLOC_SCRATCH_BYTES} of the static scratch)")
    _check(st, "qgemm_sweep_noalloc")


def validate(jobs, path: int = PATH_AUTO, workspace_ptr: int = 0, ws_bytes: int = 0) -> int:
    arr = job_array(jobs)
    return int(lib().qgemm_validate(arr, len(jobs), path, workspace_ptr, ws_bytes))


def sweep_one(packed, bits: int, N: int, K: int, X, M: int, Y=None, path: int = PATH_AUTO,
              stream=None):
    """Convenience: one matrix, fresh workspace, returns Y fp32 [M, N] (a view
    of rows padded to a multiple of four floats, the row stride the sweep
    requires, when no Y is given)."""
    import torch

    if Y is None:
        Y = torch.empty((M, (N + 3) // 4 * 4), dtype=torch.float32, device=packed.device)[:, :N]
    job = make_job(packed, bits, N, K, X, Y, M)
    ws = Workspace(workspace_bytes([job], path), device=packed.device, stream=stream)
    sweep([job], ws, path, stream)
    return Y


def make_head_job(packed, bits: int, N: int, K: int, X, M: int, Y=None) -> Job:
    """Verify-head job: like make_job, but Y may be None (logits not written)."""
    if Y is None:
        return Job(packed.data_ptr(), X.data_ptr(), None, N, K, X.stride(0), 0, M, bits)
    return make_job(packed, bits, N, K, X, Y, M)


def verify_workspace_bytes(head: Job) -> int:
    return int(lib().qgemm_verify_workspace_bytes(ctypes.byref(head)))


def slot_array(slots):
    """(row0, ndraft) pairs -> a ``qgemm_slot`` array."""
    return (Slot * len(slots))(*[Slot(int(r), int(d)) for r, d in slots])


def verify_head(head: Job, drafts, slots, argmax, accepted, workspace: Workspace, maxlogit=None,
                stream=None) -> None:
    """Greedy verify: argmax int32 [M], accepted int32 [len(slots)] (device
    tensors, written), drafts int32 [M] device tensor or None, slots a list of
    (row0, ndraft) or a slot_array."""
    arr = slots if isinstance(slots, ctypes.Array) else slot_array(slots)
    _check(lib().qgemm_verify_head(ctypes.byref(head), drafts.data_ptr() if drafts is not None else None,
                                   arr, len(arr), argmax.data_ptr(),
                                   maxlogit.data_ptr() if maxlogit is not None else None,
                                   accepted.data_ptr(), workspace.ptr, workspace.nbytes,
                                   _stream_ptr(stream)), "qgemm_verify_head")


def round_sweeps(sweeps):
    """[(jobs, path), ...] -> a ``qgemm_round_sweep`` array (the job arrays are
    kept alive on it)."""
    arrs = [job_array(j) for j, _ in sweeps]
    out = (RoundSweep * len(sweeps))(*[RoundSweep(a, len(a), int(p)) for a, (_, p) in zip(arrs, sweeps)])
    out._keep = arrs
    return out


def round_workspace_bytes(sweeps, head: Job | None = None) -> int:
    arr = sweeps if isinstance(sweeps, ctypes.Array) else round_sweeps(sweeps)
    return int(lib().qgemm_round_workspace_bytes(arr, len(arr), ctypes.byref(head) if head is not None else None))


class Round:
    """A recorded round (``qgemm_round``): sweeps in order, then optionally
    the verify head, replayed as one HIP graph."""

    def __init__(self, sweeps, workspace: "Workspace", head: Job | None = None, drafts=None, slots=(),
                 argmax=None, accepted=None, maxlogit=None, stream=None):
        self._sweeps = sweeps if isinstance(sweeps, ctypes.Array) else round_sweeps(sweeps)
        self._head = head
        self._slots = slot_array(slots) if slots else None
        self.workspace = workspace
        h = ctypes.c_void_p()
        ptr = lambda t: t.data_ptr() if t is not None else None
        _check(lib().qgemm_round_create(self._sweeps, len(self._sweeps),
                                        ctypes.byref(head) if head is not None else None, ptr(drafts),
                                        self._slots, len(self._slots) if self._slots else 0, ptr(argmax),
                                        ptr(maxlogit), ptr(accepted), workspace.ptr, workspace.nbytes,
                                        _stream_ptr(stream), ctypes.byref(h)), "qgemm_round_create")
        self.handle = h.value

    @property
    def kernels(self) -> int:
        return int(lib().qgemm_round_kernels(self.handle))

    def launch(self, stream=None) -> None:
        _check(lib().qgemm_round_launch(self.handle, _stream_ptr(stream)), "qgemm_round_launch")

    def destroy(self) -> None:
        if self.handle:
            lib().qgemm_round_destroy(self.handle)
            self.handle = None


class RoundCache:
    """Rounds keyed by what a recording fixes (``qgemm_round_cache``):
    ``run`` replays a cached round or records a new one, evicting the least
    recently used past the capacity."""

    def __init__(self, capacity: int = 64):
        h = ctypes.c_void_p()
        _check(lib().qgemm_round_cache_create(int(capacity), ctypes.byref(h)), "qgemm_round_cache_create")
        self.handle = h.value

    def run(self, sweeps, head: Job | None = None, drafts=None, slots=(), argmax=None, accepted=None,
            maxlogit=None, stream=None) -> bool:
        """One round; True when it replayed a cached one."""
        arr = sweeps if isinstance(sweeps, ctypes.Array) else round_sweeps(sweeps)
        sl = slot_array(slots) if slots else None
        hit = ctypes.c_int(0)
        ptr = lambda t: t.data_ptr() if t is not None else None
        _check(lib().qgemm_round_cache_run(self.handle, arr, len(arr),
                                           ctypes.byref(head) if head is not None else None, ptr(drafts), sl,
                                           len(sl) if sl else 0, ptr(argmax), ptr(maxlogit), ptr(accepted),
                                           _stream_ptr(stream), ctypes.byref(hit)), "qgemm_round_cache_run")
        return bool(hit.value)

    def stats(self) -> dict:
        size, hits, misses, ev = ctypes.c_int(), ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
        _check(lib().qgemm_round_cache_stats(self.handle, ctypes.byref(size), ctypes.byref(hits),
                                             ctypes.byref(misses), ctypes.byref(ev)), "qgemm_round_cache_stats")
        return {"size": size.value, "hits": hits.value, "misses": misses.value, "evictions": ev.value}

    def destroy(self) -> None:
        if self.handle:
            lib().qgemm_round_cache_destroy(self.handle)
            self.handle = None


def attn_slots(slots):
    """[(Q, K, V, O, L, W), ...] of device tensors / sizes -> a ``qgemm_attn_slot`` array."""
    return (AttnSlot * len(slots))(*[AttnSlot(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), int(L), int(W))
                                     for Q, K, V, O, L, W in slots])


def attn_workspace_bytes(slots, kv: int) -> int:
    arr = slots if isinstance(slots, ctypes.Array) else attn_slots(slots)
    return int(lib().qgemm_attn_workspace_bytes(arr, len(arr), kv))


def attn_verify(slots, kv: int, scale: float, workspace: "Workspace", stream=None) -> None:
    arr = slots if isinstance(slots, ctypes.Array) else attn_slots(slots)
    _check(lib().qgemm_attn_verify(arr, len(arr), kv, scale, workspace.ptr, workspace.nbytes, _stream_ptr(stream)),
           "qgemm_attn_verify")
