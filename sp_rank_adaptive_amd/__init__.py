"""Python binding of libflashoverlap.so, the one-GPU FlashOverlap hot path.

Argument marshalling only: every step of the path runs in the library's HIP
kernels for gfx950 (include/flashoverlap.h documents each entry point).  The
functions keep the C names.  Tensors are torch tensors on the current device
(torch provides device memory and streams); pointers may also be passed as
plain integers.  A non-OK status raises FoError.

There is no fallback: when the library has not been built this module raises
on first use.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashoverlap.so")

FO_OK, FO_ERR_NULL, FO_ERR_SHAPE, FO_ERR_ALIGN, FO_ERR_DTYPE = 0, 1, 2, 3, 4
FO_ERR_ORDER, FO_ERR_SCHEDULE, FO_ERR_WORKSPACE, FO_ERR_HIP = 5, 6, 7, 8
FO_ERR_TIMEOUT, FO_ERR_ALIAS = 9, 10
FO_F32, FO_BF16 = 0, 1
FO_SCHED_READY_FIRST, FO_SCHED_STRICT = 0, 1
FO_LINK_RING, FO_LINK_MESH = 0, 1
FO_MAX_CHUNKS = 64

FO_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("fo_workspace_bytes", "fo_ag_gemm", "fo_ag_gemm_noalloc", "fo_a2a_gemm", "fo_qsa_workspace_bytes", "fo_qsa_attention",
           "fo_gemm_rs", "fo_gemm_rs_reduce", "fo_gemm_rs_ring", "fo_chunk_reduce",
           "fo_emulate_arrivals", "fo_emulate_arrivals_gated", "fo_emulate_sends", "fo_plan_ag_schedule", "fo_plan_calibrate", "fo_plan_link_arrivals",
           "fo_plan_ag_stream", "fo_plan_rs_form", "fo_device_info", "fo_status_string",
           "fo_last_hip_error")


class FoError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {fo_status_string(status)} (status {status})"
        if status == FO_ERR_HIP:
            msg += f": {fo_last_hip_error()}"
        super().__init__(msg)
        self.status = status


class _Sched(ctypes.Structure):
    _fields_ = [
        ("nchunks", ctypes.c_int32),
        ("local", ctypes.c_int32),
        ("order", ctypes.POINTER(ctypes.c_int32)),
        ("arrived", ctypes.c_void_p),
        ("epoch", ctypes.c_uint32),
        ("mode", ctypes.c_uint32),
        ("timeout_ns", ctypes.c_uint64),
        ("status", ctypes.c_void_p),
        ("stamps", ctypes.c_void_p),
        ("split", ctypes.POINTER(ctypes.c_int32)),
        ("max_workgroups", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class PlanCalib(ctypes.Structure):
    """struct fo_plan_calib: measured facts of a launch shape (<= 0: default)."""
    _fields_ = [
        ("gemm_tflops", ctypes.c_double),
        ("alone_speedup", ctypes.c_double),
        ("flag_latency_ns", ctypes.c_double),
        ("reserve_latency_ns", ctypes.c_double),
        ("unit_fixed_ns", ctypes.c_double),
        ("hbm_gbps", ctypes.c_double),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libflashoverlap.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m sp_rank_adaptive_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, S = ctypes.c_void_p, ctypes.POINTER(_Sched)
    i32, i64, u32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    L.fo_workspace_bytes.restype = sz
    L.fo_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.fo_ag_gemm.restype = i32
    L.fo_ag_gemm.argtypes = [P, P, P, i32, i64, i64, i64, S, P, sz, P]
    L.fo_ag_gemm_noalloc.restype = i32
    L.fo_ag_gemm_noalloc.argtypes = [P, P, P, i32, i64, i64, i64, S, P]
    L.fo_a2a_gemm.restype = i32
    L.fo_a2a_gemm.argtypes = [P, P, P, i32, i64, i64, i64, S, P, sz, P]
    L.fo_qsa_workspace_bytes.restype = sz
    L.fo_qsa_workspace_bytes.argtypes = [i64, i32, i32, i32]
    L.fo_qsa_attention.restype = i32
    L.fo_qsa_attention.argtypes = [P, P, i32, i64, i32, i32, i32, S, P, sz, P]
    L.fo_gemm_rs.restype = i32
    L.fo_gemm_rs.argtypes = [P, P, P, P, i64, i64, i64, S, P, sz, P]
    L.fo_gemm_rs_reduce.restype = i32
    L.fo_gemm_rs_reduce.argtypes = [P, P, P, P, P, i32, P, i64, i64, i64, S, P, sz, P]
    L.fo_gemm_rs_ring.restype = i32
    L.fo_gemm_rs_ring.argtypes = [P, P, P, P, P, i32, P, i64, i64, i64, S, P, sz, P]
    L.fo_chunk_reduce.restype = i32
    L.fo_chunk_reduce.argtypes = [P, i32, P, i64, S, P]
    L.fo_emulate_arrivals.restype = i32
    L.fo_emulate_arrivals.argtypes = [P, P, P, P, P, P, i32, P, u32, P, P]
    L.fo_emulate_arrivals_gated.restype = i32
    L.fo_emulate_arrivals_gated.argtypes = [P, ctypes.c_uint64, P, P, P, P, P, P, i32, P, u32, P, P]
    L.fo_emulate_sends.restype = i32
    L.fo_emulate_sends.argtypes = [P, u32, P, P, P, P, P, i32, ctypes.c_uint64, P, P, P]
    L.fo_plan_ag_schedule.restype = i32
    L.fo_plan_ag_schedule.argtypes = [i64, i64, i64, i32, i32, P, ctypes.c_double, i32, P, P, P]
    L.fo_plan_calibrate.restype = i32
    L.fo_plan_calibrate.argtypes = [i64, i64, i64, i32, ctypes.c_double, ctypes.c_double, ctypes.c_double, i32,
                                    ctypes.POINTER(PlanCalib)]
    L.fo_plan_link_arrivals.restype = i32
    L.fo_plan_link_arrivals.argtypes = [i32, i32, i64, ctypes.c_double, i32, i32, P]
    L.fo_plan_ag_stream.restype = i32
    L.fo_plan_ag_stream.argtypes = [i64, i64, i64, i32, i32, ctypes.c_double, i32, ctypes.POINTER(PlanCalib), i32,
                                    P, P, P, P]
    L.fo_plan_rs_form.restype = i32
    L.fo_plan_rs_form.argtypes = [i64, i64, i64, i32, i32, P, ctypes.POINTER(PlanCalib), i32, P, P]
    L.fo_device_info.restype = i32
    L.fo_device_info.argtypes = [P, P, P]
    L.fo_status_string.restype = ctypes.c_char_p
    L.fo_status_string.argtypes = [i32]
    L.fo_last_hip_error.restype = ctypes.c_char_p
    L.fo_last_hip_error.argtypes = []
    _lib = L
    return L


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class Schedule:
    """The chunk-order / arrival-schedule argument (struct fo_schedule)."""
    nchunks: int
    local: int = 0
    order: Optional[Sequence[int]] = None
    arrived: object = None          # device uint32/int32 tensor [R] or pointer
    epoch: int = 1
    mode: int = FO_SCHED_READY_FIRST
    timeout_ns: int = 0
    status: object = None           # device int32 tensor [1]
    stamps: object = None           # device int64 tensor
    split: Optional[Sequence[int]] = None
    max_workgroups: int = 0

    def _c(self):
        s = _Sched()
        s.nchunks = self.nchunks
        s.local = self.local
        keep = []
        if self.order is not None:
            arr = (ctypes.c_int32 * len(self.order))(*[int(v) for v in self.order])
            keep.append(arr)
            s.order = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
        if self.split is not None:
            arr = (ctypes.c_int32 * len(self.split))(*[int(v) for v in self.split])
            keep.append(arr)
            s.split = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
        s.arrived = _ptr(self.arrived)
        s.epoch = self.epoch
        s.mode = self.mode
        s.timeout_ns = self.timeout_ns
        s.status = _ptr(self.status)
        s.stamps = _ptr(self.stamps)
        s.max_workgroups = self.max_workgroups
        return s, keep


def _check(st: int, where: str) -> None:
    if st != FO_OK:
        raise FoError(st, where)


def fo_status_string(status: int) -> str:
    return lib().fo_status_string(status).decode()


def fo_last_hip_error() -> str:
    return lib().fo_last_hip_error().decode()


def fo_workspace_bytes(m: int, n: int, k: int, nchunks: int) -> int:
    return int(lib().fo_workspace_bytes(m, n, k, nchunks))


def fo_plan_ag_schedule(m, n, k, nchunks, local, arrival_ns, gemm_tflops=0.0, num_workgroups=0):
    """Schedule model for fo_ag_gemm: (order, split, predicted_ns) where
    predicted_ns[i] is the predicted completion with the last-landing chunk
    split (1, 2, 4, 8)[i] ways (-1 where not possible)."""
    R = int(nchunks)
    arr = (ctypes.c_int64 * R)(*[int(v) for v in arrival_ns])
    order = (ctypes.c_int32 * R)()
    split = (ctypes.c_int32 * R)()
    pred = (ctypes.c_int64 * 4)()
    _check(lib().fo_plan_ag_schedule(int(m), int(n), int(k), R, int(local), arr, float(gemm_tflops),
                                     int(num_workgroups), order, split, pred), "fo_plan_ag_schedule")
    return list(order), list(split), list(pred)


def fo_plan_calibrate(m, n, k, nchunks, all_present_ns, chunk_alone_ns=0.0, tail_unsplit_ns=0.0,
                      num_workgroups=0) -> PlanCalib:
    """Calibration of the schedule model from measured launches."""
    out = PlanCalib()
    _check(lib().fo_plan_calibrate(int(m), int(n), int(k), int(nchunks), float(all_present_ns), float(chunk_alone_ns),
                                   float(tail_unsplit_ns), int(num_workgroups), ctypes.byref(out)),
           "fo_plan_calibrate")
    return out


def fo_plan_link_arrivals(nchunks, local, chunk_bytes, link_gbps, topology=FO_LINK_RING, sub=1):
    """Landing time (ns) of every message c * sub + j (0 for the local chunk)."""
    arr = (ctypes.c_int64 * (int(nchunks) * int(sub)))()
    _check(lib().fo_plan_link_arrivals(int(nchunks), int(local), int(chunk_bytes), float(link_gbps), int(topology),
                                       int(sub), arr), "fo_plan_link_arrivals")
    return list(arr)


def fo_plan_ag_stream(m, n, k, nchunks, local, link_gbps, topology=FO_LINK_RING, calib=None, num_workgroups=0):
    """(sub, order, split, predicted): messages per peer chunk, and the order
    and split vector over the R * sub pieces; predicted[i][j] = completion
    with (1, 2, 4, 8)[i] messages and the last piece split (1, 2, 4, 8)[j]."""
    sub = ctypes.c_int32()
    order = (ctypes.c_int32 * FO_MAX_CHUNKS)()
    split = (ctypes.c_int32 * FO_MAX_CHUNKS)()
    pred = (ctypes.c_int64 * 16)()
    _check(lib().fo_plan_ag_stream(int(m), int(n), int(k), int(nchunks), int(local), float(link_gbps), int(topology),
                                   None if calib is None else ctypes.byref(calib), int(num_workgroups),
                                   ctypes.byref(sub), order, split, pred), "fo_plan_ag_stream")
    r2 = int(nchunks) * sub.value
    return sub.value, list(order)[:r2], list(split)[:r2], [list(pred)[4 * i:4 * i + 4] for i in range(4)]


def fo_plan_rs_form(m, n, k, nchunks, local, arrival_ns, calib=None, num_workgroups=0):
    """(form, predicted): 0 GEMM-RS then reduce, 1 fused, 2 ring."""
    R = int(nchunks)
    arr = (ctypes.c_int64 * R)(*[int(v) for v in arrival_ns])
    form = ctypes.c_int32()
    pred = (ctypes.c_int64 * 3)()
    _check(lib().fo_plan_rs_form(int(m), int(n), int(k), R, int(local), arr,
                                 None if calib is None else ctypes.byref(calib), int(num_workgroups),
                                 ctypes.byref(form), pred), "fo_plan_rs_form")
    return form.value, list(pred)


def fo_device_info():
    """(number of CUs, LDS bytes per CU, device wall-clock rate in Hz)."""
    cus, lds, hz = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_uint64()
    _check(lib().fo_device_info(ctypes.byref(cus), ctypes.byref(lds), ctypes.byref(hz)),
           "fo_device_info")
    return cus.value, lds.value, hz.value


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FO_F32
    if t.dtype == torch.bfloat16:
        return FO_BF16
    return -1


def fo_ag_gemm(x, w, y, sched: Schedule, ws, stream=None, *, raise_on_error=True) -> int:
    """Y = AllGather(X) * W chunk by chunk (x [m,k] bf16, w [n,k] bf16,
    y [m,n] fp32 or bf16, ws uint8 workspace)."""
    m, k = x.shape
    n = w.shape[0]
    s, keep = sched._c()
    st = lib().fo_ag_gemm(_ptr(x), _ptr(w), _ptr(y), _dtype_code(y), m, n, k,
                          ctypes.byref(s), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream(stream))
    del keep
    if raise_on_error:
        _check(st, "fo_ag_gemm")
    return st


def fo_ag_gemm_noalloc(x, w, y, sched: Schedule, stream=None, *, raise_on_error=True) -> int:
    """fo_ag_gemm with the library's per-GPU scratch array as its workspace
    (no workspace argument; nothing is allocated)."""
    m, k = x.shape
    n = w.shape[0]
    s, keep = sched._c()
    st = lib().fo_ag_gemm_noalloc(_ptr(x), _ptr(w), _ptr(y), _dtype_code(y), m, n, k,
                                  ctypes.byref(s), _stream(stream))
    del keep
    if raise_on_error:
        _check(st, "fo_ag_gemm_noalloc")
    return st


def fo_a2a_gemm(pieces, w, y, sched: Schedule, ws, stream=None, *, raise_on_error=True) -> int:
    """y = [pieces[0] | ... | pieces[P-1]] * W, each piece [m, k/P] bf16
    multiplied once it has landed (w [n, k] bf16, y [m, n] fp32 or bf16)."""
    P = len(pieces)
    m, kp = pieces[0].shape
    n, k = w.shape
    arr = (ctypes.c_void_p * P)(*[_ptr(t) for t in pieces])
    s, keep = sched._c()
    st = lib().fo_a2a_gemm(arr, _ptr(w), _ptr(y), _dtype_code(y), m, n, k, ctypes.byref(s), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream))
    del keep
    if raise_on_error:
        _check(st, "fo_a2a_gemm")
    return st


def fo_qsa_workspace_bytes(seq: int, heads: int, head_dim: int, nchunks: int) -> int:
    return int(lib().fo_qsa_workspace_bytes(seq, heads, head_dim, nchunks))


def fo_qsa_attention(qkv, o, heads: int, head_dim: int, causal: bool, sched: Schedule, ws, stream=None, *,
                     raise_on_error=True) -> int:
    """Query-split attention: qkv [S, 3*H*d] bf16 -> o [S, H*d] fp32 or bf16."""
    seq = qkv.shape[0]
    s, keep = sched._c()
    st = lib().fo_qsa_attention(_ptr(qkv), _ptr(o), _dtype_code(o), seq, heads, head_dim, int(bool(causal)),
                                ctypes.byref(s), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    del keep
    if raise_on_error:
        _check(st, "fo_qsa_attention")
    return st


def fo_gemm_rs(x, w, partial, done, sched: Schedule, ws, stream=None, *, raise_on_error=True) -> int:
    """partial[rows of c] = X[rows of c] * W for every chunk, local chunk last."""
    m, k = x.shape
    n = w.shape[0]
    s, keep = sched._c()
    st = lib().fo_gemm_rs(_ptr(x), _ptr(w), _ptr(partial), _ptr(done), m, n, k,
                          ctypes.byref(s), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream(stream))
    del keep
    if raise_on_error:
        _check(st, "fo_gemm_rs")
    return st


def fo_gemm_rs_reduce(x, w, partial, done, shard, incoming, sched: Schedule, ws, stream=None, *,
                      raise_on_error=True) -> int:
    """fo_gemm_rs plus, in the same launch, shard = partial[rows of local] +
    incoming peers in priority order (fp32; shard fp32 or bf16).  incoming:
    R tensors or None (the entry at local is ignored)."""
    m, k = x.shape
    n = w.shape[0]
    R = len(incoming)
    arr = (ctypes.c_void_p * R)(*[_ptr(t) for t in incoming])
    s, keep = sched._c()
    st = lib().fo_gemm_rs_reduce(_ptr(x), _ptr(w), _ptr(partial), _ptr(done), _ptr(shard),
                                 _dtype_code(shard), arr, m, n, k, ctypes.byref(s), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream))
    del keep
    if raise_on_error:
        _check(st, "fo_gemm_rs_reduce")
    return st


def fo_gemm_rs_ring(x, w, partial, done, shard, incoming, sched: Schedule, ws, stream=None, *,
                    raise_on_error=True) -> int:
    """Ring form: fo_gemm_rs plus, in the same launch, partial[rows of c] +=
    incoming[c] for every peer chunk with an incoming partial (in place) and
    shard = partial[rows of local] + incoming[local].  incoming: R tensors or
    None, indexed by chunk."""
    m, k = x.shape
    n = w.shape[0]
    R = len(incoming)
    arr = (ctypes.c_void_p * R)(*[_ptr(t) for t in incoming])
    s, keep = sched._c()
    st = lib().fo_gemm_rs_ring(_ptr(x), _ptr(w), _ptr(partial), _ptr(done), _ptr(shard),
                               _dtype_code(shard), arr, m, n, k, ctypes.byref(s), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream))
    del keep
    if raise_on_error:
        _check(st, "fo_gemm_rs_ring")
    return st


def fo_chunk_reduce(dst, srcs, sched: Schedule, stream=None, *, raise_on_error=True) -> int:
    """dst = srcs[local] + peers in order (fp32 accumulate)."""
    R = len(srcs)
    arr = (ctypes.c_void_p * R)(*[_ptr(t) for t in srcs])
    s, keep = sched._c()
    st = lib().fo_chunk_reduce(_ptr(dst), _dtype_code(dst), arr, dst.numel(),
                               ctypes.byref(s), _stream(stream))
    del keep
    if raise_on_error:
        _check(st, "fo_chunk_reduce")
    return st


def fo_emulate_arrivals(dsts, srcs, release_ns, chunk_ids, arrived, epoch, stamps,
                        issue_ns=None, nbytes=None, stream=None, gate=None, gate_timeout_ns=0) -> int:
    """Enqueue emulated peer arrivals (SDMA copies + timed epoch flags).
    gate: a device uint64 word (tensor element pointer or int); the timeline
    starts once it is nonzero (fo_emulate_arrivals_gated)."""
    cnt = len(dsts)
    if nbytes is None:
        nbytes = [t.numel() * t.element_size() for t in srcs]
    d = (ctypes.c_void_p * cnt)(*[_ptr(t) for t in dsts])
    s = (ctypes.c_void_p * cnt)(*[_ptr(t) for t in srcs])
    b = (ctypes.c_size_t * cnt)(*[int(v) for v in nbytes])
    rel = (ctypes.c_int64 * cnt)(*[int(v) for v in release_ns])
    iss = None if issue_ns is None else (ctypes.c_int64 * cnt)(*[int(v) for v in issue_ns])
    cid = (ctypes.c_int32 * cnt)(*[int(v) for v in chunk_ids])
    if gate is None:
        st = lib().fo_emulate_arrivals(d, s, b, iss, rel, cid, cnt, _ptr(arrived), epoch,
                                       _ptr(stamps), _stream(stream))
        _check(st, "fo_emulate_arrivals")
    else:
        st = lib().fo_emulate_arrivals_gated(_ptr(gate), int(gate_timeout_ns), d, s, b, iss, rel, cid, cnt,
                                             _ptr(arrived), epoch, _ptr(stamps), _stream(stream))
        _check(st, "fo_emulate_arrivals_gated")
    return st


def fo_emulate_sends(done, epoch, dsts, srcs, chunk_ids, link_ns, stamps, nbytes=None, timeout_ns=0, status=None,
                     stream=None) -> int:
    """Enqueue emulated sends of finished chunks (flag wait, SDMA copy, link
    hold) on `stream`, one after another."""
    cnt = len(dsts)
    if nbytes is None:
        nbytes = [t.numel() * t.element_size() for t in srcs]
    d = (ctypes.c_void_p * cnt)(*[_ptr(t) for t in dsts])
    s = (ctypes.c_void_p * cnt)(*[_ptr(t) for t in srcs])
    b = (ctypes.c_size_t * cnt)(*[int(v) for v in nbytes])
    cid = (ctypes.c_int32 * cnt)(*[int(v) for v in chunk_ids])
    ln = (ctypes.c_int64 * cnt)(*[int(v) for v in link_ns])
    st = lib().fo_emulate_sends(_ptr(done), int(epoch), d, s, b, cid, ln, cnt, int(timeout_ns), _ptr(status),
                                _ptr(stamps), _stream(stream))
    _check(st, "fo_emulate_sends")
    return st
