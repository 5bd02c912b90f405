"""Argument fuzzing of the C ABI on the CPU (hypothesis): random sizes,
chunk counts, local ranks, orders, splits, epochs, modes, workgroup caps,
dtypes and pointers (NULL, aligned, misaligned, overlapping) for the GEMM,
reduce and attention calls.  Validation runs before any HIP call, so every
call must return a defined status without crashing: a validation error for
arguments the header rules out, and otherwise FO_ERR_HIP (this container
has no GPU).  The host arrays the schedule points to always hold the
entries the header asks for; device pointers are never dereferenced here."""
import ctypes

import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st

import sp_rank_adaptive_amd as fo

CODES = {fo.FO_OK, fo.FO_ERR_NULL, fo.FO_ERR_SHAPE, fo.FO_ERR_ALIGN, fo.FO_ERR_DTYPE, fo.FO_ERR_ORDER,
         fo.FO_ERR_SCHEDULE, fo.FO_ERR_WORKSPACE, fo.FO_ERR_HIP, fo.FO_ERR_ALIAS}
PTRS = st.sampled_from([0, 0x10000, 0x10008, 0x20000000, 0x40000000, 0x7f0000000000])
SIZES = st.one_of(st.integers(-3, 3), st.integers(1, 5000), st.sampled_from([1 << 20, 1 << 30, 1 << 31, 1 << 40]))
CHUNKS = st.one_of(st.integers(-1, 17), st.sampled_from([63, 64, 65, 1000]))


@st.composite
def schedules(draw):
    R = draw(CHUNKS)
    n_arr = max(1, min(R, 70))
    s = fo._Sched()
    s.nchunks = R
    s.local = draw(st.integers(-1, 20))
    keep = []
    if draw(st.booleans()):
        arr = (ctypes.c_int32 * n_arr)(*[draw(st.integers(-2, 20)) for _ in range(n_arr)])
        keep.append(arr)
        s.order = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    if draw(st.booleans()):
        arr = (ctypes.c_int32 * n_arr)(*[draw(st.integers(-1, 10)) for _ in range(n_arr)])
        keep.append(arr)
        s.split = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    s.arrived = draw(PTRS)
    s.epoch = draw(st.sampled_from([0, 1, 7, 0xFFFFFFFF]))
    s.mode = draw(st.integers(-1, 3))
    s.timeout_ns = draw(st.sampled_from([0, 1000, 10 ** 12]))
    s.status = draw(PTRS)
    s.stamps = draw(PTRS)
    s.max_workgroups = draw(st.integers(-2, 2000))
    return s, keep, n_arr


@settings(max_examples=400, deadline=None)
@given(schedules(), PTRS, PTRS, PTRS, SIZES, SIZES, SIZES, st.integers(-1, 5), PTRS,
       st.sampled_from([0, 16, 1 << 20, 1 << 40]))
def test_ag_gemm_and_gemm_rs_arguments(sch, x, w, y, m, n, k, dt, ws, wsb):
    s, keep, _ = sch
    L = fo.lib()
    st1 = L.fo_ag_gemm(x, w, y, dt, m, n, k, ctypes.byref(s), ws, wsb, None)
    assert st1 in CODES
    st2 = L.fo_gemm_rs(x, w, y, 0x30000000, m, n, k, ctypes.byref(s), ws, wsb, None)
    assert st2 in CODES
    assert L.fo_workspace_bytes(m, n, k, s.nchunks) >= 0


@settings(max_examples=400, deadline=None)
@given(schedules(), PTRS, st.integers(-1, 5), SIZES, st.lists(PTRS, min_size=70, max_size=70))
def test_chunk_reduce_arguments(sch, dst, dt, n, srcs):
    s, keep, n_arr = sch
    arr = (ctypes.c_void_p * 70)(*srcs)
    st_ = fo.lib().fo_chunk_reduce(dst, dt, arr, n, ctypes.byref(s), None)
    assert st_ in CODES


@settings(max_examples=400, deadline=None)
@given(schedules(), PTRS, PTRS, st.integers(-1, 5), SIZES, st.integers(-1, 40), st.sampled_from([0, 64, 128, 256]),
       st.booleans(), PTRS, st.sampled_from([0, 16, 1 << 30, 1 << 40]))
def test_qsa_attention_arguments(sch, qkv, o, dt, S, H, d, causal, ws, wsb):
    s, keep, _ = sch
    L = fo.lib()
    st_ = L.fo_qsa_attention(qkv, o, dt, S, H, d, int(causal), ctypes.byref(s), ws, wsb, None)
    assert st_ in CODES
    assert L.fo_qsa_workspace_bytes(S, H, d, s.nchunks) >= 0


@settings(max_examples=300, deadline=None)
@given(schedules(), st.lists(PTRS, min_size=70, max_size=70), PTRS, PTRS, st.integers(-1, 5), SIZES, SIZES, SIZES,
       PTRS)
def test_a2a_gemm_arguments(sch, pieces, w, y, dt, m, n, k, ws):
    s, keep, _ = sch
    arr = (ctypes.c_void_p * 70)(*pieces)
    st_ = fo.lib().fo_a2a_gemm(arr, w, y, dt, m, n, k, ctypes.byref(s), ws, 1 << 20, None)
    assert st_ in CODES
