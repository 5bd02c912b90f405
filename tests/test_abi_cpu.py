"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the ctypes struct matches the C layout, and argument
validation rejects bad calls before any HIP call is made."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import sp_rank_adaptive_amd as fo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashoverlap.h")

A = 0x10000          # an aligned fake device address (never dereferenced)
A2 = 0x20000000
WS = 0x40000000


@pytest.fixture(scope="module")
def L():
    return fo.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fo_status|size_t|const char \*)\s*(fo_\w+)\s*\(",
                                 text, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(fo.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", fo.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(fo_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_schedule_struct_layout_matches_header():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "flashoverlap.h"
int main(void){
  printf("%zu", sizeof(fo_schedule));
#define O(f) printf(" %zu", offsetof(fo_schedule, f));
  O(nchunks) O(local) O(order) O(arrived) O(epoch) O(mode) O(timeout_ns) O(status)
  O(stamps) O(split) O(max_workgroups) O(reserved)
  printf("\n"); return 0; }
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        vals = [int(v) for v in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    S = fo._Sched
    py = [ctypes.sizeof(S)] + [getattr(S, f).offset for f, _ in S._fields_]
    assert vals == py


def test_status_strings(L):
    for code in range(0, 11):
        s = fo.fo_status_string(code)
        assert s and s != "unknown status"
    assert fo.fo_status_string(99) == "unknown status"


def test_workspace_bytes(L):
    assert fo.fo_workspace_bytes(4096, 1792, 4096, 8) > 1024
    assert fo.fo_workspace_bytes(4096, 1792, 4096, 7) == 0      # m % R != 0
    assert fo.fo_workspace_bytes(0, 1, 8, 1) == 0
    assert fo.fo_workspace_bytes(64, 64, 64, 65) == 0            # R > max
    assert fo.fo_workspace_bytes(64, 64, 1 << 21, 1) > 0         # largest k
    assert fo.fo_workspace_bytes(64, 64, (1 << 21) + 8, 1) == 0  # k too large


# The tile shapes the GEMM launches may pick (BM x BN).
TILE_SHAPES = [(256, 256), (256, 160), (128, 224), (128, 128)]


@pytest.mark.parametrize("R", [8, 16])
def test_workspace_covers_every_tile_shape(L, R):
    """fo_workspace_bytes must hold 8 split partials of the padded chunk area
    for whichever tile shape the launch picks, plus its counters and ready
    lists, on ragged n (a 224-wide tile pads n further than a 256-wide one)."""
    for mc in (256, 512, 1000, 1024):
        for n in range(2272, 2945, 32):
            ws = fo.fo_workspace_bytes(mc * R, n, 8192, R)
            for bm, bn in TILE_SHAPES:
                tiles = -(-mc // bm) * -(-n // bn)
                counters = 4096 + 2 * R * tiles * 4
                start = (counters + 255) // 256 * 256
                need = start + 8 * tiles * bm * bn * 4
                assert ws >= need, (mc, n, R, bm, bn, ws, need)


def sched(R=4, **kw):
    s = fo.Schedule(nchunks=R, **kw)
    c, keep = s._c()
    return c, keep


def ag(L, x=A, w=A, y=A2, dt=fo.FO_F32, m=256, n=512, k=512, s=None, ws=WS, wsb=1 << 30):
    if s is None:
        s, keep = sched()
    return L.fo_ag_gemm(x, w, y, dt, m, n, k, ctypes.byref(s) if s is not False else None,
                        ws, wsb, None)


def test_ag_gemm_validation(L):
    assert ag(L, x=None) == fo.FO_ERR_NULL
    assert ag(L, s=False) == fo.FO_ERR_NULL
    assert ag(L, dt=7) == fo.FO_ERR_DTYPE
    assert ag(L, m=255) == fo.FO_ERR_SHAPE                  # m % R
    assert ag(L, n=0) == fo.FO_ERR_SHAPE
    assert ag(L, k=12) == fo.FO_ERR_ALIGN                   # k % 8
    assert ag(L, k=(1 << 21) + 8) == fo.FO_ERR_SHAPE        # 32-bit row-block offsets
    assert ag(L, x=A + 8) == fo.FO_ERR_ALIGN
    assert ag(L, y=A) == fo.FO_ERR_ALIAS                    # y overlaps x
    assert ag(L, ws=None) == fo.FO_ERR_WORKSPACE
    assert ag(L, wsb=16) == fo.FO_ERR_WORKSPACE
    s, k1 = sched(order=[0, 1, 1, 2])
    assert ag(L, s=s) == fo.FO_ERR_ORDER
    s, k1 = sched(order=[0, 1, 2, 4])
    assert ag(L, s=s) == fo.FO_ERR_ORDER
    s, k1 = sched(local=4)
    assert ag(L, s=s) == fo.FO_ERR_SCHEDULE
    s, k1 = sched(epoch=0)
    assert ag(L, s=s) == fo.FO_ERR_SCHEDULE
    s, k1 = sched(mode=3)
    assert ag(L, s=s) == fo.FO_ERR_SCHEDULE
    s, k1 = sched(split=[1, 9, 1, 1])
    assert ag(L, s=s) == fo.FO_ERR_SCHEDULE
    s, k1 = sched(R=0)
    assert ag(L, s=s) == fo.FO_ERR_SHAPE
    s, k1 = sched(R=65)
    assert ag(L, s=s) == fo.FO_ERR_SHAPE


def test_gemm_rs_validation(L):
    s, keep = sched()
    assert L.fo_gemm_rs(A, A, None, None, 256, 512, 512, ctypes.byref(s), WS, 1 << 30, None) == fo.FO_ERR_NULL
    s, keep = sched(arrived=A)        # GEMM-RS takes no arrival flags
    assert L.fo_gemm_rs(A, A, A2, None, 256, 512, 512, ctypes.byref(s), WS, 1 << 30, None) == fo.FO_ERR_SCHEDULE
    s, keep = sched()
    assert L.fo_gemm_rs(A, A, A2, None, 256, 512, 500, ctypes.byref(s), WS, 1 << 30, None) == fo.FO_ERR_ALIGN


def test_gemm_rs_reduce_validation(L):
    R, m, n, k = 4, 256, 512, 512
    mc = m // R
    inc_ok = [A2 + 0x1000000 * (q + 1) for q in range(R)]
    shard = A2 + 0x8000000

    def fz(part=A2, sh=shard, dt=fo.FO_F32, inc=inc_ok, nn=n, s=None, x=A, wsb=1 << 30):
        if s is None:
            s, fz.keep = sched()
        arr = None if inc is None else (ctypes.c_void_p * R)(*inc)
        return L.fo_gemm_rs_reduce(x, A + 0x100000, part, None, sh, dt, arr, m, nn, k,
                                   ctypes.byref(s), WS, wsb, None)
    assert fz(x=None) == fo.FO_ERR_NULL
    assert fz(sh=None) == fo.FO_ERR_NULL
    assert fz(inc=None) == fo.FO_ERR_NULL
    nul = list(inc_ok)
    nul[1] = None
    assert fz(inc=nul) == fo.FO_ERR_NULL
    nul[0] = None                                   # the local chunk's entry is ignored:
    nul[1] = inc_ok[1]                              # the call gets as far as the workspace
    assert fz(inc=nul, wsb=16) == fo.FO_ERR_WORKSPACE
    assert fz(dt=7) == fo.FO_ERR_DTYPE
    assert fz(nn=510) == fo.FO_ERR_ALIGN              # n % 4
    assert fz(sh=shard + 4) == fo.FO_ERR_ALIGN
    mis = list(inc_ok)
    mis[2] += 4
    assert fz(inc=mis) == fo.FO_ERR_ALIGN
    s, keep = sched(split=[1, 2, 1, 1])             # the fused launch takes no split
    assert fz(s=s) == fo.FO_ERR_SCHEDULE
    assert fz(sh=A2 + 64) == fo.FO_ERR_ALIAS          # shard inside the partials
    over = list(inc_ok)
    over[3] = shard + mc * n * 4 - 16                 # incoming overlaps the shard
    assert fz(inc=over) == fo.FO_ERR_ALIAS
    over[3] = A2 + 4096                               # incoming inside the partials
    assert fz(inc=over) == fo.FO_ERR_ALIAS


def test_gemm_rs_ring_validation(L):
    R, m, n, k = 4, 256, 512, 512
    mc = m // R
    inc_ok = [A2 + 0x1000000 * (q + 1) for q in range(R)]
    shard = A2 + 0x8000000

    def rg(sh=shard, dt=fo.FO_F32, inc=inc_ok, nn=n, wsb=1 << 30):
        s, keep = sched()
        arr = None if inc is None else (ctypes.c_void_p * R)(*inc)
        return L.fo_gemm_rs_ring(A, A + 0x100000, A2, None, sh, dt, arr, m, nn, k,
                                 ctypes.byref(s), WS, wsb, None)
    assert rg(sh=None) == fo.FO_ERR_NULL
    assert rg(inc=None) == fo.FO_ERR_NULL
    assert rg(dt=9) == fo.FO_ERR_DTYPE
    # any entry may be null (no incoming partial): the call gets as far as the workspace
    assert rg(inc=[None] * R, wsb=16) == fo.FO_ERR_WORKSPACE
    assert rg(inc=[inc_ok[0], None, None, inc_ok[3]], wsb=16) == fo.FO_ERR_WORKSPACE
    assert rg(nn=510) == fo.FO_ERR_ALIGN
    mis = list(inc_ok)
    mis[0] += 4                                        # the local chunk's entry is used too
    assert rg(inc=mis) == fo.FO_ERR_ALIGN
    over = list(inc_ok)
    over[0] = A2 + 4096                                # incoming inside the partials
    assert rg(inc=over) == fo.FO_ERR_ALIAS
    over[0] = shard + mc * n * 4 - 16                  # incoming overlapping the shard
    assert rg(inc=over) == fo.FO_ERR_ALIAS


def test_chunk_reduce_validation(L):
    R = 4
    n = 1024
    srcs = (ctypes.c_void_p * R)(*[A + i * 0x100000 for i in range(R)])
    s, keep = sched(R)
    red = L.fo_chunk_reduce
    assert red(None, fo.FO_F32, srcs, n, ctypes.byref(s), None) == fo.FO_ERR_NULL
    assert red(A2, 5, srcs, n, ctypes.byref(s), None) == fo.FO_ERR_DTYPE
    assert red(A2, fo.FO_F32, srcs, 0, ctypes.byref(s), None) == fo.FO_ERR_SHAPE
    assert red(A2, fo.FO_F32, srcs, 1022, ctypes.byref(s), None) == fo.FO_ERR_ALIGN
    assert red(A2 + 4, fo.FO_F32, srcs, n, ctypes.byref(s), None) == fo.FO_ERR_ALIGN
    # dst overlapping a peer source is refused; dst == srcs[local] (fp32) is allowed
    assert red(A + 0x100000, fo.FO_F32, srcs, n, ctypes.byref(s), None) == fo.FO_ERR_ALIAS
    assert red(A, fo.FO_BF16, srcs, n, ctypes.byref(s), None) == fo.FO_ERR_ALIAS
    bad = (ctypes.c_void_p * R)(*[A, A + 64, A + 0x200000, A + 0x300000])
    assert red(A2, fo.FO_F32, bad, n, ctypes.byref(s), None) == fo.FO_ERR_ALIAS
    nul = (ctypes.c_void_p * R)(*[A, None, A + 0x200000, A + 0x300000])
    assert red(A2, fo.FO_F32, nul, n, ctypes.byref(s), None) == fo.FO_ERR_NULL
    s, keep = sched(R, order=[3, 2, 1, 1])
    assert red(A2, fo.FO_F32, srcs, n, ctypes.byref(s), None) == fo.FO_ERR_ORDER


def test_emulate_validation(L):
    P = ctypes.c_void_p
    d = (P * 1)(A)
    s = (P * 1)(A2)
    b = (ctypes.c_size_t * 1)(64)
    rel = (ctypes.c_int64 * 1)(100)
    iss = (ctypes.c_int64 * 1)(200)             # issue after release
    cid = (ctypes.c_int32 * 1)(1)
    em = L.fo_emulate_arrivals
    assert em(d, s, b, None, rel, cid, 0, A, 1, A, None) == fo.FO_OK   # nothing to do
    assert em(d, s, b, None, rel, cid, -1, A, 1, A, None) == fo.FO_ERR_SHAPE
    assert em(d, s, b, None, rel, cid, 1, None, 1, A, None) == fo.FO_ERR_NULL
    assert em(d, s, b, None, rel, cid, 1, A, 1, None, None) == fo.FO_ERR_NULL
    assert em(d, s, b, None, rel, cid, 1, A, 0, A, None) == fo.FO_ERR_SCHEDULE
    assert em(d, s, b, iss, rel, cid, 1, A, 1, A, None) == fo.FO_ERR_SCHEDULE
    bad = (ctypes.c_int32 * 1)(64)
    assert em(d, s, b, None, rel, bad, 1, A, 1, A, None) == fo.FO_ERR_SCHEDULE
    # the gated form validates the same way before anything is enqueued
    eg = L.fo_emulate_arrivals_gated
    for gate in (None, A):
        assert eg(gate, 0, d, s, b, None, rel, cid, 0, A, 1, A, None) == fo.FO_OK
        assert eg(gate, 0, d, s, b, None, rel, cid, -1, A, 1, A, None) == fo.FO_ERR_SHAPE
        assert eg(gate, 0, d, s, b, None, rel, cid, 1, None, 1, A, None) == fo.FO_ERR_NULL
        assert eg(gate, 0, d, s, b, None, rel, cid, 1, A, 0, A, None) == fo.FO_ERR_SCHEDULE
        assert eg(gate, 0, d, s, b, iss, rel, cid, 1, A, 1, A, None) == fo.FO_ERR_SCHEDULE
        assert eg(gate, 0, d, s, b, None, rel, bad, 1, A, 1, A, None) == fo.FO_ERR_SCHEDULE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fo, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fo, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        fo.lib()


def test_ag_gemm_noalloc_validation(L):
    """The allocation-free AG-GEMM validates like fo_ag_gemm and refuses a
    problem whose workspace bound exceeds its scratch array, before any HIP
    call."""
    s, keep = sched()
    na = L.fo_ag_gemm_noalloc
    assert na(None, A, A2, fo.FO_F32, 256, 512, 512, ctypes.byref(s), None) == fo.FO_ERR_NULL
    assert na(A, A, A2, fo.FO_F32, 256, 512, 512, None, None) == fo.FO_ERR_NULL
    assert na(A, A, A2, 7, 256, 512, 512, ctypes.byref(s), None) == fo.FO_ERR_DTYPE
    assert na(A, A, A2, fo.FO_F32, 255, 512, 512, ctypes.byref(s), None) == fo.FO_ERR_SHAPE
    assert na(A, A, A2, fo.FO_F32, 256, 512, (1 << 21) + 8, ctypes.byref(s), None) == fo.FO_ERR_SHAPE
    s8, keep8 = sched(R=8)
    assert fo.fo_workspace_bytes(65536, 8192, 4096, 8) > fo.FO_NOALLOC_SCRATCH_BYTES
    assert na(A, A, A2, fo.FO_F32, 65536, 8192, 4096, ctypes.byref(s8), None) == fo.FO_ERR_WORKSPACE


def test_a2a_gemm_validation(L):
    R = 4
    pcs = [A + 0x100000 * q for q in range(R)]

    def a2(pieces=pcs, w=A2, y=A2 + 0x8000000, dt=fo.FO_F32, m=256, n=512, k=512, s=None, ws=WS, wsb=4096):
        if s is None:
            s, a2.keep = sched(R)
        arr = None if pieces is None else (ctypes.c_void_p * R)(*pieces)
        return L.fo_a2a_gemm(arr, w, y, dt, m, n, k, ctypes.byref(s) if s is not False else None, ws, wsb, None)
    assert a2(pieces=None) == fo.FO_ERR_NULL
    assert a2(pieces=[A, None, A, A]) == fo.FO_ERR_NULL
    assert a2(w=None) == fo.FO_ERR_NULL
    assert a2(s=False) == fo.FO_ERR_NULL
    assert a2(dt=3) == fo.FO_ERR_DTYPE
    assert a2(k=510) == fo.FO_ERR_SHAPE                     # k % P
    assert a2(k=(1 << 21) + 32) == fo.FO_ERR_SHAPE
    assert a2(k=48) == fo.FO_ERR_ALIGN                      # (k/P) % 8
    assert a2(pieces=[A, A + 8, A, A]) == fo.FO_ERR_ALIGN
    assert a2(y=A2 + 4) == fo.FO_ERR_ALIGN
    assert a2(y=A2) == fo.FO_ERR_ALIAS                      # y overlaps w
    assert a2(y=pcs[3]) == fo.FO_ERR_ALIAS                  # y overlaps a piece
    assert a2(ws=None) == fo.FO_ERR_WORKSPACE
    assert a2(wsb=1024) == fo.FO_ERR_WORKSPACE
    s, keep = sched(R, split=[1, 2, 1, 1])
    assert a2(s=s) == fo.FO_ERR_SCHEDULE
    s, keep = sched(R, order=[0, 0, 1, 2])
    assert a2(s=s) == fo.FO_ERR_ORDER


def test_qsa_validation(L):
    R, S, H, d = 4, 512, 2, 128
    wsb = fo.fo_qsa_workspace_bytes(S, H, d, R)
    assert wsb > 0
    assert fo.fo_qsa_workspace_bytes(S, H, 64, R) == 0          # head_dim must be 128
    assert fo.fo_qsa_workspace_bytes(500, H, d, R) == 0         # S % R
    assert fo.fo_qsa_workspace_bytes(S, H, d, 17) == 0          # at most 16 chunks
    assert fo.fo_qsa_workspace_bytes(4 * 64, H, d, 4) == 0      # chunk of 64 rows < 128

    def qa(qkv=A, o=A2, dt=fo.FO_F32, seq=S, heads=H, hd=d, causal=1, s=None, ws=WS, n=wsb):
        if s is None:
            s, qa.keep = sched(R)
        return L.fo_qsa_attention(qkv, o, dt, seq, heads, hd, causal,
                                  ctypes.byref(s) if s is not False else None, ws, n, None)
    assert qa(qkv=None) == fo.FO_ERR_NULL
    assert qa(s=False) == fo.FO_ERR_NULL
    assert qa(dt=2) == fo.FO_ERR_DTYPE
    assert qa(hd=64) == fo.FO_ERR_SHAPE
    assert qa(seq=640) == fo.FO_ERR_SHAPE                    # chunk 160 not a multiple of 128
    assert qa(causal=2) == fo.FO_ERR_SCHEDULE
    assert qa(qkv=A + 8) == fo.FO_ERR_ALIGN
    assert qa(o=A + 4096) == fo.FO_ERR_ALIAS                 # o inside qkv
    assert qa(ws=None) == fo.FO_ERR_WORKSPACE
    assert qa(n=wsb - 16) == fo.FO_ERR_WORKSPACE
    s, keep = sched(R, split=[1, 1, 2, 1])
    assert qa(s=s) == fo.FO_ERR_SCHEDULE
    s, keep = sched(R, order=[1, 1, 2, 3])
    assert qa(s=s) == fo.FO_ERR_ORDER


def test_emulate_sends_validation(L):
    P = ctypes.c_void_p
    d = (P * 1)(A)
    s = (P * 1)(A2)
    b = (ctypes.c_size_t * 1)(64)
    cid = (ctypes.c_int32 * 1)(1)
    ln = (ctypes.c_int64 * 1)(1000)
    es = L.fo_emulate_sends
    assert es(A, 1, d, s, b, cid, ln, 0, 0, None, A, None) == fo.FO_OK          # nothing to do
    assert es(A, 1, d, s, b, cid, ln, -1, 0, None, A, None) == fo.FO_ERR_SHAPE
    assert es(None, 1, d, s, b, cid, ln, 1, 0, None, A, None) == fo.FO_ERR_NULL
    assert es(A, 1, d, s, b, cid, ln, 1, 0, None, None, None) == fo.FO_ERR_NULL   # stamps required
    assert es(A, 0, d, s, b, cid, ln, 1, 0, None, A, None) == fo.FO_ERR_SCHEDULE  # epoch 0
    bad = (ctypes.c_int32 * 1)(64)
    assert es(A, 1, d, s, b, bad, ln, 1, 0, None, A, None) == fo.FO_ERR_SCHEDULE
    neg = (ctypes.c_int64 * 1)(-5)
    assert es(A, 1, d, s, b, cid, neg, 1, 0, None, A, None) == fo.FO_ERR_SCHEDULE
    nul = (P * 1)(None)
    assert es(A, 1, nul, s, b, cid, ln, 1, 0, None, A, None) == fo.FO_ERR_NULL
