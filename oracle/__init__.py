"""CPU oracle for the FlashOverlap one-GPU hot path (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the device
library ``sp_rank_adaptive_amd`` and neither imports the other; the seeded
input generators in ``workloads.py`` are the only thing both sides use.

The arithmetic lives in ``oracle.c`` (plain fp64 loops, built with gcc),
loaded here with ctypes; ``brute.py`` holds an exact rational brute force for
tiny shapes and ``ring.py`` a simulation of every rank's ring steps.  What the
oracle computes, and which passage of the pages each function follows, is
stated in ``oracle.c``'s header and in each function below.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BUILD_CMD = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
             "-Wall", _SRC, "-o", _LIB, "-lm"]


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    subprocess.run(BUILD_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_bf16_array.argtypes = [P, i64, P]
        L.oracle_sum_exact.restype = ctypes.c_double
        L.oracle_sum_exact.argtypes = [P, ctypes.c_int]
        L.oracle_gemm.argtypes = [P, P, i64, i64, i64, P]
        L.oracle_ag_gemm.restype = ctypes.c_int
        L.oracle_ag_gemm.argtypes = [P, P, i64, i64, i64, i32, P, P]
        L.oracle_reduce.argtypes = [P, i32, i64, P]
        L.oracle_gemm_rs_shard.restype = ctypes.c_int
        L.oracle_gemm_rs_shard.argtypes = [P, P, i64, i64, i64, i32, i32, P, P]
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 operands are passed as uint16 bit patterns")
    return a


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def bf16_to_f64(bits) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float64."""
    b = _u16(bits)
    f = lib().oracle_bf16_to_f64
    out = np.empty(b.shape, dtype=np.float64)
    flat, of = b.reshape(-1), out.reshape(-1)
    for i in range(flat.size):
        of[i] = f(int(flat[i]))
    return out


def bf16_to_f64_fast(bits) -> np.ndarray:
    """Exact decode of bf16 bit patterns to float64 by placing them in the
    upper half of a binary32 (a bf16 value is a binary32 with its low 16
    fraction bits zero); pinned against the C decode in the tests."""
    b = _u16(bits)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(v) -> np.ndarray:
    """float64 -> bf16 bits, one rounding to nearest even."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_f64_to_bf16_array(_p(v), v.size, _p(out))
    return out


def sum_exact(terms) -> float:
    """Exactly rounded sum of a sequence of floats."""
    t = np.ascontiguousarray(terms, dtype=np.float64)
    return float(lib().oracle_sum_exact(_p(t), t.size))


def gemm(x_bits, w_bits) -> np.ndarray:
    """AG-GEMM definition: Y = X * W (X bf16 [m,k], W stored bf16 [n,k]), fp64.

    Pages: FlashOverlap abstract (the decomposed all-gather is exact, so the
    result is the GEMM over the gathered rows); gist.science technical summary
    §2, Flash-AG.
    """
    x, w = _u16(x_bits), _u16(w_bits)
    m, k = x.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("k mismatch")
    y = np.empty((m, n), dtype=np.float64)
    lib().oracle_gemm(_p(x), _p(w), m, n, k, _p(y))
    return y


def ag_gemm(x_bits, w_bits, R: int, order) -> np.ndarray:
    """Chunked AG-GEMM: row-chunks of X multiplied by W in the given order."""
    x, w = _u16(x_bits), _u16(w_bits)
    m, k = x.shape
    n = w.shape[0]
    o = np.ascontiguousarray(order, dtype=np.int32)
    if o.size != R:
        raise ValueError("order length")
    y = np.empty((m, n), dtype=np.float64)
    rc = lib().oracle_ag_gemm(_p(x), _p(w), m, n, k, R, _p(o), _p(y))
    if rc:
        raise ValueError("bad chunking or order")
    return y


def reduce(srcs) -> np.ndarray:
    """Element-wise exactly rounded sum of R fp32 arrays.

    Pages: gist.science technical summary §1 (DP needs reduce-scatter) and §2
    (Flash-RS: partial outputs summed into the shard that stays local).
    """
    arrs = [np.ascontiguousarray(s, dtype=np.float32).reshape(-1) for s in srcs]
    n = arrs[0].size
    if any(a.size != n for a in arrs):
        raise ValueError("size mismatch")
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    out = np.empty(n, dtype=np.float64)
    lib().oracle_reduce(ptrs, len(arrs), n, _p(out))
    return out.reshape(np.shape(srcs[0]))


def ring_rs_rank(x_bits, w_bits, R: int, local: int, incoming):
    """One rank's step of the ring reduce-scatter fused with its GEMM: its
    partials X*W by row chunk, each chunk with an incoming accumulated partial
    (from the predecessor) plus that partial; the local chunk's sum is the
    shard.  Returns (forward, shard): forward [m, n] fp64 holds, per chunk c,
    P_c + incoming[c] (or P_c when incoming[c] is None); shard = the local
    chunk's rows of forward.

    Pages: gist.science technical summary §2, Flash-RS (each step adds the
    rank's own partial of the passing chunk to the accumulated one received
    and forwards the sum; the local chunk is the last step).
    """
    p = gemm(x_bits, w_bits)
    m, n = p.shape
    mc = m // R
    fwd = p.copy()
    for c in range(R):
        a = incoming[c]
        if a is None:
            continue
        a = np.asarray(a, dtype=np.float64)
        if a.shape != (mc, n):
            raise ValueError("incoming partial shape")
        fwd[c * mc:(c + 1) * mc] += a
    return fwd, fwd[local * mc:(local + 1) * mc].copy()


def gemm_rs_shard(x_bits, w_bits, R: int, local: int, incoming) -> np.ndarray:
    """GEMM-RS local shard: rows of chunk `local` of X*W plus every incoming
    fp32 partial (incoming[local] ignored), summed exactly.

    Pages: gist.science technical summary §2, Flash-RS.
    """
    x, w = _u16(x_bits), _u16(w_bits)
    m, k = x.shape
    n = w.shape[0]
    mc = m // R
    keep = []
    ptrs = (ctypes.c_void_p * R)()
    for q in range(R):
        if q == local:
            ptrs[q] = None
            continue
        a = np.ascontiguousarray(incoming[q], dtype=np.float32)
        if a.shape != (mc, n):
            raise ValueError("incoming partial shape")
        keep.append(a)
        ptrs[q] = a.ctypes.data
    out = np.empty((mc, n), dtype=np.float64)
    rc = lib().oracle_gemm_rs_shard(_p(x), _p(w), m, n, k, R, local, ptrs, _p(out))
    if rc:
        raise ValueError("bad shape or local rank")
    return out


def a2a_gemm(pieces, w_bits) -> np.ndarray:
    """Flash All-to-All output projection: Y = [A_0 | A_1 | ... | A_{P-1}] * W.

    The all-to-all of Ulysses parallelism hands each rank, from every rank q,
    the rows of its own sequence slice for q's group of heads: a column block
    A_q of the attention output [m, k/P] (bf16).  Decomposed into P2P pieces,
    the output projection over the gathered heads is still exactly the plain
    GEMM over the blocks placed side by side along k, which is what this
    returns (fp64, k ascending).  W is stored [n, k]; block q meets columns
    [q*k/P, (q+1)*k/P) of it.

    Pages: gist.science technical summary §1 (Ulysses parallelism needs
    all-to-all) and §2 (Flash All-to-All, the extension of the decomposed
    primitives to Ulysses parallelism); the abstract (the decomposition is
    exact).
    """
    blocks = [_u16(p) for p in pieces]
    if not blocks:
        raise ValueError("no pieces")
    m = blocks[0].shape[0]
    if any(b.ndim != 2 or b.shape[0] != m for b in blocks):
        raise ValueError("pieces must be [m, k/P] with one m")
    x = np.ascontiguousarray(np.concatenate(blocks, axis=1))
    if x.shape[1] != _u16(w_bits).shape[1]:
        raise ValueError("k mismatch")
    return gemm(x, w_bits)
