"""Seeded synthetic inputs for the FlashOverlap one-GPU hot path.

This module is shared by the oracle side (``oracle/``, ``tests/``) and the
device side (``bench.py``, GPU tests).  It holds only shapes, seeds and random
number generation: none of the method's arithmetic (no products, no sums, no
output rounding) lives here.

Every tensor is drawn from numpy's PCG64 with a per-tensor seed
``SEED_BASE + 100 * cfg + tensor_id`` and, for bf16 operands, converted from
float32 to bf16 bit patterns with round-to-nearest-even, so the oracle and the
GPU see identical bits.

The five workloads restate the problem statement of the pages (FlashOverlap,
arXiv 2604.24013: the abstract's all-gather / reduce-scatter replaced by
decomposed peer-to-peer pieces; the gist.science technical summary §2,
Flash-AG and Flash-RS) as concrete shapes at tensor-parallel degree 8 or 16,
with the hidden size 4096 of the summary's §4 experiments.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 2604240131

# Modelled per-link bandwidth of the emulated peers (bytes per second).
LINK_BW = 50e9


@dataclass(frozen=True)
class GemmCfg:
    """Shape of one chunked GEMM workload (AG mode or RS mode)."""
    cfg: int
    name: str
    mode: str          # "ag", "rs" or "a2a"
    m: int
    n: int
    k: int
    R: int
    local: int = 0
    x_std: float = 1.0
    w_std: float = 0.02
    inc_std: float = 0.0   # RS mode: std of the incoming fp32 partials


@dataclass(frozen=True)
class ReduceCfg:
    cfg: int
    name: str
    n: int
    R: int
    local: int = 0
    std: float = 1e-3
    int_range: int = 1 << 20
    extra: dict = field(default_factory=dict)


CFG1 = GemmCfg(1, "tiny_ag_gemm_r4", "ag", 256, 512, 512, 4)
CFG2 = GemmCfg(2, "tpsp_mlp_up_ag_gemm_tp8", "ag", 4096, 1792, 4096, 8)
CFG3 = GemmCfg(3, "tpsp_mlp_down_gemm_rs_tp8", "rs", 4096, 4096, 1792, 8,
               inc_std=0.02 * float(np.sqrt(1792.0)))
CFG4 = ReduceCfg(4, "dp_grad_reduce_r8", 1 << 27, 8)
CFG5 = GemmCfg(5, "long_seq_qkv_ag_gemm_tp16", "ag", 16384, 1280, 8192, 16)

# Ulysses attention output projection, one rank's share at Ulysses degree 8:
# a 16K-token sequence (the long end of the summary's 1K-16K sweep) with the
# summary's hidden size 4096 as 32 heads of 128; the all-to-all hands this
# rank its 2048 rows of every rank's 4 heads (8 pieces of 2048 x 512), and W
# is the 4096 x 4096 output projection.
CFG6 = GemmCfg(6, "ulysses_out_proj_a2a_up8", "a2a", 2048, 4096, 4096, 8)

@dataclass(frozen=True)
class AttnCfg:
    """Query-split attention share: the QKV projection's output for S tokens
    and H local heads of dimension d, arriving in R sequence chunks."""
    cfg: int
    name: str
    S: int
    H: int
    d: int
    R: int
    local: int = 0
    causal: bool = True
    std: float = 1.0


# Query-split attention, one rank's share of the summary's setting (hidden
# size 4096, TP = 4): 8 of 32 heads of 128, a 4K-token causal sequence in 4
# chunks of 1024 tokens (this rank's and three that arrive).
CFG7 = AttnCfg(7, "tp4_query_split_attention", 4096, 8, 128, 4)

CONFIGS = {1: CFG1, 2: CFG2, 3: CFG3, 4: CFG4, 5: CFG5, 6: CFG6, 7: CFG7}

# tensor ids used in seeds
T_X, T_W, T_INC, T_SRC, T_ORDER = 1, 2, 3, 10, 50


def seed_for(cfg: int, tensor_id: int) -> int:
    return SEED_BASE + 100 * cfg + tensor_id


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_operand(shape, mode: str, std: float, seed: int,
                 lo: int = -3, hi: int = 3) -> np.ndarray:
    """bf16 bits of shape `shape`.

    mode "int": integers uniform in [lo, hi] (exact in bf16).
    mode "gauss": N(0, std) drawn in float32, rounded to bf16.
    """
    g = _rng(seed)
    if mode == "int":
        v = g.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.float32)
    elif mode == "gauss":
        v = g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    else:
        raise ValueError(mode)
    return f32_to_bf16_bits(v)


def f32_operand(shape, mode: str, std: float, seed: int,
                int_range: int = 4096) -> np.ndarray:
    """float32 array: integers uniform in [-int_range, int_range] or N(0, std)."""
    g = _rng(seed)
    if mode == "int":
        return g.integers(-int_range, int_range + 1, size=shape,
                          dtype=np.int64).astype(np.float32)
    if mode == "gauss":
        return g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    raise ValueError(mode)


def gemm_inputs(c: GemmCfg, mode: str, m: int | None = None):
    """(x_bits [m,k], w_bits [n,k]) for a GEMM config; optional smaller m."""
    m = c.m if m is None else m
    x = bf16_operand((m, c.k), mode, c.x_std, seed_for(c.cfg, T_X))
    w = bf16_operand((c.n, c.k), mode, c.w_std, seed_for(c.cfg, T_W))
    return x, w


def a2a_pieces(c: GemmCfg, mode: str, m: int | None = None):
    """(pieces, w_bits) of an all-to-all workload: the gathered operand
    [m, k] drawn as one matrix and cut into R column blocks [m, k/R] (piece
    q = the block that rank q's heads contribute), each contiguous."""
    x, w = gemm_inputs(c, mode, m=m)
    kp = c.k // c.R
    return [np.ascontiguousarray(x[:, q * kp:(q + 1) * kp]) for q in range(c.R)], w


def qkv_input(c: AttnCfg, mode: str, S: int | None = None) -> np.ndarray:
    """bf16 bits of the attention input qkv [S, 3*H*d] (queries, keys,
    values of every head, one row per token)."""
    S = c.S if S is None else S
    return bf16_operand((S, 3 * c.H * c.d), mode, c.std, seed_for(c.cfg, T_X))


def incoming_partials(c: GemmCfg, mode: str, rows: int | None = None):
    """Incoming fp32 partials for the local shard, one per peer (None at local)."""
    rows = c.m // c.R if rows is None else rows
    out = []
    for q in range(c.R):
        if q == c.local:
            out.append(None)
        else:
            out.append(f32_operand((rows, c.n), mode, c.inc_std,
                                   seed_for(c.cfg, T_INC + 10 * q), int_range=4096))
    return out


def reduce_sources(c: ReduceCfg, mode: str, n: int | None = None):
    """R fp32 source arrays of n elements."""
    n = c.n if n is None else n
    return [f32_operand((n,), mode, c.std, seed_for(c.cfg, T_SRC + i),
                        int_range=c.int_range) for i in range(c.R)]


def ring_arrival_order(R: int, local: int) -> list[int]:
    """Chunks in the order a ring delivers them to `local`: local-1, local-2, ..."""
    return [(local - s) % R for s in range(1, R)]


def seeded_permutation(values: list[int], seed: int) -> list[int]:
    g = _rng(seed)
    idx = g.permutation(len(values))
    return [values[i] for i in idx]


def ring_release_ns(nbytes: int, count: int, bw: float = LINK_BW) -> list[float]:
    """Release times t_s = s * B / BW (s = 1..count) in nanoseconds."""
    return [s * nbytes / bw * 1e9 for s in range(1, count + 1)]


MESH_STAGGER_NS = 250_000.0


def mesh_staggered_release_ns(nbytes: int, count: int, bw: float = LINK_BW) -> list[float]:
    """Mesh-staggered release times t_s = B / BW + (s - 1) * 250 us
    (s = 1..count) in nanoseconds: one link per peer, the peers starting a
    little apart."""
    return [nbytes / bw * 1e9 + (s - 1) * MESH_STAGGER_NS for s in range(1, count + 1)]
