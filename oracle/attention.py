"""Attention oracle for Query-Split Attention (TEST INFRASTRUCTURE).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module; it shares no code with the device library.

What is computed (gist.science technical summary §2, Query-Split Attention:
attention decomposed into scores, softmax and weighted sum so that more of
it overlaps the communication; the abstract: the decomposition is exact).
The input is the QKV projection's output for the whole sequence, one row per
token: qkv [S, 3*H*d] bf16 with the queries of head h in columns
[h*d, (h+1)*d), its keys at H*d + that, its values at 2*H*d + that.  For
every head, O = softmax(scale * Q K^T + mask) V with scale = 1/sqrt(d) and,
when causal, -inf above the diagonal (token i sees tokens 0..i).  Out is
[S, H*d], head h in columns [h*d, (h+1)*d).

`attention` is the plain definition in fp64 (the softmax with the row
maximum subtracted, then normalised).  `attention_blocks` evaluates the same
result the way the query-split decomposition does: the sequence is cut into
R chunks; for every pair (query chunk i, key chunk j) the block's scores give
a row maximum m, a sum of exponentials l and an unnormalised weighted sum;
the blocks of a query chunk are merged in a given key-chunk order.  It exists
to pin the decomposition against the plain definition.
"""
from __future__ import annotations

import numpy as np


def _split(qkv_bits, H: int, d: int):
    from . import bf16_to_f64_fast
    x = bf16_to_f64_fast(qkv_bits)
    S = x.shape[0]
    if x.shape[1] != 3 * H * d:
        raise ValueError("qkv must be [S, 3*H*d]")
    q = x[:, :H * d].reshape(S, H, d).transpose(1, 0, 2)
    k = x[:, H * d:2 * H * d].reshape(S, H, d).transpose(1, 0, 2)
    v = x[:, 2 * H * d:].reshape(S, H, d).transpose(1, 0, 2)
    return q, k, v


def attention(qkv_bits, H: int, d: int, causal: bool) -> np.ndarray:
    """O [S, H*d] fp64: per head, softmax(Q K^T / sqrt(d) [+ causal mask]) V."""
    q, k, v = _split(qkv_bits, H, d)
    S = q.shape[1]
    out = np.empty((S, H * d), dtype=np.float64)
    scale = 1.0 / np.sqrt(d)
    for h in range(H):
        s = (q[h] @ k[h].T) * scale
        if causal:
            s[np.triu_indices(S, 1)] = -np.inf
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h * d:(h + 1) * d] = p @ v[h]
    return out


def attention_blocks(qkv_bits, H: int, d: int, causal: bool, R: int, key_order=None) -> np.ndarray:
    """The same O, from per-(query chunk, key chunk) blocks merged per query
    chunk in key_order (default 0..R-1); blocks a causal mask empties are
    skipped."""
    q, k, v = _split(qkv_bits, H, d)
    S = q.shape[1]
    if S % R:
        raise ValueError("S must divide by R")
    c = S // R
    order = list(range(R)) if key_order is None else list(key_order)
    scale = 1.0 / np.sqrt(d)
    out = np.empty((S, H * d), dtype=np.float64)
    for h in range(H):
        for i in range(R):
            rows = slice(i * c, (i + 1) * c)
            parts = []
            for j in order:
                if causal and j > i:
                    continue
                cols = slice(j * c, (j + 1) * c)
                s = (q[h][rows] @ k[h][cols].T) * scale
                if causal and j == i:
                    s[np.triu_indices(c, 1)] = -np.inf
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                parts.append((m, e.sum(axis=1, keepdims=True), e @ v[h][cols]))
            M = np.max(np.concatenate([p[0] for p in parts], axis=1), axis=1, keepdims=True)
            L = sum(np.exp(m - M) * l for m, l, _ in parts)
            O = sum(np.exp(m - M) * o for m, _, o in parts)
            out[rows, h * d:(h + 1) * d] = O / L
    return out
