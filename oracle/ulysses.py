"""Simulation of every rank's all-to-all of Ulysses parallelism, decomposed
into peer-to-peer messages (TEST INFRASTRUCTURE).

Pins the oracle's reading of Flash All-to-All (gist.science technical summary
§2: the decomposed primitives extend to Ulysses parallelism; §1: Ulysses
parallelism needs all-to-all) and of "exact" (the abstract): after attention
each rank holds the attention output of its own group of heads for the whole
sequence; the all-to-all returns to each rank the rows of its own sequence
slice from every rank's heads, and the output projection follows.  Here the
all-to-all runs as P - 1 pairwise steps (step s: rank r sends to r + s and
receives from r - s); each rank multiplies every piece as it arrives by the
matching rows of the weight and adds the products in arrival order.  The
messages are the actual arrays handed from rank to rank, so a wrong peer, a
wrong sequence slice or a wrong head block shows up in the values.
"""
from __future__ import annotations

import numpy as np

from . import gemm


def ulysses_out_proj(o_full_bits, w_bits, P: int):
    """o_full_bits: bf16 [S, k] attention output for every token and head
    (the head-parallel layout: rank q holds the columns [q*k/P, (q+1)*k/P) for
    every row); w_bits: bf16 [n, k] output projection (stored [n, k]).

    Returns (y_per_rank, received): y_per_rank[r] = fp64 [S/P, n], rank r's
    output rows, summed piece by piece in arrival order; received[r] = the
    peers in the order rank r received their pieces (its own piece first).
    """
    S, k = o_full_bits.shape
    if S % P or k % P:
        raise ValueError("S and k must divide by P")
    sp, kp = S // P, k // P
    # what each rank holds after attention: all rows, its own head columns
    held = [np.ascontiguousarray(o_full_bits[:, q * kp:(q + 1) * kp]) for q in range(P)]
    ys = [np.zeros((sp, w_bits.shape[0])) for _ in range(P)]
    received = [[] for _ in range(P)]

    def consume(r, q, piece):
        # piece: rows of rank r's sequence slice, head columns of rank q
        ys[r] += gemm(piece, np.ascontiguousarray(w_bits[:, q * kp:(q + 1) * kp]))
        received[r].append(q)

    for r in range(P):                                   # the piece each rank keeps
        consume(r, r, held[r][r * sp:(r + 1) * sp])
    for s in range(1, P):                                # pairwise exchange steps
        inbox = [None] * P
        for q in range(P):
            dst = (q + s) % P
            inbox[dst] = (q, held[q][dst * sp:(dst + 1) * sp])
        for r in range(P):
            q, piece = inbox[r]
            consume(r, q, piece)
    return ys, received
