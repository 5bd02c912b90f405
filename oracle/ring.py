"""Simulation of every rank's ring steps (TEST INFRASTRUCTURE).

Pins the oracle's reading of "exact" in the FlashOverlap abstract: the
decomposed peer-to-peer form of all-gather and reduce-scatter, with the
partitioned GEMMs scheduled as the pages describe, yields the same result as
the collective it replaces.

- Flash-AG (gist.science technical summary §2): all-gather as a ring of
  peer-to-peer steps; each rank computes the slice it already holds first,
  then each slice as it is received from its predecessor.
- Flash-RS (same section): reduce-scatter as peer-to-peer exchanges; at each
  step a rank computes its partial of the chunk that travels through it, adds
  the accumulated partial received from its predecessor and forwards the sum;
  the chunk that stays local is computed as the very last step.

Messages are simulated by handing the actual arrays from rank to rank, so a
wrong neighbour or a wrong chunk index shows up in the values.
"""
from __future__ import annotations

import numpy as np

from . import gemm


def ring_ag(x_chunks, w_per_rank):
    """x_chunks[r]: bf16 [mc,k] held by rank r; w_per_rank[r]: bf16 [n_r,k].

    Returns (y_per_rank, computed_order): y_per_rank[r] = gathered X times
    rank r's weights, fp64 [R*mc, n_r]; computed_order[r] = chunk indices in
    the order rank r computed them.
    """
    R = len(x_chunks)
    mc = x_chunks[0].shape[0]
    ys = [np.full((R * mc, w.shape[0]), np.nan) for w in w_per_rank]
    held = [(r, x_chunks[r]) for r in range(R)]        # (chunk id, data)
    done = [[] for _ in range(R)]
    for step in range(R):
        for r in range(R):
            c, data = held[r]
            ys[r][c * mc:(c + 1) * mc] = gemm(data, w_per_rank[r])
            done[r].append(c)
        if step < R - 1:                                 # send to successor
            held = [held[(r - 1) % R] for r in range(R)]
    return ys, done


def ring_rs(x_per_rank, w_per_rank):
    """x_per_rank[r]: bf16 [m, k_r]; w_per_rank[r]: bf16 [n, k_r] (rank r's
    slice of the contraction dimension).

    Returns (shards, computed_order): shards[r] = rows of chunk r of
    sum_q X_q W_q^T accumulated along the ring (fp64 adds, one per hop);
    computed_order[r] = chunk indices in the order rank r computed them.
    """
    R = len(x_per_rank)
    m = x_per_rank[0].shape[0]
    mc = m // R
    partial = [gemm(x_per_rank[r], w_per_rank[r]) for r in range(R)]
    inbox = [None] * R
    shards = [None] * R
    done = [[] for _ in range(R)]
    for step in range(R):
        outbox = [None] * R
        for r in range(R):
            c = (r - 1 - step) % R
            p = partial[r][c * mc:(c + 1) * mc]
            acc = p.copy() if step == 0 else inbox[r] + p
            done[r].append(c)
            if step == R - 1:
                shards[r] = acc
            else:
                outbox[(r + 1) % R] = acc
        inbox = outbox
    return shards, done
