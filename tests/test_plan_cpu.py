"""Schedule model (fo_plan_ag_schedule): host-only planning, run on the CPU.

The model predicts the completion of one chunked AG-GEMM launch from the
expected landing time of every peer chunk (euno.news "Methodology" step 3;
technical summary §2: incoming-data work first, the local slice last) and
picks the split of the chunk that lands last.  These tests check its
decisions against what the arrival pattern implies, not against timings.
"""
import ctypes

import pytest

import sp_rank_adaptive_amd as fo
import workloads as wl

CFG2 = wl.CFG2
GRID = 256


def ring_arrivals(cfg, bw):
    mc = cfg.m // cfg.R
    rel = wl.ring_release_ns(mc * cfg.k * 2, cfg.R - 1, bw)
    order = wl.ring_arrival_order(cfg.R, cfg.local)
    arr = [0] * cfg.R
    for q, t in zip(order, rel):
        arr[q] = int(t)
    return arr, order


def plan(cfg, arr, **kw):
    return fo.fo_plan_ag_schedule(cfg.m, cfg.n, cfg.k, cfg.R, cfg.local, arr,
                                  num_workgroups=kw.pop("grid", GRID), **kw)


def test_order_is_landing_order_local_last():
    arr, ring = ring_arrivals(CFG2, 50e9)
    order, split, _ = plan(CFG2, arr)
    assert order == ring + [CFG2.local]
    # any landing pattern: peers sorted by landing time, local last
    arr2 = [0, 30_000, 10_000, 50_000, 20_000, 20_000, 70_000, 5_000]
    order2, split2, _ = plan(CFG2, arr2)
    assert order2[-1] == 0
    times = [arr2[c] for c in order2[:-1]]
    assert times == sorted(times)
    assert sorted(order2) == list(range(CFG2.R))
    # equal landing times keep ring order (local-1 before local-2 ...)
    assert order2.index(5) < order2.index(4)
    # only the last-landing peer may be split
    assert all(s == 1 for c, s in enumerate(split2) if c != order2[-2])


def chosen_is_earliest(split_last, pred):
    chosen = pred[[1, 2, 4, 8].index(split_last)]
    # the earliest prediction, up to the 0.5 us a larger split must win by
    return chosen <= min(p for p in pred if p > 0) + 500


def test_slow_links_split_the_last_chunk():
    # 50 GB/s: the GPU is idle when the last chunk lands, so its tiles are
    # shared by the idle workgroups
    arr, _ = ring_arrivals(CFG2, 50e9)
    order, split, pred = plan(CFG2, arr)
    last = order[-2]
    assert split[last] >= 4
    assert all(s == 1 for c, s in enumerate(split) if c != last)
    assert chosen_is_earliest(split[last], pred)
    assert pred[[1, 2, 4, 8].index(split[last])] < pred[0]


def test_fast_links_do_not_split():
    # 1 TB/s: every workgroup is still busy with earlier chunks when the last
    # one lands, so split units would queue behind them
    arr, _ = ring_arrivals(CFG2, 1000e9)
    order, split, pred = plan(CFG2, arr)
    assert split == [1] * CFG2.R
    assert chosen_is_earliest(1, pred)


def test_split_shrinks_as_links_get_faster():
    # the last chunk's split never grows with the link bandwidth
    prev = 8
    for bw in (50e9, 153e9, 400e9, 1000e9):
        arr, order = ring_arrivals(CFG2, bw)
        _, split, pred = plan(CFG2, arr)
        sk = split[order[-1]]
        assert sk <= prev, bw
        assert chosen_is_earliest(sk, pred), bw
        prev = sk


def test_prediction_properties():
    present = [0] * CFG2.R
    _, _, p0 = plan(CFG2, present)
    arr, _ = ring_arrivals(CFG2, 50e9)
    _, _, p50 = plan(CFG2, arr)
    # later landings never finish earlier, and never before the last landing
    assert all(b >= a for a, b in zip(p0, p50) if a > 0 and b > 0)
    assert min(p for p in p50 if p > 0) > max(arr)
    # all present: one round of full-K tiles, about the measured 60-70 us
    assert 40_000 < p0[0] < 100_000
    # a faster rate predicts an earlier completion
    _, _, fast = plan(CFG2, present, gemm_tflops=1800.0)
    assert fast[0] < p0[0]


def test_single_chunk_and_short_k():
    order, split, pred = fo.fo_plan_ag_schedule(512, 512, 512, 1, 0, [0], num_workgroups=GRID)
    assert order == [0] and split == [1]
    assert pred[0] > 0 and pred[1:] == [-1, -1, -1]
    # k of one 64-wide stage cannot be split
    order, split, pred = fo.fo_plan_ag_schedule(256, 512, 64, 4, 0, [0, 3000, 2000, 1000], num_workgroups=GRID)
    assert split == [1] * 4 and pred[1:] == [-1, -1, -1]


def test_validation():
    L = fo.lib()
    arr = (ctypes.c_int64 * 4)(0, 1, 2, 3)
    o = (ctypes.c_int32 * 4)()
    s = (ctypes.c_int32 * 4)()
    args = dict(m=256, n=512, k=512)
    assert L.fo_plan_ag_schedule(256, 512, 512, 4, 0, None, 0.0, GRID, o, s, None) == fo.FO_ERR_NULL
    assert L.fo_plan_ag_schedule(256, 512, 512, 4, 0, arr, 0.0, GRID, None, s, None) == fo.FO_ERR_NULL
    assert L.fo_plan_ag_schedule(258, 512, 512, 4, 0, arr, 0.0, GRID, o, s, None) == fo.FO_ERR_SHAPE
    assert L.fo_plan_ag_schedule(256, 512, 512, 0, 0, arr, 0.0, GRID, o, s, None) == fo.FO_ERR_SHAPE
    assert L.fo_plan_ag_schedule(256, 512, 512, 4, 4, arr, 0.0, GRID, o, s, None) == fo.FO_ERR_SCHEDULE
    bad = (ctypes.c_int64 * 4)(0, -5, 2, 3)
    assert L.fo_plan_ag_schedule(256, 512, 512, 4, 0, bad, 0.0, GRID, o, s, None) == fo.FO_ERR_SCHEDULE
    # the local chunk's entry is ignored, even when negative
    loc = (ctypes.c_int64 * 4)(-1, 1, 2, 3)
    assert L.fo_plan_ag_schedule(args["m"], args["n"], args["k"], 4, 0, loc, 0.0, GRID, o, s, None) == fo.FO_OK


def test_long_sequence_share_at_slow_links():
    # the QKV share (16 chunks of 1024 x 8192, 256x160 tiles) at 50 GB/s: the
    # GPU is idle at the last landing and 8 splits of its 32 tiles fill it
    cfg = wl.CFG5
    arr, order = ring_arrivals(cfg, 50e9)
    o, split, pred = fo.fo_plan_ag_schedule(cfg.m, cfg.n, cfg.k, cfg.R, cfg.local, arr, num_workgroups=GRID)
    assert o == order + [cfg.local]
    assert split[order[-1]] == 8 and chosen_is_earliest(8, pred)
