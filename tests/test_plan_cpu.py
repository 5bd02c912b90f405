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


# ---- link model, streamed schedules, calibration, reduce-scatter form -------

def test_link_arrivals_ring_and_mesh():
    R, local, nbytes, bw = 8, 3, 4 << 20, 50.0          # 50 bytes per ns
    T = nbytes / bw
    ring = fo.fo_plan_link_arrivals(R, local, nbytes, bw, fo.FO_LINK_RING, 1)
    for d in range(1, R):
        c = (local - d) % R
        assert abs(ring[c] - d * T) <= 1
    assert ring[local] == 0
    mesh = fo.fo_plan_link_arrivals(R, local, nbytes, bw, fo.FO_LINK_MESH, 1)
    assert all(abs(mesh[c] - T) <= 1 for c in range(R) if c != local)
    # streamed: the last message of a chunk lands when the whole chunk would
    # have, the others evenly before it, in order
    sub = 4
    s = fo.fo_plan_link_arrivals(R, local, nbytes, bw, fo.FO_LINK_RING, sub)
    for c in range(R):
        if c == local:
            assert s[c * sub:(c + 1) * sub] == [0] * sub
            continue
        pieces = s[c * sub:(c + 1) * sub]
        assert abs(pieces[-1] - ring[c]) <= 1
        assert all(b - a > 0 and abs((b - a) - T / sub) <= 2 for a, b in zip(pieces, pieces[1:]))
    with pytest.raises(fo.FoError):
        fo.fo_plan_link_arrivals(R, local, nbytes, bw, 7, 1)
    with pytest.raises(fo.FoError):
        fo.fo_plan_link_arrivals(16, 0, nbytes, bw, fo.FO_LINK_RING, 8)     # 128 pieces


@pytest.mark.parametrize("bw", [50, 153, 400, 1000])
@pytest.mark.parametrize("topo", [0, 1])
def test_stream_plan_is_a_valid_schedule(bw, topo):
    c = CFG2
    sub, order, split, pred = fo.fo_plan_ag_stream(c.m, c.n, c.k, c.R, c.local, bw, topo, num_workgroups=GRID)
    R2 = c.R * sub
    assert sub in (1, 2, 4, 8)
    assert sorted(order) == list(range(R2)) and len(split) == R2
    local_pieces = list(range(c.local * sub, (c.local + 1) * sub))
    assert order[-sub:] == local_pieces                        # the local pieces last
    last = order[R2 - sub - 1]                                 # the piece that lands last
    assert all(sp == 1 for p, sp in enumerate(split) if p != last)
    # the pieces by landing time, as the link model delivers them
    land = fo.fo_plan_link_arrivals(c.R, c.local, c.m // c.R * c.k * 2, bw, topo, sub)
    t = [land[p] for p in order[:R2 - sub]]
    assert t == sorted(t)
    # the chosen schedule has the earliest prediction, up to the margins
    chosen = pred[[1, 2, 4, 8].index(sub)][[1, 2, 4, 8].index(split[last])]
    best = min(p for row in pred for p in row if p > 0)
    assert 0 < chosen <= best + 1000


def test_stream_plan_streams_on_slow_links_and_rows_must_allow_it():
    c = CFG2
    sub, _, _, pred = fo.fo_plan_ag_stream(c.m, c.n, c.k, c.R, c.local, 50, fo.FO_LINK_RING, num_workgroups=GRID)
    assert sub > 1, "at 50 GB/s the GPU is idle at the last landing: streaming the chunks pays"
    assert min(p for p in pred[[1, 2, 4, 8].index(sub)] if p > 0) < min(p for p in pred[0] if p > 0)
    q = wl.CFG5                                                 # 16 chunks: 8 messages would need 128 pieces
    _, _, _, pred5 = fo.fo_plan_ag_stream(q.m, q.n, q.k, q.R, q.local, 50, fo.FO_LINK_RING, num_workgroups=GRID)
    assert pred5[3] == [-1, -1, -1, -1]
    # one chunk cannot be streamed (nothing lands)
    sub1, order1, split1, _ = fo.fo_plan_ag_stream(512, 256, 512, 1, 0, 50, fo.FO_LINK_RING, num_workgroups=GRID)
    assert sub1 == 1 and order1 == [0] and split1 == [1]


def test_calibration_from_measured_launches():
    c = CFG2
    cal = fo.fo_plan_calibrate(c.m, c.n, c.k, c.R, 64_000, 58_000, 30_000, GRID)
    # the rate is the launch's flops over its time less start and end (4 us)
    assert abs(cal.gemm_tflops - 2.0 * c.m * c.n * c.k / 60_000 / 1e3) < 1e-6
    assert 1.0 <= cal.alone_speedup <= 4.0
    assert cal.reserve_latency_ns >= 200
    # a slower measured launch calibrates a lower rate, and the model then
    # predicts later completions
    slow = fo.fo_plan_calibrate(c.m, c.n, c.k, c.R, 128_000, 0, 0, GRID)
    assert slow.gemm_tflops < cal.gemm_tflops
    _, _, _, p_fast = fo.fo_plan_ag_stream(c.m, c.n, c.k, c.R, 0, 1000, fo.FO_LINK_RING, calib=cal,
                                           num_workgroups=GRID)
    _, _, _, p_slow = fo.fo_plan_ag_stream(c.m, c.n, c.k, c.R, 0, 1000, fo.FO_LINK_RING, calib=slow,
                                           num_workgroups=GRID)
    assert p_slow[0][0] > p_fast[0][0]
    with pytest.raises(fo.FoError):
        fo.fo_plan_calibrate(c.m, c.n, c.k, c.R, 1000, 0, 0, GRID)      # shorter than a launch's start


def test_rs_form_choice_follows_the_landings():
    c = wl.CFG3
    part_ns_50 = (c.m // c.R) * c.n * 4 / 50            # one partial at 50 GB/s
    slow = [0] + [int(part_ns_50 * d) for d in range(c.R - 1, 0, -1)]
    form, pred = fo.fo_plan_rs_form(c.m, c.n, c.k, c.R, 0, slow, num_workgroups=GRID)
    # every form ends after the last landing
    assert all(p > max(slow) for p in pred)
    # fast links: the partials land during the GEMM, and the ring form adds a
    # single partial after it, so it is predicted first
    fast = [0] + [int(part_ns_50 / 20 * d) for d in range(c.R - 1, 0, -1)]
    form2, pred2 = fo.fo_plan_rs_form(c.m, c.n, c.k, c.R, 0, fast, num_workgroups=GRID)
    assert form2 == 2 and pred2[2] < pred2[0]
    assert pred2[1] <= pred2[0]                          # the fused form never waits for a second launch
    with pytest.raises(fo.FoError):
        fo.fo_plan_rs_form(c.m, c.n, c.k, c.R, 9, fast, num_workgroups=GRID)
