"""Unsampled parity at the workloads' full sizes, through the C ABI.

Integer-valued inputs make every fp32 sum exact, so each output element of
the GPU path must equal the fp64 oracle bit for bit: the whole output is
compared, not sampled rows.  The launches are the ones the benchmark times:
the TP=8 MLP up-projection share (4096 x 1792 x 4096, R = 8), its
down-projection GEMM-RS share with the reduce of 7 incoming partials
(4096 x 4096 x 1792), the long-sequence QKV share (16384 x 1280 x 8192,
R = 16, the claim walk's second batch of chunk positions and the automatic
8-way split of the last-landing chunk on 256 x 160 tiles) and the DP
gradient reduce (8 x 2^27 fp32), with emulated SDMA arrivals into poisoned
destinations and with the schedule model's order and split.
"""
import numpy as np
import pytest

import workloads as wl
from helpers import (bf16_bits_to_f64, check_exact, check_tolerance, dev_bf16, dev_f32, host,
                     log)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_EP = [20000]
_SIDE = []


def epoch():
    _EP[0] += 1
    return _EP[0]


def side_stream():
    # one side stream per process, created before any other stream here (see
    # the emulated-arrival tests): it must not share a hardware queue with the
    # stream the consumer kernels run on
    if not _SIDE:
        _SIDE.append(torch.cuda.Stream())
    return _SIDE[0]


@pytest.fixture(scope="module")
def fo():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sp_rank_adaptive_amd as fo
    fo.lib()
    side_stream()
    return fo


_REF = {}


def int_case(orc, cfg):
    """Integer-mode operands of a GEMM workload and the oracle's product
    (computed once per process)."""
    if cfg.cfg not in _REF:
        xb, wb = wl.gemm_inputs(cfg, "int")
        log(f"oracle: cfg{cfg.cfg} int {cfg.m}x{cfg.n}x{cfg.k}")
        _REF[cfg.cfg] = (xb, wb, orc.gemm(xb, wb))
    return _REF[cfg.cfg]


def ag_emulated(fo, xb, wb, R, local, order, release_ns, split=None, gated=True, reps=1):
    """fo_ag_gemm with the peers' chunks copied in by SDMA at release_ns[i]
    (chunk order[i]) into destinations filled with NaN first; returns the
    outputs of every repetition."""
    m, k = xb.shape
    n = wb.shape[0]
    mc = m // R
    staging = dev_bf16(xb)
    w = dev_bf16(wb)
    x = staging.clone()
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    gs = torch.zeros(2 * R + 2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    side = side_stream()
    peers = [q for q in order if q != local]
    outs = []
    for _ in range(reps):
        e = epoch()
        for q in peers:
            x[q * mc:(q + 1) * mc].fill_(float("nan"))
        y = torch.full((m, n), float("nan"), device="cuda")
        gs.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            fo.fo_emulate_arrivals([x[q * mc:(q + 1) * mc] for q in peers],
                                   [staging[q * mc:(q + 1) * mc] for q in peers],
                                   [int(t) for t in release_ns], peers, flags, e, es, stream=side,
                                   gate=gs[2 * R:2 * R + 1] if gated else None)
        fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=R, local=local, order=order, arrived=flags, epoch=e,
                                           stamps=gs, status=status, split=split,
                                           timeout_ns=5_000_000_000), ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "flag wait timed out"
        assert int(ws[:4096].sum()) == 0, "counters not returned to zero"
        st = host(gs).astype(np.int64)
        last = max(host(es).astype(np.int64)[1 + q] for q in peers)
        assert st[2 * R + 1] >= last, "output completed before the last landing"
        outs.append(host(y))
        del y
    return outs


def test_tp8_mlp_ag_full_int_every_schedule(fo, orc):
    """4096 x 1792 x 4096, R = 8: no flags (static claims), preset flags,
    emulated 50 GB/s ring arrivals with the automatic split, and the schedule
    model's order and split: every element exact."""
    c = wl.CFG2
    xb, wb, ref = int_case(orc, c)
    x, w = dev_bf16(xb), dev_bf16(wb)
    ws = torch.zeros(fo.fo_workspace_bytes(c.m, c.n, c.k, c.R), dtype=torch.uint8, device="cuda")
    flags = torch.zeros(c.R, dtype=torch.int32, device="cuda")
    for what, kw in (("no flags", {}), ("preset flags, unsplit", {"flags": True, "split": [1] * c.R}),
                     ("preset flags, automatic split", {"flags": True})):
        log(f"case: cfg2 int {what}")
        e = epoch()
        flags.fill_(e)
        y = torch.full((c.m, c.n), float("nan"), device="cuda")
        fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=c.R, epoch=e, arrived=flags if kw.get("flags") else None,
                                           split=kw.get("split")), ws)
        torch.cuda.synchronize()
        check_exact(host(y), ref, f"cfg2 {what}")
        del y
    order = wl.ring_arrival_order(c.R, c.local)
    nbytes = (c.m // c.R) * c.k * 2
    rel = wl.ring_release_ns(nbytes, c.R - 1)
    log("case: cfg2 int, emulated 50 GB/s ring arrivals, automatic split")
    (y,) = ag_emulated(fo, xb, wb, c.R, c.local, order + [c.local], rel)
    check_exact(y, ref, "cfg2 emulated")
    arr = [0] * c.R
    for q, t in zip(order, rel):
        arr[q] = int(t)
    p_order, p_split, _ = fo.fo_plan_ag_schedule(c.m, c.n, c.k, c.R, c.local, arr)
    log(f"case: cfg2 int, planned order {p_order} split {p_split}")
    (y,) = ag_emulated(fo, xb, wb, c.R, c.local, p_order, rel, split=p_split)
    check_exact(y, ref, "cfg2 planned schedule")
    # the model's plan at a fast link (flags released 31 us apart): unsplit
    fast = wl.ring_release_ns(nbytes, c.R - 1, 1000e9)
    for q, t in zip(order, fast):
        arr[q] = int(t)
    p_order, p_split, _ = fo.fo_plan_ag_schedule(c.m, c.n, c.k, c.R, c.local, arr)
    log(f"case: cfg2 int, planned at 1 TB/s: order {p_order} split {p_split}")
    (y,) = ag_emulated(fo, xb, wb, c.R, c.local, p_order, fast, split=p_split)
    check_exact(y, ref, "cfg2 planned schedule, fast links")


def test_qkv_r16_full_int_claim_walk_second_batch(fo, orc):
    """16384 x 1280 x 8192, R = 16: priority positions 8-15 sit in the claim
    walk's second 64-lane batch.  Preset flags (automatic split 8 of the last
    peer), emulated 50 GB/s ring arrivals (automatic split), out-of-order
    arrivals under the default priority, STRICT mode and the schedule
    model's plan: every element exact."""
    c = wl.CFG5
    xb, wb, ref = int_case(orc, c)
    x, w = dev_bf16(xb), dev_bf16(wb)
    ws = torch.zeros(fo.fo_workspace_bytes(c.m, c.n, c.k, c.R), dtype=torch.uint8, device="cuda")
    flags = torch.zeros(c.R, dtype=torch.int32, device="cuda")
    for what, kw in (("no flags", {}), ("preset flags, automatic split", {"flags": True}),
                     ("preset flags, unsplit", {"flags": True, "split": [1] * c.R})):
        log(f"case: cfg5 int {what}")
        e = epoch()
        flags.fill_(e)
        y = torch.full((c.m, c.n), float("nan"), device="cuda")
        fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=c.R, epoch=e, arrived=flags if kw.get("flags") else None,
                                           split=kw.get("split")), ws)
        torch.cuda.synchronize()
        check_exact(host(y), ref, f"cfg5 {what}")
        del y
    del x, ws
    order = wl.ring_arrival_order(c.R, c.local)
    nbytes = (c.m // c.R) * c.k * 2
    rel = wl.ring_release_ns(nbytes, c.R - 1)
    log("case: cfg5 int, emulated 50 GB/s ring arrivals, automatic split")
    (y,) = ag_emulated(fo, xb, wb, c.R, c.local, order + [c.local], rel)
    check_exact(y, ref, "cfg5 emulated")
    arr = [0] * c.R
    for q, t in zip(order, rel):
        arr[q] = int(t)
    p_order, p_split, _ = fo.fo_plan_ag_schedule(c.m, c.n, c.k, c.R, c.local, arr)
    log(f"case: cfg5 int, planned order {p_order} split {p_split}")
    (y,) = ag_emulated(fo, xb, wb, c.R, c.local, p_order, rel, split=p_split)
    check_exact(y, ref, "cfg5 planned schedule")
    # arrivals in a seeded random order, 40 us apart, against the default
    # priority (ring order): chunks of the second batch land before the first
    shuffled = wl.seeded_permutation(order, 515)
    gap = [40_000 * (i + 1) for i in range(c.R - 1)]
    log(f"case: cfg5 int, out-of-order arrivals {shuffled}")
    (y,) = ag_emulated_in(fo, xb, wb, c, shuffled, gap)
    check_exact(y, ref, "cfg5 out of order")
    log("case: cfg5 int, STRICT priority over ring arrivals 20 us apart")
    (y,) = ag_emulated_in(fo, xb, wb, c, order, [20_000 * (i + 1) for i in range(c.R - 1)],
                          mode=fo.FO_SCHED_STRICT)
    check_exact(y, ref, "cfg5 strict")


def ag_emulated_in(fo, xb, wb, c, arrival, release_ns, mode=None):
    """As ag_emulated with the default priority (order NULL) and peers landing
    in `arrival` order."""
    m, k = xb.shape
    n = wb.shape[0]
    R, local = c.R, c.local
    mc = m // R
    staging = dev_bf16(xb)
    w = dev_bf16(wb)
    x = staging.clone()
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    gs = torch.zeros(2 * R + 2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    side = side_stream()
    e = epoch()
    for q in arrival:
        x[q * mc:(q + 1) * mc].fill_(float("nan"))
    y = torch.full((m, n), float("nan"), device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        fo.fo_emulate_arrivals([x[q * mc:(q + 1) * mc] for q in arrival],
                               [staging[q * mc:(q + 1) * mc] for q in arrival],
                               [int(t) for t in release_ns], arrival, flags, e, es, stream=side,
                               gate=gs[2 * R:2 * R + 1])
    kw = {} if mode is None else {"mode": mode}
    fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=R, local=local, arrived=flags, epoch=e, stamps=gs,
                                       status=status, timeout_ns=5_000_000_000, **kw), ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "flag wait timed out"
    assert int(ws[:4096].sum()) == 0
    return [host(y)]


def test_qkv_r16_gauss_emulated_within_bar(fo, orc):
    """The same R = 16 emulated path on Gaussian inputs: within the bar on
    rows covering every chunk and every 256-row tile band (the split chunk's
    rows included), and run-to-run identical."""
    c = wl.CFG5
    xb, wb = wl.gemm_inputs(c, "gauss")
    order = wl.ring_arrival_order(c.R, c.local)
    nbytes = (c.m // c.R) * c.k * 2
    rel = wl.ring_release_ns(nbytes, c.R - 1, 200e9)
    log("case: cfg5 gauss, emulated 200 GB/s ring arrivals, two repetitions")
    y1, y2 = ag_emulated(fo, xb, wb, c.R, c.local, order + [c.local], rel, reps=2)
    assert np.array_equal(y1, y2), "split result not run-to-run identical"
    rows = np.unique(np.concatenate([np.arange(0, c.m, 37), np.arange(255, c.m, 256), [c.m - 1]]))
    check_tolerance(y1[rows], orc.gemm(xb[rows], wb), what="cfg5 gauss emulated")


def test_tp8_mlp_rs_full_int_partials_and_shards(fo, orc):
    """4096 x 4096 x 1792, R = 8: every partial element, and every shard
    element of the unfused reduce (bf16 and fp32), the fused reduce, and the
    ring form, exact."""
    c = wl.CFG3
    xb, wb, ref = int_case(orc, c)
    x, w = dev_bf16(xb), dev_bf16(wb)
    mc = c.m // c.R
    inc = wl.incoming_partials(c, "int")
    want = orc.gemm_rs_shard(xb, wb, c.R, c.local, inc)
    ws = torch.zeros(fo.fo_workspace_bytes(c.m, c.n, c.k, c.R), dtype=torch.uint8, device="cuda")
    part = torch.full((c.m, c.n), float("nan"), device="cuda")
    done = torch.zeros(c.R, dtype=torch.int32, device="cuda")
    e = epoch()
    log("case: cfg3 int gemm_rs partials")
    fo.fo_gemm_rs(x, w, part, done, fo.Schedule(nchunks=c.R, epoch=e), ws)
    torch.cuda.synchronize()
    assert (host(done) == e).all()
    check_exact(host(part), ref, "cfg3 partials")
    d_inc = [None if a is None else dev_f32(a) for a in inc]
    srcs = [part[c.local * mc:(c.local + 1) * mc] if q == c.local else d_inc[q] for q in range(c.R)]
    log("case: cfg3 int reduce, fp32 and bf16 shard")
    sh32 = torch.full((mc, c.n), float("nan"), device="cuda")
    fo.fo_chunk_reduce(sh32, srcs, fo.Schedule(nchunks=c.R, epoch=epoch()))
    torch.cuda.synchronize()
    check_exact(host(sh32), want, "cfg3 shard fp32")
    sh16 = torch.empty((mc, c.n), dtype=torch.bfloat16, device="cuda")
    fo.fo_chunk_reduce(sh16, srcs, fo.Schedule(nchunks=c.R, epoch=epoch()))
    torch.cuda.synchronize()
    assert np.array_equal(host(sh16), orc.f64_to_bf16(want)), "cfg3 shard bf16"
    log("case: cfg3 int fused gemm_rs_reduce")
    part.fill_(float("nan"))
    sh = torch.full((mc, c.n), float("nan"), device="cuda")
    e = epoch()
    fo.fo_gemm_rs_reduce(x, w, part, done, sh, d_inc, fo.Schedule(nchunks=c.R, epoch=e), ws)
    torch.cuda.synchronize()
    assert (host(done) == e).all()
    check_exact(host(part), ref, "cfg3 fused partials")
    check_exact(host(sh), want, "cfg3 fused shard")
    log("case: cfg3 int ring form")
    start = (c.local - 1) % c.R
    ring_inc = [None if q == start else d_inc[q if q != c.local else start] for q in range(c.R)]
    host_inc = [None if q == start else inc[q if q != c.local else start] for q in range(c.R)]
    fwd, shard = orc.ring_rs_rank(xb, wb, c.R, c.local, host_inc)
    # the local chunk's partial rows keep its own product; its sum is the shard
    fwd[c.local * mc:(c.local + 1) * mc] = ref[c.local * mc:(c.local + 1) * mc]
    part.fill_(float("nan"))
    sh.fill_(float("nan"))
    e = epoch()
    fo.fo_gemm_rs_ring(x, w, part, done, sh, ring_inc, fo.Schedule(nchunks=c.R, epoch=e), ws)
    torch.cuda.synchronize()
    assert (host(done) == e).all()
    check_exact(host(part), fwd, "cfg3 ring forwards")
    check_exact(host(sh), shard, "cfg3 ring shard")


def test_dp_reduce_full_int(fo, orc):
    """8 x 2^27 fp32 integer gradients, in place into the local source, all
    landed and with SDMA ring arrivals 2 ms apart in a seeded order: every
    element exact."""
    c = wl.CFG4
    srcs = wl.reduce_sources(c, "int")
    log("oracle: cfg4 int reduce 8 x 2^27")
    ref = orc.reduce(srcs)
    d = [dev_f32(s) for s in srcs]
    local = c.local
    order = [local] + [q for q in range(c.R) if q != local]
    fo.fo_chunk_reduce(d[local], d, fo.Schedule(nchunks=c.R, local=local, order=order, epoch=epoch()))
    torch.cuda.synchronize()
    check_exact(host(d[local]), ref, "cfg4 all landed")
    log("case: cfg4 int emulated arrivals")
    peers = wl.seeded_permutation([q for q in range(c.R) if q != local], 4)
    d[local].copy_(torch.from_numpy(srcs[local]))
    staging = [None] * c.R
    for q in peers:
        staging[q] = d[q]
        d[q] = torch.full((c.n,), float("nan"), device="cuda")
    flags = torch.zeros(c.R, dtype=torch.int32, device="cuda")
    es = torch.zeros(c.R + 2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    e = epoch()
    side = side_stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        fo.fo_emulate_arrivals([d[q] for q in peers], [staging[q] for q in peers],
                               [2_000_000 * (i + 1) for i in range(len(peers))], peers, flags, e, es,
                               stream=side)
    fo.fo_chunk_reduce(d[local], d, fo.Schedule(nchunks=c.R, local=local, order=[local] + peers, arrived=flags,
                                                epoch=e, status=status, timeout_ns=5_000_000_000))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_exact(host(d[local]), ref, "cfg4 emulated")


def test_tp8_mlp_ag_streamed_planned_schedule_int(fo, orc):
    """The schedule model's streamed plan at 50 GB/s ring links: each peer
    chunk sent as `sub` messages (pieces of m / (R * sub) rows) landing by
    SDMA into poisoned rows, the local pieces present, the plan's order and
    split: every element exact, and again with every chunk sent as 8."""
    c = wl.CFG2
    xb, wb, ref = int_case(orc, c)
    plans = [fo.fo_plan_ag_stream(c.m, c.n, c.k, c.R, c.local, 50.0, fo.FO_LINK_RING)[:3]]
    sub8 = 8
    land8 = fo.fo_plan_link_arrivals(c.R, c.local, c.m // c.R * c.k * 2, 50.0, fo.FO_LINK_RING, sub8)
    peers8 = sorted((p for p in range(c.R * sub8) if p // sub8 != c.local), key=lambda p: land8[p])
    split8 = [1] * (c.R * sub8)
    split8[peers8[-1]] = 8
    plans.append((sub8, peers8 + [c.local * sub8 + j for j in range(sub8)], split8))
    for sub, order, split in plans:
        R2 = c.R * sub
        mc2 = c.m // R2
        land = fo.fo_plan_link_arrivals(c.R, c.local, c.m // c.R * c.k * 2, 50.0, fo.FO_LINK_RING, sub)
        locals_ = [c.local * sub + j for j in range(sub)]
        peers = [p for p in order if p not in locals_]
        staging = dev_bf16(xb)
        w = dev_bf16(wb)
        x = staging.clone()
        for p in peers:
            x[p * mc2:(p + 1) * mc2].fill_(float("nan"))
        flags = torch.zeros(R2, dtype=torch.int32, device="cuda")
        e = epoch()
        flags[locals_] = e
        es = torch.zeros(R2 + 2, dtype=torch.int64, device="cuda")
        gs = torch.zeros(2 * R2 + 2, dtype=torch.int64, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        ws = torch.zeros(fo.fo_workspace_bytes(c.m, c.n, c.k, R2), dtype=torch.uint8, device="cuda")
        y = torch.full((c.m, c.n), float("nan"), device="cuda")
        torch.cuda.synchronize()
        log(f"case: cfg2 int streamed in {sub} messages, last piece split {max(split)}")
        side = side_stream()
        # the launch first: enqueueing many gated messages can block the host
        # until the gate (the launch's start) opens
        fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=R2, local=locals_[0], order=order, arrived=flags, epoch=e,
                                           stamps=gs, status=status, split=split, timeout_ns=5_000_000_000), ws)
        with torch.cuda.stream(side):
            fo.fo_emulate_arrivals([x[p * mc2:(p + 1) * mc2] for p in peers], [staging[p * mc2:(p + 1) * mc2] for p in peers],
                                   [land[p] for p in peers], peers, flags, e, es, stream=side, gate=gs[2 * R2:2 * R2 + 1])
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert int(ws[:4096].sum()) == 0
        check_exact(host(y), ref, f"streamed in {sub}")
        del x, y, staging
