"""Benchmark of the one-GPU FlashOverlap hot path on MI355X.

One step = one pass of the whole path over one batch of the tensor-parallel
MLP workload at TP=8 (one rank's share, every peer chunk landed, epoch flags
preset, inputs resident in HBM):
  1. fo_ag_gemm   X 4096x4096 (8 row-chunks) * W 4096x1792 -> Y fp32,
  2. fo_gemm_rs   X 4096x1792 * W 1792x4096 -> 8 partial chunks 512x4096 fp32,
  3. fo_chunk_reduce  local partial + 7 incoming fp32 partials -> 512x4096 bf16.
`value` = (AG + RS GEMM flops) / step time.  Extra fields report each call's
rate, the exposed tail under emulated 50 GB/s links (FlashOverlap schedule and
naive wait-then-compute), the DP gradient reduce-add rate, the long-sequence
QKV AG-GEMM rate, the roofline of the dominant kernel and the CPU oracle's
rate on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_tp8_mlp.json")
GEMM_SRC = os.path.join(ROOT, "sp_rank_adaptive_amd", "csrc", "fo_gemm.hip")


def source_hash(path: str) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(launch):
    """HBM bytes per launch of `launch` ("ag_gemm" or "gemm_rs") from the
    committed counter profile, or None when the profile is missing or the
    kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != source_hash(GEMM_SRC):
        return None
    return d.get("launches", {}).get(launch, {}).get("bytes_per_launch")


def copy_calibration(nbytes=1 << 29, reps=3):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE, WRITE_SIZE) of a profiled run."""
    import torch
    a = torch.ones(nbytes // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class Timer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, stream):
        self.stream = stream
        self.pairs = []

    def __enter__(self):
        import torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)
        self.a.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.b.record(self.stream)
        self.pairs.append((self.a, self.b))

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


class Path:
    """Device buffers for one rank's share of the TP=8 MLP (cfg2 + cfg3)."""

    def __init__(self, fo, mode="gauss"):
        import torch
        self.fo = fo
        c2, c3 = wl.CFG2, wl.CFG3
        self.c2, self.c3 = c2, c3
        x2, w2 = wl.gemm_inputs(c2, mode)
        x3, w3 = wl.gemm_inputs(c3, mode)
        self.x2, self.w2 = dev_bf16(x2), dev_bf16(w2)
        self.x3, self.w3 = dev_bf16(x3), dev_bf16(w3)
        self.y2 = torch.empty((c2.m, c2.n), device="cuda")
        self.part = torch.empty((c3.m, c3.n), device="cuda")
        mc3 = c3.m // c3.R
        inc = wl.incoming_partials(c3, mode)
        self.inc = [None if a is None else torch.from_numpy(a).cuda() for a in inc]
        self.shard = torch.empty((mc3, c3.n), dtype=torch.bfloat16, device="cuda")
        self.ws2 = torch.zeros(fo.fo_workspace_bytes(c2.m, c2.n, c2.k, c2.R), dtype=torch.uint8, device="cuda")
        self.ws3 = torch.zeros(fo.fo_workspace_bytes(c3.m, c3.n, c3.k, c3.R), dtype=torch.uint8, device="cuda")
        self.flags2 = torch.zeros(c2.R, dtype=torch.int32, device="cuda")
        self.done3 = torch.zeros(c3.R, dtype=torch.int32, device="cuda")
        self.epoch = 0
        self.srcs = [self.part[c3.local * mc3:(c3.local + 1) * mc3] if q == c3.local else self.inc[q]
                     for q in range(c3.R)]

    def step(self, timers=None):
        fo = self.fo
        self.epoch += 1
        e = self.epoch
        self.flags2.fill_(e)      # every peer chunk has landed
        t = timers or {}
        # every chunk has landed, so no chunk is split (the automatic policy
        # splits the chunk expected to land last, for the arrival case)
        with t.get("ag", _Null()):
            fo.fo_ag_gemm(self.x2, self.w2, self.y2,
                          fo.Schedule(nchunks=self.c2.R, arrived=self.flags2, epoch=e,
                                      split=[1] * self.c2.R), self.ws2)
        with t.get("rs", _Null()):
            fo.fo_gemm_rs(self.x3, self.w3, self.part, self.done3,
                          fo.Schedule(nchunks=self.c3.R, epoch=e), self.ws3)
        with t.get("red", _Null()):
            fo.fo_chunk_reduce(self.shard, self.srcs, fo.Schedule(nchunks=self.c3.R, epoch=e))


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


def _spread(out, values):
    """p10 and p90 of the repetitions, into the dict `out` when one is given."""
    if out is not None:
        out["p10"], out["p90"] = (round(float(v), 2) for v in np.percentile(values, [10, 90]))
        out["reps"] = len(values)


def ticks_to_us(t, hz):
    return float(t) * 1e6 / hz


def _hip_wait_value():
    """hipStreamWaitValue32 from the HIP runtime (for the sliced baseline)."""
    import ctypes
    L = ctypes.CDLL("libamdhip64.so")
    f = L.hipStreamWaitValue32
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint, ctypes.c_uint32]
    f.restype = ctypes.c_int
    return f


_SIDE = []


def side_stream():
    """The one side stream every emulated arrival runs on.  HIP multiplexes
    streams over a few hardware queues; a stream created per measurement can
    land on the main stream's queue, and the consumer kernel then waits behind
    the whole arrival sequence."""
    import torch
    if not _SIDE:
        _SIDE.append(torch.cuda.Stream())
    return _SIDE[0]


def _emulate(fo, dsts, srcs, order, nbytes, flags, e, es, side, link_bw, copy=True, gate=None):
    """Enqueue ring arrivals of `order` on the side stream: chunk s lands at
    s * B / BW, its copy issued B / BW earlier.  copy=False: the data are
    already in place and only the flags are released at those times.  gate:
    a device word (the consumer kernel's start stamp); the timeline starts
    once it is nonzero."""
    import torch
    rel = wl.ring_release_ns(nbytes, len(order), link_bw)
    iss = [r - nbytes / link_bw * 1e9 for r in rel] if copy else list(rel)
    with torch.cuda.stream(side):
        fo.fo_emulate_arrivals(dsts, srcs, rel, order, flags, e, es, issue_ns=iss,
                               nbytes=None if copy else [0] * len(order), stream=side, gate=gate)


def measure_tail_ag(fo, cfg, hz, schedule="flashoverlap", reps=20, link_bw=wl.LINK_BW, copy=True, split=None,
                    spread=None, sub=1, order=None):
    """Exposed tail of the AG-GEMM under emulated ring arrivals (us): time
    from the last chunk's landing to the last output written.
      flashoverlap: one persistent launch, ready-first claims over the flags;
      strict: the same launch taking chunks exactly in priority order;
      naive: wait for every chunk, then one GEMM launch;
      sliced: one launch per chunk, each after a stream wait on its flag.
    sub > 1 (flashoverlap): each peer's chunk is sent as `sub` messages of
    m/(R*sub) rows over the same link, one after another (the last byte lands
    when the whole chunk would have), and the launch sees R*sub chunks with
    the local ones flagged present; split then indexes those chunks."""
    import torch
    xb, wb = wl.gemm_inputs(cfg, "gauss")
    staging = dev_bf16(xb)
    w = dev_bf16(wb)
    x = staging.clone()
    y = torch.empty((cfg.m, cfg.n), device="cuda")
    if sub > 1:
        return _tail_ag_sub(fo, cfg, hz, staging, x, w, y, sub, reps, link_bw, split, spread, order)
    mc = cfg.m // cfg.R
    order = wl.ring_arrival_order(cfg.R, cfg.local)
    nbytes = mc * cfg.k * 2
    flags = torch.zeros(cfg.R, dtype=torch.int32, device="cuda")
    es = torch.zeros(cfg.R + 2, dtype=torch.int64, device="cuda")
    gs = torch.zeros(2 * cfg.R + 2, dtype=torch.int64, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(cfg.m, cfg.n, cfg.k, cfg.R), dtype=torch.uint8, device="cuda")
    side = side_stream()
    main = torch.cuda.current_stream()
    wait_value = _hip_wait_value() if schedule == "sliced" else None
    tails, spans = [], []
    start_idx = 2 * cfg.R
    for rep in range(reps + 1):   # the first repetition is a warm-up
        e = 100 + rep
        gs.zero_()
        torch.cuda.synchronize()
        emulate = lambda gate=None: _emulate(fo, [x[q * mc:(q + 1) * mc] for q in order],
                                             [staging[q * mc:(q + 1) * mc] for q in order],
                                             order, nbytes, flags, e, es, side, link_bw, copy, gate)
        # For consumers that wait on the flags themselves the emulator is
        # enqueued first with its timeline gated on the consumer kernel's
        # start stamp: its timer kernel is resident and waiting when the
        # consumer starts, so t0 follows the kernel start within about a
        # microsecond, as in a layer whose kernel runs while the transfers
        # start.  Ungated, the host's enqueue time decides which starts first
        # (tens of microseconds either way).
        if schedule == "naive":
            emulate()
            ev = torch.cuda.Event()
            ev.record(side)
            main.wait_event(ev)
            fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=cfg.R, epoch=e, stamps=gs), ws)
            done_idx = 2 * cfg.R + 1
        elif schedule == "sliced":
            one = torch.zeros(4, dtype=torch.int64, device="cuda")
            start_idx = None
            emulate(one[2:3])
            for q in [cfg.local] + order:
                if q != cfg.local:
                    st = wait_value(main.cuda_stream, flags[q:q + 1].data_ptr(), e, 0, 0xFFFFFFFF)
                    if st != 0:
                        raise RuntimeError(f"hipStreamWaitValue32 failed ({st})")
                rows = slice(q * mc, (q + 1) * mc)
                fo.fo_ag_gemm(x[rows], w, y[rows], fo.Schedule(nchunks=1, epoch=e, stamps=one), ws)
            gs_used = one
            done_idx = 3
        else:
            mode = fo.FO_SCHED_STRICT if schedule == "strict" else fo.FO_SCHED_READY_FIRST
            emulate(gs[start_idx:start_idx + 1])
            fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=cfg.R, epoch=e, arrived=flags, stamps=gs, mode=mode,
                                               timeout_ns=5_000_000_000, split=split), ws)
            done_idx = 2 * cfg.R + 1
        if schedule != "sliced":
            gs_used = gs
        torch.cuda.synchronize()
        e_st = es.cpu().numpy().astype(np.int64)
        g_st = gs_used.cpu().numpy().astype(np.int64)
        last_arrival = max(e_st[1 + q] for q in order)
        # the run starts at the emulator's t0 or at the consumer kernel's own
        # start, whichever is earlier
        t_start = e_st[0] if schedule == "naive" else min(e_st[0], g_st[2 if start_idx is None else start_idx])
        if rep > 0:
            tails.append(ticks_to_us(g_st[done_idx] - last_arrival, hz))
            spans.append(ticks_to_us(last_arrival - t_start, hz))
    _spread(spread, tails)
    return float(np.median(tails)), float(np.median(spans))


def sub_chunk_schedule(R, local, sub, nbytes, link_bw=wl.LINK_BW):
    """Ring arrivals with each peer chunk sent as `sub` messages: the launch's
    chunks are the R*sub sub-chunks (sub-chunk j of chunk c is index c*sub+j).
    Returns (priority order over the sub-chunks: peers' in landing order, then
    the local ones; the peers' sub-chunks in landing order; their release
    times in ns; the local sub-chunks)."""
    ring = wl.ring_arrival_order(R, local)
    step = nbytes / link_bw * 1e9
    peers, rel = [], []
    for s_, c in enumerate(ring):
        for j in range(sub):
            peers.append(c * sub + j)
            rel.append(s_ * step + (j + 1) * step / sub)
    locals_ = [local * sub + j for j in range(sub)]
    return peers + locals_, peers, rel, locals_


def _tail_ag_sub(fo, cfg, hz, staging, x, w, y, sub, reps, link_bw, split, spread, order=None):
    import torch
    R2 = cfg.R * sub
    mc2 = cfg.m // R2
    order0, peers, rel, locals_ = sub_chunk_schedule(cfg.R, cfg.local, sub, (cfg.m // cfg.R) * cfg.k * 2, link_bw)
    order = order0 if order is None else order
    nb2 = mc2 * cfg.k * 2
    iss = [r - nb2 / link_bw * 1e9 for r in rel]
    flags = torch.zeros(R2, dtype=torch.int32, device="cuda")
    es = torch.zeros(R2 + 2, dtype=torch.int64, device="cuda")
    gs = torch.zeros(2 * R2 + 2, dtype=torch.int64, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(cfg.m, cfg.n, cfg.k, R2), dtype=torch.uint8, device="cuda")
    side = side_stream()
    tails = []
    for rep in range(reps + 1):
        e = 700 + rep
        gs.zero_()
        for q in locals_:
            flags[q] = e            # the local rows are present
        torch.cuda.synchronize()
        # The launch goes first: with many messages the emulation's enqueue
        # can block the host until its gate (this launch's start) opens.
        fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=R2, local=locals_[0], order=order, arrived=flags, epoch=e,
                                           stamps=gs, timeout_ns=5_000_000_000, split=split), ws)
        with torch.cuda.stream(side):
            fo.fo_emulate_arrivals([x[q * mc2:(q + 1) * mc2] for q in peers], [staging[q * mc2:(q + 1) * mc2] for q in peers],
                                   rel, peers, flags, e, es, issue_ns=iss, stream=side, gate=gs[2 * R2:2 * R2 + 1])
        torch.cuda.synchronize()
        e_st = es.cpu().numpy().astype(np.int64)
        g_st = gs.cpu().numpy().astype(np.int64)
        last = max(e_st[1 + q] for q in peers)
        if rep > 0:
            tails.append(ticks_to_us(g_st[2 * R2 + 1] - last, hz))
    _spread(spread, tails)
    return float(np.median(tails)), 0.0


def measure_tail_rs(fo, cfg, hz, schedule="flashoverlap", reps=20, link_bw=wl.LINK_BW, copy=True, span=False,
                    spread=None):
    """Exposed tail of GEMM-RS + chunk reduce-add: the 7 incoming fp32
    partials of the local shard land by emulated ring arrivals; the tail is
    the time from the last landing to the bf16 shard written.
      flashoverlap: GEMM-RS, then a reduce that adds partials as they land;
      fused: one fo_gemm_rs_reduce launch whose shard units wait for them;
      ring: the ring form (fo_gemm_rs_ring): the accumulated partials of
        chunks local-2, local-3, ..., local land one per step and each is
        added to this rank's partial of its chunk (in place, to forward; the
        local chunk's sum is the shard);
      naive: wait for every partial, then GEMM-RS and the reduce;
      sliced: GEMM-RS, then one reduce launch per incoming partial, each
        after a stream wait on its flag, adding it to an fp32 accumulator
        (the last one writes the bf16 shard)."""
    import torch
    xb, wb = wl.gemm_inputs(cfg, "gauss")
    x, w = dev_bf16(xb), dev_bf16(wb)
    mc = cfg.m // cfg.R
    part = torch.empty((cfg.m, cfg.n), device="cuda")
    done = torch.zeros(cfg.R, dtype=torch.int32, device="cuda")
    inc = wl.incoming_partials(cfg, "gauss")
    staging = [None if a is None else torch.from_numpy(a).cuda() for a in inc]
    inbox = [None if a is None else (torch.empty_like(a) if copy else a.clone()) for a in staging]
    shard = torch.empty((mc, cfg.n), dtype=torch.bfloat16, device="cuda")
    order = wl.ring_arrival_order(cfg.R, cfg.local)
    if schedule == "ring":
        # chunk local-1 starts here (nothing incoming); the local chunk's
        # accumulated partial lands last
        start = (cfg.local - 1) % cfg.R
        order = [(cfg.local - 2 - s_) % cfg.R for s_ in range(cfg.R - 1)]
        staging[cfg.local], staging[start] = staging[start], None
        inbox[cfg.local], inbox[start] = inbox[start], None
    nbytes = mc * cfg.n * 4
    flags = torch.zeros(cfg.R, dtype=torch.int32, device="cuda")
    es = torch.zeros(cfg.R + 2, dtype=torch.int64, device="cuda")
    rs_st = torch.zeros(2, dtype=torch.int64, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(cfg.m, cfg.n, cfg.k, cfg.R), dtype=torch.uint8, device="cuda")
    side = side_stream()
    main = torch.cuda.current_stream()
    gs = torch.zeros(2 * cfg.R + 2, dtype=torch.int64, device="cuda")
    if schedule == "sliced":
        wait_value = _hip_wait_value()
        acc = torch.empty((mc, cfg.n), device="cuda")
    tails, spans = [], []
    for rep in range(reps + 1):   # the first repetition is a warm-up
        e = 200 + rep
        rs_st.zero_()
        gs.zero_()
        torch.cuda.synchronize()
        emulate = lambda gate=None: _emulate(fo, [inbox[q] for q in order], [staging[q] for q in order], order,
                                             nbytes, flags, e, es, side, link_bw, copy, gate)
        if schedule == "naive":
            emulate()
            ev = torch.cuda.Event()
            ev.record(side)
            main.wait_event(ev)
        else:
            # the emulator's timeline starts with the GEMM-RS kernel (see
            # measure_tail_ag)
            emulate(gs[2 * cfg.R:2 * cfg.R + 1])
        if schedule == "fused":
            fo.fo_gemm_rs_reduce(x, w, part, done, shard, inbox,
                                 fo.Schedule(nchunks=cfg.R, epoch=e, arrived=flags, stamps=gs,
                                             timeout_ns=5_000_000_000), ws)
        elif schedule == "ring":
            fo.fo_gemm_rs_ring(x, w, part, done, shard, inbox,
                               fo.Schedule(nchunks=cfg.R, epoch=e, arrived=flags, stamps=gs,
                                           timeout_ns=5_000_000_000), ws)
        elif schedule == "sliced":
            fo.fo_gemm_rs(x, w, part, done, fo.Schedule(nchunks=cfg.R, epoch=e, stamps=gs), ws)
            running = part[cfg.local * mc:(cfg.local + 1) * mc]
            for i, q in enumerate(order):
                st = wait_value(main.cuda_stream, flags[q:q + 1].data_ptr(), e, 0, 0xFFFFFFFF)
                if st != 0:
                    raise RuntimeError(f"hipStreamWaitValue32 failed ({st})")
                last = i == len(order) - 1
                fo.fo_chunk_reduce(shard if last else acc, [running, inbox[q]],
                                   fo.Schedule(nchunks=2, epoch=e, stamps=rs_st if last else None))
                running = acc
        else:
            fo.fo_gemm_rs(x, w, part, done, fo.Schedule(nchunks=cfg.R, epoch=e, stamps=gs), ws)
            srcs = [part[cfg.local * mc:(cfg.local + 1) * mc] if q == cfg.local else inbox[q]
                    for q in range(cfg.R)]
            arrived = None if schedule == "naive" else flags
            fo.fo_chunk_reduce(shard, srcs, fo.Schedule(nchunks=cfg.R, epoch=e, arrived=arrived, stamps=rs_st,
                                                        timeout_ns=5_000_000_000))
        torch.cuda.synchronize()
        e_st = es.cpu().numpy().astype(np.int64)
        last_arrival = max(e_st[1 + q] for q in order)
        g0 = int(gs[2 * cfg.R].item())
        t_start = e_st[0] if schedule == "naive" else min(e_st[0], g0)
        t_done = int(gs[2 * cfg.R + 1].item()) if schedule in ("fused", "ring") else int(rs_st[1].item())
        if rep > 0:
            tails.append(ticks_to_us(t_done - last_arrival, hz))
            spans.append(ticks_to_us(last_arrival - t_start, hz))
    _spread(spread, tails)
    if span:
        return float(np.median(tails)), float(np.median(spans))
    return float(np.median(tails))


def a2a_rate(fo, cfg, launches=30):
    """All-landed Flash All-to-All GEMM (flags preset) over launches in a row:
    (average us per launch, TFLOP/s)."""
    import torch
    pieces, wb = wl.a2a_pieces(cfg, "gauss")
    dp = [dev_bf16(p_) for p_ in pieces]
    w = dev_bf16(wb)
    y = torch.empty((cfg.m, cfg.n), device="cuda")
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    flags = torch.full((cfg.R,), 1 << 30, dtype=torch.int32, device="cuda")
    for e in range(3):
        fo.fo_a2a_gemm(dp, w, y, fo.Schedule(nchunks=cfg.R, epoch=1 + e, arrived=flags), ws)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(torch.cuda.current_stream())
    for e in range(launches):
        fo.fo_a2a_gemm(dp, w, y, fo.Schedule(nchunks=cfg.R, epoch=10 + e, arrived=flags), ws)
    b.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / launches
    return us, 2.0 * cfg.m * cfg.n * cfg.k / us / 1e6


def measure_tail_a2a(fo, cfg, hz, schedule="flashoverlap", reps=20, link_bw=wl.LINK_BW, spread=None):
    """Exposed tail of the Flash All-to-All GEMM: the peers' pieces land by
    emulated pairwise-exchange arrivals (piece local-s at step s); the tail is
    the time from the last landing to the last output tile written.
      flashoverlap: one launch that multiplies each piece once it landed;
      naive: wait for every piece, then the same launch."""
    import torch
    pieces, wb = wl.a2a_pieces(cfg, "gauss")
    staging = [dev_bf16(p_) for p_ in pieces]
    inbox = [t.clone() for t in staging]
    w = dev_bf16(wb)
    y = torch.empty((cfg.m, cfg.n), device="cuda")
    P, local = cfg.R, cfg.local
    order = [(local - s_) % P for s_ in range(1, P)]
    nbytes = cfg.m * (cfg.k // P) * 2
    flags = torch.zeros(P, dtype=torch.int32, device="cuda")
    es = torch.zeros(P + 2, dtype=torch.int64, device="cuda")
    gs = torch.zeros(2 * P + 2, dtype=torch.int64, device="cuda")
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    side = side_stream()
    main = torch.cuda.current_stream()
    tails, spans = [], []
    for rep in range(reps + 1):
        e = 400 + rep
        gs.zero_()
        torch.cuda.synchronize()
        if schedule == "naive":
            _emulate(fo, [inbox[q] for q in order], [staging[q] for q in order], order, nbytes, flags, e, es,
                     side, link_bw)
            ev = torch.cuda.Event()
            ev.record(side)
            main.wait_event(ev)
            fo.fo_a2a_gemm(inbox, w, y, fo.Schedule(nchunks=P, epoch=e, stamps=gs), ws)
        else:
            _emulate(fo, [inbox[q] for q in order], [staging[q] for q in order], order, nbytes, flags, e, es,
                     side, link_bw, gate=gs[2 * P:2 * P + 1])
            fo.fo_a2a_gemm(inbox, w, y, fo.Schedule(nchunks=P, epoch=e, arrived=flags, stamps=gs,
                                                    timeout_ns=5_000_000_000), ws)
        torch.cuda.synchronize()
        e_st = es.cpu().numpy().astype(np.int64)
        g_st = gs.cpu().numpy().astype(np.int64)
        last = max(e_st[1 + q] for q in order)
        if rep > 0:
            tails.append(ticks_to_us(g_st[2 * P + 1] - last, hz))
            spans.append(ticks_to_us(last - e_st[0], hz))
    _spread(spread, tails)
    return float(np.median(tails)), float(np.median(spans))


def qsa_rate(fo, cfg, launches=20):
    """All-landed query-split attention over launches in a row: (average us,
    TFLOP/s of the attention work: 4 S^2 d H, halved with the causal mask)."""
    import torch
    qkv = dev_bf16(wl.qkv_input(cfg, "gauss"))
    o = torch.empty((cfg.S, cfg.H * cfg.d), device="cuda")
    ws = torch.zeros(fo.fo_qsa_workspace_bytes(cfg.S, cfg.H, cfg.d, cfg.R), dtype=torch.uint8, device="cuda")
    sched = lambda e: fo.Schedule(nchunks=cfg.R, epoch=e)   # every chunk present: no flags
    for e in range(3):
        fo.fo_qsa_attention(qkv, o, cfg.H, cfg.d, cfg.causal, sched(1 + e), ws)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(torch.cuda.current_stream())
    for e in range(launches):
        fo.fo_qsa_attention(qkv, o, cfg.H, cfg.d, cfg.causal, sched(10 + e), ws)
    b.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / launches
    flops = 4.0 * cfg.S * cfg.S * cfg.d * cfg.H * (0.5 if cfg.causal else 1.0)
    return us, flops / us / 1e6


def measure_tail_qsa(fo, cfg, hz, schedule="flashoverlap", reps=20, link_bw=wl.LINK_BW, spread=None):
    """Exposed tail of query-split attention: the peers' chunks of QKV rows
    land by emulated ring arrivals; the tail is the time from the last landing
    to the last output row written.
      flashoverlap: one launch whose blocks run as their chunks land;
      naive: wait for every chunk, then the same launch."""
    import torch
    staging = dev_bf16(wl.qkv_input(cfg, "gauss"))
    qkv = staging.clone()
    o = torch.empty((cfg.S, cfg.H * cfg.d), device="cuda")
    R, local, c = cfg.R, cfg.local, cfg.S // cfg.R
    order = wl.ring_arrival_order(R, local)
    nbytes = c * 3 * cfg.H * cfg.d * 2
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    gs = torch.zeros(2 * R + 2, dtype=torch.int64, device="cuda")
    ws = torch.zeros(fo.fo_qsa_workspace_bytes(cfg.S, cfg.H, cfg.d, R), dtype=torch.uint8, device="cuda")
    side = side_stream()
    main = torch.cuda.current_stream()
    tails, spans = [], []
    for rep in range(reps + 1):
        e = 500 + rep
        gs.zero_()
        torch.cuda.synchronize()
        dsts = [qkv[q * c:(q + 1) * c] for q in order]
        srcs = [staging[q * c:(q + 1) * c] for q in order]
        if schedule == "naive":
            _emulate(fo, dsts, srcs, order, nbytes, flags, e, es, side, link_bw)
            ev = torch.cuda.Event()
            ev.record(side)
            main.wait_event(ev)
            fo.fo_qsa_attention(qkv, o, cfg.H, cfg.d, cfg.causal, fo.Schedule(nchunks=R, epoch=e, stamps=gs), ws)
        else:
            _emulate(fo, dsts, srcs, order, nbytes, flags, e, es, side, link_bw, gate=gs[2 * R:2 * R + 1])
            fo.fo_qsa_attention(qkv, o, cfg.H, cfg.d, cfg.causal,
                                fo.Schedule(nchunks=R, epoch=e, arrived=flags, stamps=gs, timeout_ns=5_000_000_000),
                                ws)
        torch.cuda.synchronize()
        e_st = es.cpu().numpy().astype(np.int64)
        g_st = gs.cpu().numpy().astype(np.int64)
        last = max(e_st[1 + q] for q in order)
        if rep > 0:
            tails.append(ticks_to_us(g_st[2 * R + 1] - last, hz))
            spans.append(ticks_to_us(last - e_st[0], hz))
    _spread(spread, tails)
    return float(np.median(tails)), float(np.median(spans))


def measure_sends(fo, cfg, hz, form="gemm_rs", reps=10, link_bw=wl.LINK_BW, schedule="flashoverlap"):
    """Send side of the reduce-scatter: the 7 peer-destined fp32 partials of
    the GEMM-RS share are sent by emulated SDMA copies, one link, each
    occupying it for B / BW.
      flashoverlap: each send starts once its chunk's done flag is released
        (fo_emulate_sends enqueued on the side stream before the launch);
      naive: the sends start after the launch has completed.
    Returns medians (us) of: the launch's duration, the first send's start
    after the launch start, and the last send's completion after the launch
    end (the sends' exposed tail)."""
    import torch
    xb, wb = wl.gemm_inputs(cfg, "gauss")
    x, w = dev_bf16(xb), dev_bf16(wb)
    R, local = cfg.R, cfg.local
    mc = cfg.m // R
    part = torch.empty((cfg.m, cfg.n), device="cuda")
    done = torch.zeros(R, dtype=torch.int32, device="cuda")
    gs = torch.zeros(2 * R + 2, dtype=torch.int64, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(cfg.m, cfg.n, cfg.k, R), dtype=torch.uint8, device="cuda")
    peers = wl.ring_arrival_order(R, local)
    inbox = [torch.empty((mc, cfg.n), device="cuda") for _ in peers]
    st = torch.zeros(2 * len(peers), dtype=torch.int64, device="cuda")
    shard = torch.empty((mc, cfg.n), dtype=torch.bfloat16, device="cuda")
    inc = [None if q == local else torch.zeros((mc, cfg.n), device="cuda") for q in range(R)]
    link_ns = [mc * cfg.n * 4 / link_bw * 1e9] * len(peers)
    side = side_stream()
    main = torch.cuda.current_stream()
    g_len, first, tail = [], [], []
    for rep in range(reps + 1):
        e = 900 + rep
        gs.zero_()
        torch.cuda.synchronize()
        enqueue = lambda: fo.fo_emulate_sends(done, e, inbox, [part[q * mc:(q + 1) * mc] for q in peers], peers,
                                              link_ns, st, timeout_ns=5_000_000_000, stream=side)
        if schedule != "naive":
            with torch.cuda.stream(side):
                enqueue()
        if form == "fused":
            fo.fo_gemm_rs_reduce(x, w, part, done, shard, inc, fo.Schedule(nchunks=R, epoch=e, stamps=gs), ws)
        else:
            fo.fo_gemm_rs(x, w, part, done, fo.Schedule(nchunks=R, epoch=e, stamps=gs), ws)
        if schedule == "naive":
            ev = torch.cuda.Event()
            ev.record(main)
            side.wait_event(ev)
            with torch.cuda.stream(side):
                enqueue()
        torch.cuda.synchronize()
        g = gs.cpu().numpy().astype(np.int64)
        t = st.cpu().numpy().astype(np.int64)
        if rep > 0:
            g_len.append(ticks_to_us(g[2 * R + 1] - g[2 * R], hz))
            first.append(ticks_to_us(t[0] - g[2 * R], hz))
            tail.append(ticks_to_us(t[-1] - g[2 * R + 1], hz))
    return float(np.median(g_len)), float(np.median(first)), float(np.median(tail))


def link_sweep(fo, hz, bws=(50e9, 153e9, 400e9, 1000e9)):
    """End-to-end time (first release to output complete) and exposed tail at
    several per-link bandwidths.  The data are copied in before the timed
    window and only the flags are released at the modelled ring times, so
    the sweep is not limited by the copy engine's own rate."""
    out = {}
    c2, c3 = wl.CFG2, wl.CFG3
    for bw in bws:
        row = {}
        # the schedule model's split, and every split of the last-landing chunk
        mc = c2.m // c2.R
        order = wl.ring_arrival_order(c2.R, c2.local)
        arr = [0] * c2.R
        for q, t in zip(order, wl.ring_release_ns(mc * c2.k * 2, c2.R - 1, bw)):
            arr[q] = int(t)
        _, plan_split, pred = fo.fo_plan_ag_schedule(c2.m, c2.n, c2.k, c2.R, c2.local, arr)
        last = order[-1]
        for i, sk in enumerate((1, 2, 4, 8)):
            sp = [1] * c2.R
            sp[last] = sk
            t, spn = measure_tail_ag(fo, c2, hz, "flashoverlap", link_bw=bw, copy=False, split=sp)
            row[f"cfg2_split{sk}_total_us"] = round(t + spn, 2)
            row[f"cfg2_split{sk}_predicted_us"] = round(pred[i] / 1e3, 2)
        row["cfg2_planned_split"] = plan_split[last]
        row["cfg2_planned_total_us"] = row[f"cfg2_split{plan_split[last]}_total_us"]
        for sched in ("flashoverlap", "naive", "sliced"):
            t, sp = measure_tail_ag(fo, c2, hz, sched, link_bw=bw, copy=False)
            row[f"cfg2_{sched}_total_us"] = round(t + sp, 2)
            row[f"cfg2_{sched}_tail_us"] = round(t, 2)
        row["cfg2_last_arrival_us"] = round(sp, 2)
        for sched in ("flashoverlap", "fused", "ring", "naive"):
            t, sp = measure_tail_rs(fo, c3, hz, sched, link_bw=bw, copy=False, span=True)
            row[f"cfg3_{sched}_total_us"] = round(t + sp, 2)
            row[f"cfg3_{sched}_tail_us"] = round(t, 2)
        row["cfg3_last_arrival_us"] = round(sp, 2)
        out[f"{bw / 1e9:g}GBps"] = row
        log(f"link sweep {bw / 1e9:g} GB/s: {row}")
    return out


def measure_tail_dp(fo, cfg, hz, schedule="flashoverlap", reps=10, link_bw=wl.LINK_BW, spread=None, mesh=False):
    """Exposed tail of the DP gradient reduce-add (in place into the local
    shard): the 7 peer chunks land by emulated arrivals in a seeded order; the
    tail is the time from the last landing to the reduce's completion.
    mesh=False: ring arrivals (chunk s lands at s * B / BW, SDMA copies).
    mesh=True: mesh-staggered arrivals, one link per peer, chunk s landing at
    B / BW + (s - 1) * 250 us; the copies of all seven would overlap on one
    GPU's copy engine, so the data are copied in before the timeline starts
    and only the flags are released at those times."""
    import torch
    n, R, local = cfg.n, cfg.R, 0
    srcs = [torch.randn(n, device="cuda") * 1e-3 for _ in range(R)]
    staging = [None if q == local else torch.randn(n, device="cuda") * 1e-3 for q in range(R)]
    order = wl.seeded_permutation([q for q in range(R) if q != local], 4)
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    st = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = side_stream()
    main = torch.cuda.current_stream()
    tails = []
    for rep in range(reps + 1):   # the first repetition is a warm-up
        e = 300 + rep
        st.zero_()
        torch.cuda.synchronize()
        if mesh:
            for q in order:
                srcs[q].copy_(staging[q])
            torch.cuda.synchronize()
            rel = wl.mesh_staggered_release_ns(n * 4, len(order), link_bw)
            with torch.cuda.stream(side):
                fo.fo_emulate_arrivals([srcs[q] for q in order], [staging[q] for q in order], rel, order, flags, e,
                                       es, issue_ns=list(rel), nbytes=[0] * len(order), stream=side)
        else:
            _emulate(fo, [srcs[q] for q in order], [staging[q] for q in order], order, n * 4, flags, e, es, side,
                     link_bw)
        if schedule == "naive":
            ev = torch.cuda.Event()
            ev.record(side)
            main.wait_event(ev)
        fo.fo_chunk_reduce(srcs[local], srcs, fo.Schedule(nchunks=R, local=local, order=[local] + order,
                                                          epoch=e, arrived=None if schedule == "naive" else flags,
                                                          stamps=st, timeout_ns=5_000_000_000))
        torch.cuda.synchronize()
        e_st = es.cpu().numpy().astype(np.int64)
        last_arrival = max(e_st[1 + q] for q in order)
        if rep > 0:
            tails.append(ticks_to_us(int(st[1].item()) - last_arrival, hz))
    del srcs, staging
    torch.cuda.empty_cache()
    _spread(spread, tails)
    return float(np.median(tails))


def chunk_gemm_us(fo, cfg, reps=20):
    """Standalone GEMM of one chunk (m/R rows, all present) with the
    library's best single-chunk schedule: the chunk alone has too few tiles
    to fill the GPU, so it is split along k (1, 2, 4 or 8 ways, the split
    policy of the tail chunk) and the fastest split is kept.  Returns
    (median us of the best split, that split, {split: us})."""
    import torch
    xb, wb = wl.gemm_inputs(cfg, "gauss", m=cfg.m // cfg.R)
    x, w = dev_bf16(xb), dev_bf16(wb)
    y = torch.empty((x.shape[0], cfg.n), device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(x.shape[0], cfg.n, cfg.k, 1), dtype=torch.uint8, device="cuda")
    per = {}
    for sk in (1, 2, 4, 8):
        if cfg.k // 64 < sk:
            continue
        tm = Timer(torch.cuda.current_stream())
        for i in range(reps + 3):
            s = fo.Schedule(nchunks=1, epoch=1 + i, split=[sk])
            if i >= 3:
                with tm:
                    fo.fo_ag_gemm(x, w, y, s, ws)
            else:
                fo.fo_ag_gemm(x, w, y, s, ws)
        torch.cuda.synchronize()
        per[sk] = round(float(np.median(tm.ms()) * 1e3), 2)
    best = min(per, key=per.get)
    return per[best], best, per


def gemm_rate(fo, cfg, reps=20):
    """All-present AG-GEMM TFLOP/s on a config (median launch time)."""
    import torch
    xb, wb = wl.gemm_inputs(cfg, "gauss")
    x, w = dev_bf16(xb), dev_bf16(wb)
    del xb
    y = torch.empty((cfg.m, cfg.n), device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(cfg.m, cfg.n, cfg.k, cfg.R), dtype=torch.uint8, device="cuda")
    tm = Timer(torch.cuda.current_stream())
    for i in range(reps + 3):
        s = fo.Schedule(nchunks=cfg.R, epoch=1 + i)
        if i >= 3:
            with tm:
                fo.fo_ag_gemm(x, w, y, s, ws)
        else:
            fo.fo_ag_gemm(x, w, y, s, ws)
    torch.cuda.synchronize()
    ms = float(np.median(tm.ms()))
    return 2.0 * cfg.m * cfg.n * cfg.k / (ms * 1e-3) / 1e12, ms


def fused_rs_us(fo, path, reps=50):
    """cfg3 all present: one fo_gemm_rs_reduce launch against fo_gemm_rs +
    fo_chunk_reduce on the same buffers (HIP events; means over reps)."""
    import torch
    c3 = path.c3
    stream = torch.cuda.current_stream()
    inc = [None if q == c3.local else path.inc[q] for q in range(c3.R)]
    tf, tu = Timer(stream), Timer(stream)
    for i in range(reps + 3):
        path.epoch += 1
        e = path.epoch
        with (tf if i >= 3 else _Null()):
            fo.fo_gemm_rs_reduce(path.x3, path.w3, path.part, path.done3, path.shard, inc,
                                 fo.Schedule(nchunks=c3.R, epoch=e), path.ws3)
        path.epoch += 1
        e = path.epoch
        with (tu if i >= 3 else _Null()):
            fo.fo_gemm_rs(path.x3, path.w3, path.part, path.done3, fo.Schedule(nchunks=c3.R, epoch=e), path.ws3)
            fo.fo_chunk_reduce(path.shard, path.srcs, fo.Schedule(nchunks=c3.R, epoch=e))
    torch.cuda.synchronize()
    return float(np.mean(tf.ms())) * 1e3, float(np.mean(tu.ms())) * 1e3


def reduce_rate(fo, cfg, reps=10):
    """All-landed DP reduce-add (in place) GB/s: (R+1) * n * 4 bytes per call."""
    import torch
    n = cfg.n
    srcs = [torch.randn(n, device="cuda") * 1e-3 for _ in range(cfg.R)]
    tm = Timer(torch.cuda.current_stream())
    for i in range(reps + 2):
        s = fo.Schedule(nchunks=cfg.R, epoch=1 + i)
        if i >= 2:
            with tm:
                fo.fo_chunk_reduce(srcs[0], srcs, s)
        else:
            fo.fo_chunk_reduce(srcs[0], srcs, s)
    torch.cuda.synchronize()
    ms = float(np.median(tm.ms()))
    nbytes = (cfg.R + 1) * n * 4
    del srcs
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9, ms


def library_gemm_us(m, n, k, launches=30):
    """The vendor library's bf16 GEMM on the same shape (torch.matmul, X @ W^T
    with W stored [n][k] as here, bf16 out): average us over launches in a
    row.  A reference for what this GPU sustains on the shape, not the
    product path."""
    import torch
    x = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
    w = torch.randn(n, k, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        x @ w.t()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(launches):
        x @ w.t()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / launches


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_set_threads(n):
    """Thread count of the oracle's OpenMP loops (its libgomp instance)."""
    import ctypes
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def cpu_baseline():
    """The oracle (fp64, all host threads) on the GEMMs of one whole step:
    the AG-GEMM 4096x1792x4096 and the GEMM-RS 4096x4096x1792 (120 GFLOP).
    Also: the oracle's reduce (exactly rounded sums) on an 8 x 2^24 sample of
    the DP gradient reduce at all threads and on one, and the tiny R=4
    AG-GEMM on one thread."""
    import oracle
    oracle.lib()
    cores = oracle.num_threads()
    flops = 0.0
    t = 0.0
    for c in (wl.CFG2, wl.CFG3):
        xb, wb = wl.gemm_inputs(c, "gauss")
        t0 = time.perf_counter()
        oracle.gemm(xb, wb)
        t += time.perf_counter() - t0
        flops += 2.0 * c.m * c.n * c.k
    out = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": f"fp64 oracle GEMMs of one step: AG 4096x1792x4096 + RS 4096x4096x1792 "
                     f"({flops / 1e9:.1f} GFLOP, {t:.1f} s)",
           "cpu_model": cpu_model()}
    n = 1 << 24
    srcs = wl.reduce_sources(wl.CFG4, "gauss", n=n)
    nbytes = (wl.CFG4.R + 1) * n * 4
    t0 = time.perf_counter()
    oracle.reduce(srcs)
    tr = time.perf_counter() - t0
    out["reduce_sample"] = {"what": "8 x 2^24 fp32 exactly rounded sums (1/8 of the DP gradient reduce)",
                            "gbps": round(nbytes / tr / 1e9, 2), "s": round(tr, 3), "cores": cores}
    try:
        _omp_set_threads(1)
        t0 = time.perf_counter()
        oracle.reduce(srcs)
        t1 = time.perf_counter() - t0
        c1 = wl.CFG1
        xb, wb = wl.gemm_inputs(c1, "int")
        t0 = time.perf_counter()
        oracle.gemm(xb, wb)
        tg = time.perf_counter() - t0
        out["one_core"] = {"reduce_sample_gbps": round(nbytes / t1 / 1e9, 2), "reduce_sample_s": round(t1, 3),
                           "tiny_ag_gemm_256x512x512_s": round(tg, 4),
                           "tiny_ag_gemm_gflops": round(2.0 * c1.m * c1.n * c1.k / tg / 1e9, 3)}
    finally:
        _omp_set_threads(cores)
    return out


def back_to_back_us(fo, path, which, launches=50):
    """Average duration of one launch of the AG-GEMM or the GEMM-RS of the
    step, measured with one pair of HIP events around `launches` launches in
    a row on the launch stream (nothing else between them), so the event
    record and the dispatch of each launch overlap the previous one."""
    import torch
    stream = torch.cuda.current_stream()
    c2, c3 = path.c2, path.c3
    e0 = path.epoch + 1
    path.epoch += launches + 1
    path.flags2.fill_(path.epoch)          # landed for every epoch of the batch
    calls = []
    for i in range(launches + 1):
        e = e0 + i
        if which == "ag_gemm":
            calls.append(lambda e=e: fo.fo_ag_gemm(path.x2, path.w2, path.y2,
                                                   fo.Schedule(nchunks=c2.R, arrived=path.flags2, epoch=e,
                                                               split=[1] * c2.R), path.ws2))
        else:
            calls.append(lambda e=e: fo.fo_gemm_rs(path.x3, path.w3, path.part, path.done3,
                                                   fo.Schedule(nchunks=c3.R, epoch=e), path.ws3))
    calls[0]()                              # warm
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for f in calls[1:]:
        f()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / launches


def profile_kernels(fo, names, launches):
    """Launch the named workloads `launches` times each (all inputs present)
    and nothing else, for profiler runs."""
    import torch
    names = ["step", "reduce4", "a2a", "qsa"] if names == "all" else names.split(",")
    for nm in names:
        if nm == "step":
            path = Path(fo)
            for _ in range(launches):
                path.step()
        elif nm == "reduce4":
            c4 = wl.CFG4
            srcs = [torch.randn(c4.n, device="cuda") * 1e-3 for _ in range(c4.R)]
            for i in range(launches):
                fo.fo_chunk_reduce(srcs[0], srcs, fo.Schedule(nchunks=c4.R, epoch=1 + i))
            torch.cuda.synchronize()
            del srcs
        elif nm == "a2a":
            a2a_rate(fo, wl.CFG6, launches=launches)
        elif nm == "qsa":
            qsa_rate(fo, wl.CFG7, launches=launches)
        elif nm == "library":
            # the vendor library's GEMM (torch.matmul) on the shapes of the
            # step's AG-GEMM, GEMM-RS and the QKV AG-GEMM, as a reference
            for cfg in (wl.CFG2, wl.CFG3, wl.CFG5):
                us = library_gemm_us(cfg.m, cfg.n, cfg.k, launches=launches)
                log(f"library GEMM {cfg.m}x{cfg.n}x{cfg.k}: {us:.1f} us")
        else:
            raise SystemExit(f"unknown workload {nm}")
        torch.cuda.synchronize()
        log(f"profiled workload {nm}: {launches} launches")


def sustain(fo, seconds):
    """The step's AG-GEMM back to back for `seconds` (clock sampling under load)."""
    path = Path(fo)
    t_end = time.perf_counter() + seconds
    n = 0
    next_log = time.perf_counter() + 1.0
    while time.perf_counter() < t_end:
        us = back_to_back_us(fo, path, "ag_gemm", launches=200)
        n += 200
        if time.perf_counter() >= next_log:
            log(f"sustain: {n} AG-GEMM launches, {us:.1f} us each")
            next_log += 1.0
    log(f"sustain done: {n} launches in {seconds:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="skip tails, cfg4/cfg5 and the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--link-sweep", action="store_true",
                    help="also sweep the per-link bandwidth (end-to-end time and tail per schedule)")
    ap.add_argument("--steps-only", action="store_true",
                    help="time the steps and launch nothing else (counter runs name the GEMM launches "
                         "by their order: fo_ag_gemm, fo_gemm_rs, ...)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB copy (for scaling profiled byte counters)")
    ap.add_argument("--profile-kernels", default="",
                    help="launch only these workloads, --launches times each, for a profiler run: "
                         "comma list of step (AG-GEMM, GEMM-RS, reduce of the TP=8 MLP share), reduce4 "
                         "(DP gradient reduce), a2a (Ulysses all-to-all GEMM), qsa (TP=4 attention), or all; "
                         "library runs the vendor GEMM (torch.matmul) on the GEMM shapes instead")
    ap.add_argument("--launches", type=int, default=5)
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="launch the AG-GEMM of the step back to back for this many seconds (to sample "
                         "the clocks under load), printing a line every second")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the path and runs on one GPU only; the "
              "library has no multi-GPU transport (its sharding is a design, not code).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sp_rank_adaptive_amd as fo
    torch.cuda.set_device(0)
    cus, lds, hz = fo.fo_device_info()
    log(f"device: {torch.cuda.get_device_name(0)} CUs={cus} LDS/CU={lds} wall_clock={hz} Hz")

    side_stream()   # created first, so it gets a hardware queue of its own
    if args.profile_kernels:
        profile_kernels(fo, args.profile_kernels, args.launches)
        if args.copy_calibration:
            copy_calibration()
        return
    if args.sustain > 0:
        sustain(fo, args.sustain)
        return
    path = Path(fo)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()
    timers = {"ag": Timer(stream), "rs": Timer(stream), "red": Timer(stream)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        path.step(timers)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    c2, c3 = wl.CFG2, wl.CFG3
    f_ag = 2.0 * c2.m * c2.n * c2.k
    f_rs = 2.0 * c3.m * c3.n * c3.k
    ag_ms = float(np.mean(timers["ag"].ms()))
    rs_ms = float(np.mean(timers["rs"].ms()))
    red_ms = float(np.mean(timers["red"].ms()))
    red_bytes = (c3.R * (c3.m // c3.R) * c3.n * 4) + (c3.m // c3.R) * c3.n * 2
    value = (f_ag + f_rs) / (ms_step * 1e-3) / 1e12
    # each GEMM launch's average duration over launches in a row (events
    # around the batch); the dominant kernel is the one with the longer one
    b2b = {"ag_gemm": back_to_back_us(fo, path, "ag_gemm"), "gemm_rs": back_to_back_us(fo, path, "gemm_rs")}
    launches = {"ag_gemm": (f_ag, b2b["ag_gemm"] * 1e-3, "fo_ag_gemm 4096x1792x4096 R=8"),
                "gemm_rs": (f_rs, b2b["gemm_rs"] * 1e-3, "fo_gemm_rs 4096x4096x1792 R=8")}
    dom = max(launches, key=lambda q: launches[q][1])
    d_flops, d_ms, d_what = launches[dom]
    achieved = d_flops / (d_ms * 1e-3) / 1e12
    log(f"back to back: ag {b2b['ag_gemm']:.1f} us, rs {b2b['gemm_rs']:.1f} us")
    lib_ag = library_gemm_us(c2.m, c2.n, c2.k)
    lib_rs = library_gemm_us(c3.m, c3.n, c3.k)
    log(f"library GEMM on the same shapes: ag {lib_ag:.1f} us, rs {lib_rs:.1f} us")
    log(f"step {ms_step * 1e3:.1f} us: ag {ag_ms * 1e3:.1f} us, rs {rs_ms * 1e3:.1f} us, "
        f"reduce {red_ms * 1e3:.1f} us")

    out = {
        "metric": "AG-GEMM/GEMM-RS TFLOP/s + exposed tail us (1 GPU); chunk-reduce GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "tp8_mlp_rank_share: ag_gemm 4096x1792x4096 R=8 + gemm_rs 4096x4096x1792 R=8 "
                        "+ reduce 8x(512x4096) fp32 -> bf16",
            "R": 8, "local": 0, "schedule": "ready_first, all chunks landed (flags preset)",
        },
        "ag_gemm": {"us": round(ag_ms * 1e3, 2), "tflops": round(f_ag / ag_ms / 1e9, 1),
                    "back_to_back_us": round(b2b["ag_gemm"], 2),
                    "back_to_back_tflops": round(f_ag / b2b["ag_gemm"] / 1e6, 1),
                    "traffic": committed_traffic("ag_gemm")},
        "gemm_rs": {"us": round(rs_ms * 1e3, 2), "tflops": round(f_rs / rs_ms / 1e9, 1),
                    "back_to_back_us": round(b2b["gemm_rs"], 2),
                    "back_to_back_tflops": round(f_rs / b2b["gemm_rs"] / 1e6, 1),
                    "traffic": committed_traffic("gemm_rs")},
        "reduce_cfg3": {"us": round(red_ms * 1e3, 2), "gbps": round(red_bytes / red_ms / 1e6, 1)},
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": committed_traffic(dom),
            "kernel": f"gemm_kernel, {d_what} launch", "launch_us": round(d_ms * 1e3, 2),
            "flops_per_launch": d_flops,
            "timing": "HIP events around 50 launches in a row on the launch stream",
        },
        "library_reference": {
            "what": "torch.matmul (hipBLASLt) bf16 GEMM on the same shapes, launches in a row",
            "ag_gemm_shape_us": round(lib_ag, 2), "ag_gemm_shape_tflops": round(f_ag / lib_ag / 1e6, 1),
            "gemm_rs_shape_us": round(lib_rs, 2), "gemm_rs_shape_tflops": round(f_rs / lib_rs / 1e6, 1),
        },
        "pages_context": {
            "training_time_reduction": "up to 25% shorter training time, no hardware added",
            "source": "euno.news digest, Practical Implications",
            "hardware": "not stated by the pages", "role": "context, not the target",
        },
    }
    if not args.steps_only:
        f_us, u_us = fused_rs_us(fo, path)
        out["gemm_rs_reduce_fused_cfg3"] = {"us": round(f_us, 2), "unfused_rs_plus_reduce_us": round(u_us, 2)}
        log(f"fused GEMM-RS + reduce {f_us:.1f} us against {u_us:.1f} us unfused")
    if not args.quick and not args.steps_only:
        for cfg in (wl.CFG5,):
            tf, ms = gemm_rate(fo, cfg)
            out["qkv_ag_gemm_cfg5"] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1)}
        us, tf = a2a_rate(fo, wl.CFG6)
        out["a2a_gemm_ulysses_cfg6"] = {"us": round(us, 2), "tflops": round(tf, 1),
                                        "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                        "timing": "HIP events around 30 launches in a row, pieces landed"}
        log(f"a2a ulysses: {us:.1f} us, {tf:.0f} TFLOP/s")
        us, tf = qsa_rate(fo, wl.CFG7)
        out["qsa_attention_tp4_cfg7"] = {"us": round(us, 2), "tflops": round(tf, 1),
                                         "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                         "timing": "HIP events around 20 launches in a row, chunks landed"}
        log(f"qsa attention: {us:.1f} us, {tf:.0f} TFLOP/s")
        gbps, ms = reduce_rate(fo, wl.CFG4)
        out["dp_reduce_cfg4"] = {"us": round(ms * 1e3, 1), "gbps": round(gbps, 1),
                                 "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)}
        tails = {}
        for cfg, key in ((c2, "cfg2_ag_gemm"), (wl.CFG5, "cfg5_qkv_ag_gemm")):
            cg, cg_split, cg_per = chunk_gemm_us(fo, cfg)
            log(f"  {key} chunk GEMM {cg:.1f} us (split {cg_split})")
            at70 = 2.0 * (cfg.m // cfg.R) * cfg.n * cfg.k / (0.7 * PEAK_BF16_TFLOPS * 1e12) * 1e6
            row = {"chunk_gemm_us": round(cg, 2), "chunk_gemm_split": cg_split, "chunk_gemm_us_per_split": cg_per,
                   "chunk_gemm_at_70pct_peak_us": round(at70, 2)}
            for sched in ("flashoverlap", "strict", "naive", "sliced"):
                sp = {}
                t, span = measure_tail_ag(fo, cfg, hz, sched, spread=sp)
                log(f"  {key} {sched}: tail {t:.1f} us")
                row[sched + "_us"] = round(t, 2)
                row[sched + "_p10_p90_us"] = [sp["p10"], sp["p90"]]
                row["last_arrival_us"] = round(span, 1)
                row["reps"] = sp["reps"]
            # primary: the tail against the chunk's flops at 70% of peak;
            # also against the best measured single-chunk launch
            row["tail_over_chunk_gemm_at_70pct"] = round(row["flashoverlap_us"] / at70, 3)
            row["tail_over_chunk_gemm"] = round(row["flashoverlap_us"] / cg, 3)
            # the schedule model's order and split for these ring arrivals
            order = wl.ring_arrival_order(cfg.R, cfg.local)
            arr = [0] * cfg.R
            for q, t_ in zip(order, wl.ring_release_ns((cfg.m // cfg.R) * cfg.k * 2, cfg.R - 1, wl.LINK_BW)):
                arr[q] = int(t_)
            p_order, p_split, _ = fo.fo_plan_ag_schedule(cfg.m, cfg.n, cfg.k, cfg.R, cfg.local, arr)
            assert p_order == order + [cfg.local]   # the default priority
            sp = {}
            t, _ = measure_tail_ag(fo, cfg, hz, "flashoverlap", split=p_split, spread=sp)
            log(f"  {key} planned split {p_split[order[-1]]}: tail {t:.1f} us")
            row["planned_split"] = p_split[order[-1]]
            row["planned_us"] = round(t, 2)
            row["planned_p10_p90_us"] = [sp["p10"], sp["p90"]]
            row["planned_tail_over_chunk_gemm_at_70pct"] = round(t / at70, 3)
            row["planned_tail_over_chunk_gemm"] = round(t / cg, 3)
            # the streamed schedule: the model, calibrated on this shape's
            # measured all-present launch and lone chunk, chooses how many
            # messages each peer chunk is sent in and the last piece's split
            all_us = launches["ag_gemm"][1] * 1e3 if cfg is c2 else gemm_rate(fo, cfg)[1] * 1e3
            cal = fo.fo_plan_calibrate(cfg.m, cfg.n, cfg.k, cfg.R, all_us * 1e3, cg_per[1] * 1e3, 0.0)
            sub, s_order, s_split, s_pred = fo.fo_plan_ag_stream(cfg.m, cfg.n, cfg.k, cfg.R, cfg.local,
                                                                  wl.LINK_BW / 1e9, fo.FO_LINK_RING, calib=cal)
            sp = {}
            t, _ = measure_tail_ag(fo, cfg, hz, "flashoverlap", split=s_split, spread=sp, sub=sub, order=s_order)
            last_piece = s_order[cfg.R * sub - sub - 1]
            pred_end = min(v for v in s_pred[[1, 2, 4, 8].index(sub)] if v > 0)
            row["streamed"] = {"messages_per_chunk": sub, "last_piece_split": s_split[last_piece],
                               "tail_us": round(t, 2), "p10_p90_us": [sp["p10"], sp["p90"]],
                               "predicted_tail_us": round(pred_end / 1e3 - row["last_arrival_us"], 2),
                               "tail_over_chunk_gemm_at_70pct": round(t / at70, 3),
                               "calibration": {"gemm_tflops": round(cal.gemm_tflops, 1),
                                               "alone_speedup": round(cal.alone_speedup, 3)}}
            tails[key] = row
            log(f"tail {key}: {row}")
        row = {}
        for s_ in ("flashoverlap", "fused", "ring", "naive", "sliced"):
            sp = {}
            row[s_ + "_us"] = round(measure_tail_rs(fo, c3, hz, s_, spread=sp), 2)
            row[s_ + "_p10_p90_us"] = [sp["p10"], sp["p90"]]
            row["reps"] = sp["reps"]
        tails["cfg3_gemm_rs_reduce"] = row
        log(f"tail cfg3: {row}")
        row = {}
        for bw in (50e9, 1000e9):
            for form in ("gemm_rs", "fused"):
                for sched in ("flashoverlap", "naive"):
                    glen, first, tail = measure_sends(fo, c3, hz, form, link_bw=bw, schedule=sched)
                    row[f"{form}_{sched}_{bw / 1e9:g}GBps"] = {"launch_us": round(glen, 2),
                                                               "first_send_start_us": round(first, 2),
                                                               "last_send_after_launch_end_us": round(tail, 2)}
        tails["cfg3_peer_sends"] = row
        log(f"sends cfg3: {row}")
        c6 = wl.CFG6
        row = {"piece_gemm_at_70pct_peak_us": round(2.0 * c6.m * c6.n * (c6.k // c6.R) /
                                                    (0.7 * PEAK_BF16_TFLOPS * 1e12) * 1e6, 2)}
        for s_ in ("flashoverlap", "naive"):
            sp = {}
            t, span = measure_tail_a2a(fo, c6, hz, s_, spread=sp)
            row[s_ + "_us"] = round(t, 2)
            row[s_ + "_p10_p90_us"] = [sp["p10"], sp["p90"]]
            row["last_arrival_us"] = round(span, 1)
            row["reps"] = sp["reps"]
        row["tail_over_piece_gemm_at_70pct"] = round(row["flashoverlap_us"] / row["piece_gemm_at_70pct_peak_us"], 3)
        tails["cfg6_ulysses_a2a_gemm"] = row
        log(f"tail cfg6: {row}")
        row = {}
        for s_ in ("flashoverlap", "naive"):
            sp = {}
            t, span = measure_tail_qsa(fo, wl.CFG7, hz, s_, spread=sp)
            row[s_ + "_us"] = round(t, 2)
            row[s_ + "_p10_p90_us"] = [sp["p10"], sp["p90"]]
            row["last_arrival_us"] = round(span, 1)
            row["reps"] = sp["reps"]
        tails["cfg7_query_split_attention"] = row
        log(f"tail cfg7: {row}")
        row = {}
        for s_ in ("flashoverlap", "naive"):
            sp = {}
            row[s_ + "_us"] = round(measure_tail_dp(fo, wl.CFG4, hz, s_, spread=sp), 1)
            row[s_ + "_p10_p90_us"] = [sp["p10"], sp["p90"]]
            row["reps"] = sp["reps"]
        mesh = {"arrivals": "mesh-staggered, flags only (data copied in before t0)"}
        for s_ in ("flashoverlap", "naive"):
            sp = {}
            mesh[s_ + "_us"] = round(measure_tail_dp(fo, wl.CFG4, hz, s_, spread=sp, mesh=True), 1)
            mesh[s_ + "_p10_p90_us"] = [sp["p10"], sp["p90"]]
        row["mesh_staggered"] = mesh
        tails["cfg4_dp_reduce"] = row
        log(f"tail cfg4: {row}")
        out["tails_50GBps_links"] = tails
    if args.link_sweep:
        out["link_sweep_flags_only"] = link_sweep(fo, hz)
    if args.copy_calibration:
        copy_calibration()
    if not args.quick and not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
