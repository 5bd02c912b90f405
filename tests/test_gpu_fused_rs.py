"""GPU parity of fo_gemm_rs_reduce (GEMM-RS with the local chunk's reduce fused
in) against the fp64 oracle and against the unfused pair fo_gemm_rs +
fo_chunk_reduce, through the C ABI.

The shard sums the local partial and the incoming partials in the order
fo_chunk_reduce uses, so the fused and unfused shards must be bit-identical;
integer-valued inputs must equal the oracle exactly.
"""
import numpy as np
import pytest

import workloads as wl
from helpers import check_exact, check_tolerance, dev_bf16, dev_f32, host, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_EP = [20000]


def epoch():
    _EP[0] += 1
    return _EP[0]


@pytest.fixture(scope="module")
def fo():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sp_rank_adaptive_amd as fo
    fo.lib()
    return fo


def case(m, n, k, R, mode, seed, inc_std=1.0):
    xb = wl.bf16_operand((m, k), mode, 1.0, seed)
    wb = wl.bf16_operand((n, k), mode, 0.02 if mode == "gauss" else 1.0, seed + 1)
    mc = m // R
    inc = [wl.f32_operand((mc, n), mode, inc_std, seed + 10 + q) for q in range(R)]
    return xb, wb, inc


def run_fused(fo, xb, wb, inc, R, local, shard_dtype=torch.float32, grid=0, arrived=None, e=None):
    m, k = xb.shape
    n = wb.shape[0]
    mc = m // R
    x, w = dev_bf16(xb), dev_bf16(wb)
    part = torch.full((m, n), float("nan"), device="cuda")
    shard = torch.full((mc, n), float("nan"), dtype=shard_dtype, device="cuda")
    done = torch.zeros(R, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    incoming = [None if q == local else dev_f32(inc[q]) for q in range(R)]
    e = epoch() if e is None else e
    s = fo.Schedule(nchunks=R, local=local, epoch=e, arrived=arrived, status=status,
                    max_workgroups=grid, timeout_ns=5_000_000_000)
    fo.fo_gemm_rs_reduce(x, w, part, done, shard, incoming, s, ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "flag wait timed out"
    assert (host(done) == e).all()
    return host(part), host(shard.float()), (x, w, incoming)


@pytest.mark.parametrize("m,n,k,R,local,grid", [
    (1024, 448, 512, 4, 0, 0),      # shard units assigned statically when 1 unit per workgroup
    (1024, 448, 512, 4, 2, 64),     # fewer workgroups: dynamic shard claims
    (520, 136, 200, 5, 3, 0),       # ragged tiles
    (256, 512, 512, 1, 0, 0),       # one chunk: the shard is the partial
])
def test_fused_int_exact(fo, orc, m, n, k, R, local, grid):
    log(f"case: fused gemm_rs_reduce int {m}x{n}x{k} R={R} local={local} grid={grid}")
    xb, wb, inc = case(m, n, k, R, "int", 4100 + R + local)
    part, shard, _ = run_fused(fo, xb, wb, inc, R, local, grid=grid)
    check_exact(part, orc.gemm(xb, wb), "partials")
    ref = orc.gemm_rs_shard(xb, wb, R, local, [None if q == local else inc[q] for q in range(R)])
    check_exact(shard, ref, "shard")


def test_fused_bf16_shard(fo, orc):
    m, n, k, R, local = 1024, 448, 512, 4, 1
    xb, wb, inc = case(m, n, k, R, "int", 4200)
    _, shard, _ = run_fused(fo, xb, wb, inc, R, local, shard_dtype=torch.bfloat16)
    ref = orc.gemm_rs_shard(xb, wb, R, local, [None if q == local else inc[q] for q in range(R)])
    # integer sums below 2^8 * 2^8 are not all exact in bf16: compare with the
    # oracle rounded once to bf16
    exp = orc.bf16_to_f64(orc.f64_to_bf16(ref))
    check_exact(shard, exp, "bf16 shard")


def test_fused_matches_unfused_bitwise_cfg3(fo, orc):
    """cfg3 at full size, Gaussian: the fused shard and partials equal the
    unfused fo_gemm_rs + fo_chunk_reduce bit for bit, and the oracle within
    tolerance on sampled rows."""
    c = wl.CFG3
    xb, wb = wl.gemm_inputs(c, "gauss")
    inc = wl.incoming_partials(c, "gauss")
    inc = [np.zeros((c.m // c.R, c.n), np.float32) if a is None else a for a in inc]
    log("case: cfg3 fused vs unfused")
    part, shard, (x, w, incoming) = run_fused(fo, xb, wb, inc, c.R, c.local, shard_dtype=torch.bfloat16)
    # unfused
    mc = c.m // c.R
    part2 = torch.empty((c.m, c.n), device="cuda")
    done = torch.zeros(c.R, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(c.m, c.n, c.k, c.R), dtype=torch.uint8, device="cuda")
    e = epoch()
    fo.fo_gemm_rs(x, w, part2, done, fo.Schedule(nchunks=c.R, local=c.local, epoch=e), ws)
    shard2 = torch.empty((mc, c.n), dtype=torch.bfloat16, device="cuda")
    srcs = [part2[c.local * mc:(c.local + 1) * mc] if q == c.local else incoming[q] for q in range(c.R)]
    fo.fo_chunk_reduce(shard2, srcs, fo.Schedule(nchunks=c.R, local=c.local, epoch=e))
    torch.cuda.synchronize()
    assert np.array_equal(part.view(np.uint32), host(part2).view(np.uint32))
    assert np.array_equal(shard.view(np.uint32), host(shard2.float()).view(np.uint32))
    rows = np.arange(0, mc, 37)
    ref = orc.gemm_rs_shard(xb, wb, c.R, c.local, [None if q == c.local else inc[q] for q in range(c.R)])
    check_tolerance(shard[rows], ref[rows], frob_ref=orc.bf16_to_f64(orc.f64_to_bf16(ref[rows])),
                    what="cfg3 fused shard")


def test_fused_with_emulated_incoming(fo, orc):
    """Incoming partials land by SDMA into NaN-poisoned inboxes while the
    fused launch runs (the emulator starts with the kernel); the shard units
    wait for the flags and read the landed data coherently: exact on
    integers."""
    m, n, k, R, local = 1024, 448, 512, 8, 0
    xb, wb, inc = case(m, n, k, R, "int", 4300)
    mc = m // R
    x, w = dev_bf16(xb), dev_bf16(wb)
    staging = [None if q == local else dev_f32(inc[q]) for q in range(R)]
    inbox = [None if q == local else torch.full((mc, n), float("nan"), device="cuda") for q in range(R)]
    order = wl.ring_arrival_order(R, local)
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    gs = torch.zeros(2 * R + 2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    part = torch.empty((m, n), device="cuda")
    shard = torch.full((mc, n), float("nan"), device="cuda")
    done = torch.zeros(R, dtype=torch.int32, device="cuda")
    from test_gpu_emulated import side_stream
    side = side_stream()
    ref = orc.gemm_rs_shard(xb, wb, R, local, [None if q == local else inc[q] for q in range(R)])
    for rep in range(2):
        e = epoch()
        for q in order:
            inbox[q].fill_(float("nan"))
        shard.fill_(float("nan"))
        gs.zero_()
        torch.cuda.synchronize()
        rel = [10_000 * (i + 1) for i in range(len(order))]
        with torch.cuda.stream(side):
            fo.fo_emulate_arrivals([inbox[q] for q in order], [staging[q] for q in order], rel, order,
                                   flags, e, es, stream=side, gate=gs[2 * R:2 * R + 1])
        fo.fo_gemm_rs_reduce(x, w, part, done, shard, inbox,
                             fo.Schedule(nchunks=R, local=local, epoch=e, arrived=flags, stamps=gs,
                                         status=status, timeout_ns=5_000_000_000), ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "flag wait timed out"
        check_exact(host(shard), ref, f"fused shard with emulated arrivals, rep {rep}")
        # the shard was complete only after the last landing
        assert gs[2 * R + 1].item() >= max(int(es[1 + q].item()) for q in order)


# ---- ring form (fo_gemm_rs_ring) -------------------------------------------

def ring_incoming(m, n, R, local, mode, seed, std=1.0):
    """Accumulated partials from the predecessor, indexed by chunk: none for
    chunk local-1 (this rank starts its accumulation)."""
    mc = m // R
    start = (local - 1) % R
    return [None if (c == start and R > 1) else wl.f32_operand((mc, n), mode, std, seed + 10 + c)
            for c in range(R)]


def ring_expected_partial(orc, xb, wb, R, local, inc):
    """The partial buffer after a ring call: peer chunks hold their forwarded
    sums, the local chunk's rows its own partial (its sum goes to the shard)."""
    fwd, ref = orc.ring_rs_rank(xb, wb, R, local, inc)
    mc = xb.shape[0] // R
    fwd[local * mc:(local + 1) * mc] = orc.gemm(xb[local * mc:(local + 1) * mc], wb)
    return fwd, ref


def run_ring(fo, xb, wb, inc, R, local, shard_dtype=torch.float32, grid=0):
    m, k = xb.shape
    n = wb.shape[0]
    mc = m // R
    x, w = dev_bf16(xb), dev_bf16(wb)
    part = torch.full((m, n), float("nan"), device="cuda")
    shard = torch.full((mc, n), float("nan"), dtype=shard_dtype, device="cuda")
    done = torch.zeros(R, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    incoming = [None if a is None else dev_f32(a) for a in inc]
    e = epoch()
    s = fo.Schedule(nchunks=R, local=local, epoch=e, status=status, max_workgroups=grid,
                    timeout_ns=5_000_000_000)
    fo.fo_gemm_rs_ring(x, w, part, done, shard, incoming, s, ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "flag wait timed out"
    assert (host(done) == e).all()
    return host(part), host(shard.float()), (x, w, incoming)


@pytest.mark.parametrize("m,n,k,R,local,grid", [
    (1024, 448, 512, 4, 0, 0),
    (1024, 448, 512, 4, 2, 64),     # fewer workgroups than units
    (520, 136, 200, 5, 3, 0),       # ragged tiles
    (256, 512, 512, 1, 0, 0),       # one chunk: the shard is the partial (+ incoming, if any)
    (2048, 512, 256, 8, 5, 100),
])
def test_ring_int_exact(fo, orc, m, n, k, R, local, grid):
    log(f"case: ring gemm_rs int {m}x{n}x{k} R={R} local={local} grid={grid}")
    xb = wl.bf16_operand((m, k), "int", 1.0, 4400 + R + local)
    wb = wl.bf16_operand((n, k), "int", 1.0, 4401 + R + local)
    inc = ring_incoming(m, n, R, local, "int", 4410)
    part, shard, _ = run_ring(fo, xb, wb, inc, R, local, grid=grid)
    fwd, ref = ring_expected_partial(orc, xb, wb, R, local, inc)
    check_exact(part, fwd, "forwarded partials")
    check_exact(shard, ref, "shard")


def test_ring_bf16_shard_and_missing_local_incoming(fo, orc):
    m, n, k, R, local = 1024, 448, 512, 4, 1
    xb = wl.bf16_operand((m, k), "int", 1.0, 4500)
    wb = wl.bf16_operand((n, k), "int", 1.0, 4501)
    inc = ring_incoming(m, n, R, local, "int", 4510)
    inc[local] = None          # the shard is then the local partial itself
    part, shard, _ = run_ring(fo, xb, wb, inc, R, local, shard_dtype=torch.bfloat16)
    fwd, ref = ring_expected_partial(orc, xb, wb, R, local, inc)
    check_exact(part, fwd, "forwarded partials")
    check_exact(shard, orc.bf16_to_f64(orc.f64_to_bf16(ref)), "bf16 shard")


def test_ring_cfg3_bitwise_against_unfused_add(fo, orc):
    """cfg3 at full size, Gaussian: every forwarded chunk and the shard equal
    fo_gemm_rs's partial plus the incoming partial added once in fp32 (torch),
    bit for bit; the shard is within tolerance of the oracle on sampled rows."""
    c = wl.CFG3
    xb, wb = wl.gemm_inputs(c, "gauss")
    inc = ring_incoming(c.m, c.n, c.R, c.local, "gauss", 4600, std=0.847)
    log("case: cfg3 ring vs fo_gemm_rs + fp32 add")
    part, shard, (x, w, incoming) = run_ring(fo, xb, wb, inc, c.R, c.local)
    part2 = torch.empty((c.m, c.n), device="cuda")
    done = torch.zeros(c.R, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(c.m, c.n, c.k, c.R), dtype=torch.uint8, device="cuda")
    fo.fo_gemm_rs(x, w, part2, done, fo.Schedule(nchunks=c.R, local=c.local, epoch=epoch()), ws)
    mc = c.m // c.R
    lo = c.local * mc
    sh2 = part2[lo:lo + mc] + incoming[c.local]
    for q in range(c.R):
        if incoming[q] is not None and q != c.local:
            part2[q * mc:(q + 1) * mc] += incoming[q]
    torch.cuda.synchronize()
    p2 = host(part2)
    assert np.array_equal(part.view(np.uint32), p2.view(np.uint32))
    assert np.array_equal(shard.view(np.uint32), host(sh2).view(np.uint32))
    rows = np.arange(0, mc, 41)
    _, ref = orc.ring_rs_rank(xb, wb, c.R, c.local, inc)
    check_tolerance(shard[rows], ref[rows], what="cfg3 ring shard")


@pytest.mark.parametrize("grid", [0, 100])
def test_ring_with_emulated_arrivals(fo, orc, grid):
    """The accumulated partials land by SDMA into NaN-poisoned inboxes at ring
    times (chunk local-2 first, the local chunk last) while the launch runs:
    each chunk's sum starts only after its landing (chunk completion stamps
    after landing stamps), and the results are exact on integers.  grid 0:
    one GEMM unit per workgroup, shard units assigned statically; grid 100:
    dynamic claims, a chunk's shard units claimable once it has landed."""
    m, n, k, R, local = 1024, 448, 512, 8, 3
    log(f"case: ring with emulated arrivals, grid {grid}")
    xb = wl.bf16_operand((m, k), "int", 1.0, 4700)
    wb = wl.bf16_operand((n, k), "int", 1.0, 4701)
    inc = ring_incoming(m, n, R, local, "int", 4710)
    mc = m // R
    x, w = dev_bf16(xb), dev_bf16(wb)
    order = [(local - 2 - s) % R for s in range(R - 1)]          # landing order
    staging = {q: dev_f32(inc[q]) for q in order}
    inbox = [None] * R
    for q in order:
        inbox[q] = torch.full((mc, n), float("nan"), device="cuda")
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    gs = torch.zeros(2 * R + 2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    part = torch.empty((m, n), device="cuda")
    shard = torch.full((mc, n), float("nan"), device="cuda")
    done = torch.zeros(R, dtype=torch.int32, device="cuda")
    from test_gpu_emulated import side_stream
    side = side_stream()
    fwd, ref = ring_expected_partial(orc, xb, wb, R, local, inc)
    for rep in range(2):
        e = epoch()
        for q in order:
            inbox[q].fill_(float("nan"))
        shard.fill_(float("nan"))
        gs.zero_()
        torch.cuda.synchronize()
        rel = [15_000 * (i + 1) for i in range(len(order))]
        with torch.cuda.stream(side):
            fo.fo_emulate_arrivals([inbox[q] for q in order], [staging[q] for q in order], rel, order,
                                   flags, e, es, stream=side, gate=gs[2 * R:2 * R + 1])
        fo.fo_gemm_rs_ring(x, w, part, done, shard, inbox,
                           fo.Schedule(nchunks=R, local=local, epoch=e, arrived=flags, stamps=gs,
                                       status=status, timeout_ns=5_000_000_000, max_workgroups=grid), ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "flag wait timed out"
        assert (host(done) == e).all()
        check_exact(host(part), fwd, f"forwarded partials with emulated arrivals, rep {rep}")
        check_exact(host(shard), ref, f"ring shard with emulated arrivals, rep {rep}")
        g = host(gs)
        ev = host(es)
        for q in order:
            assert g[R + q] >= ev[1 + q], f"chunk {q} completed before its partial landed"
