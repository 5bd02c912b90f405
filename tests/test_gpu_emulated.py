"""GPU tests of the full path with emulated peers: SDMA copies from a staging
region land at modelled times, epoch flags release them, and the kernels
consume them as they land.

Race detection: before every call the peer destinations are filled with NaN
by a kernel (so poisoned lines may sit in the XCDs' L2s), flags are never
reset between calls (only the epoch grows), and arrivals are also delivered
out of priority order.  Any read of a chunk before its copy is visible shows
up as a NaN or a wrong integer in the output, which must equal the oracle
exactly on integer inputs.
"""
import numpy as np
import pytest

import workloads as wl
from helpers import check_exact, check_tolerance, dev_bf16, dev_f32, host, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fo():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sp_rank_adaptive_amd as fo
    fo.lib()
    return fo


_EP = [5000]
_SIDE = []


def side_stream():
    """One side stream for every emulated arrival in this process, created
    on first use (the first stream the process creates, as in bench.py), so
    it does not share a hardware queue with the stream the kernels run on:
    a consumer enqueued before a gated emulator would otherwise wait for
    flags that the emulator, queued behind it, cannot set."""
    if not _SIDE:
        _SIDE.append(torch.cuda.Stream())
    return _SIDE[0]


def epoch():
    _EP[0] += 1
    return _EP[0]


def ag_with_emulated_peers(fo, xb, wb, R, local, arrival, gap_ns, mode=None, reps=3,
                           split=None, gated=False):
    """Runs fo_ag_gemm with peers landing in `arrival` order, gap_ns apart;
    returns the outputs of every repetition and the stamps of the last.
    gated: the emulator's timeline starts at the GEMM kernel's start stamp
    (fo_emulate_arrivals_gated); its timer kernel waits for it."""
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
    outs = []
    for rep in range(reps):
        e = epoch()
        for q in arrival:                        # poison every peer destination
            x[q * mc:(q + 1) * mc].fill_(float("nan"))
        y = torch.full((m, n), float("nan"), device="cuda")
        gs.zero_()
        torch.cuda.synchronize()
        rel = [gap_ns * (i + 1) for i in range(len(arrival))]

        def emulate(gate=None):
            with torch.cuda.stream(side):
                fo.fo_emulate_arrivals([x[q * mc:(q + 1) * mc] for q in arrival],
                                       [staging[q * mc:(q + 1) * mc] for q in arrival],
                                       rel, arrival, flags, e, es, stream=side, gate=gate)

        emulate(gs[2 * R:2 * R + 1] if gated else None)
        kw = {} if mode is None else {"mode": mode}
        fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=R, local=local, arrived=flags, epoch=e,
                                           stamps=gs, status=status, split=split,
                                           timeout_ns=5_000_000_000, **kw), ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "flag wait timed out"
        outs.append(host(y))
    return outs, host(es).astype(np.int64), host(gs).astype(np.int64)


def test_ag_gemm_emulated_poisoned_int_exact(fo, orc):
    m, n, k, R, local = 1024, 448, 512, 8, 0
    xb = wl.bf16_operand((m, k), "int", 1.0, 3001)
    wb = wl.bf16_operand((n, k), "int", 1.0, 3002)
    ref = orc.gemm(xb, wb)
    arrival = wl.ring_arrival_order(R, local)
    log("case: emulated ring arrivals, poisoned destinations, 20 us apart")
    outs, es, gs = ag_with_emulated_peers(fo, xb, wb, R, local, arrival, 20_000)
    for y in outs:
        check_exact(y, ref, "emulated AG-GEMM")
    # every chunk landed after the emulator's start, in the order it was sent
    t = [es[1 + q] for q in arrival]
    assert all(b >= a for a, b in zip(t, t[1:])) and t[0] > es[0]
    # the last output was written after the last landing
    assert gs[2 * R + 1] >= max(t)


def test_ag_gemm_emulated_gated_timeline_int_exact(fo, orc):
    """The emulated peers start sending when the GEMM kernel starts (the
    emulator waits for its start stamp): poisoned destinations, integer
    inputs exact, and the emulator's t0 comes after the kernel's start
    stamp."""
    m, n, k, R, local = 1024, 448, 512, 8, 0
    xb = wl.bf16_operand((m, k), "int", 1.0, 3011)
    wb = wl.bf16_operand((n, k), "int", 1.0, 3012)
    ref = orc.gemm(xb, wb)
    arrival = wl.ring_arrival_order(R, local)
    log("case: gated emulator timeline, poisoned destinations, 5 us apart")
    outs, es, gs = ag_with_emulated_peers(fo, xb, wb, R, local, arrival, 5_000, gated=True)
    for y in outs:
        check_exact(y, ref, "gated emulated AG-GEMM")
    assert gs[2 * R] > 0 and es[0] >= gs[2 * R]
    t = [es[1 + q] for q in arrival]
    assert all(b >= a for a, b in zip(t, t[1:])) and t[0] > es[0]
    assert gs[2 * R + 1] >= max(t)


@pytest.mark.parametrize("local", [0, 3])
def test_ag_gemm_emulated_out_of_order_arrivals(fo, orc, local):
    """Arrivals in a seeded random order (not the priority order): the
    ready-first claim computes whatever has landed; result unchanged."""
    m, n, k, R = 512, 256, 256, 8
    xb = wl.bf16_operand((m, k), "int", 1.0, 3101 + local)
    wb = wl.bf16_operand((n, k), "int", 1.0, 3102)
    ref = orc.gemm(xb, wb)
    peers = [q for q in range(R) if q != local]
    arrival = wl.seeded_permutation(peers, 77 + local)
    outs, _, _ = ag_with_emulated_peers(fo, xb, wb, R, local, arrival, 5_000, reps=2)
    for y in outs:
        check_exact(y, ref, "out of order")
    # STRICT mode waits for each chunk in priority order
    outs, _, _ = ag_with_emulated_peers(fo, xb, wb, R, local, arrival, 5_000, reps=1,
                                        mode=fo.FO_SCHED_STRICT)
    check_exact(outs[0], ref, "strict")


def test_ag_gemm_emulated_tail_split_gauss(fo, orc):
    """cfg2's shapes at a fast link: the tail chunk is split (auto policy);
    Gaussian inputs within tolerance, split bits run-to-run identical."""
    c = wl.CFG2
    xb, wb = wl.gemm_inputs(c, "gauss")
    arrival = wl.ring_arrival_order(c.R, c.local)
    log("case: cfg2 emulated, split tail chunk")
    outs, es, gs = ag_with_emulated_peers(fo, xb, wb, c.R, c.local, arrival, 30_000, reps=2)
    assert np.array_equal(outs[0], outs[1])
    rows = np.unique(np.concatenate([np.arange(0, c.m, 61), [c.m - 1]]))
    check_tolerance(outs[0][rows], orc.gemm(xb[rows], wb), what="cfg2 emulated")


def test_reduce_emulated_poisoned(fo, orc):
    """DP reduce-add with peer gradients landing by SDMA into poisoned slots;
    in place into the local source; integer inputs exact."""
    R, n, local = 8, 1 << 20, 0
    srcs = wl.reduce_sources(wl.ReduceCfg(4, "t", n, R), "int", n=n)
    ref = orc.reduce(srcs)
    staging = [dev_f32(s) for s in srcs]
    order = [3, 6, 1, 7, 2, 5, 4]
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    side = side_stream()
    for rep in range(3):
        e = epoch()
        dst = [staging[local].clone() if q == local else torch.full((n,), float("nan"), device="cuda")
               for q in range(R)]
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            fo.fo_emulate_arrivals([dst[q] for q in order], [staging[q] for q in order],
                                   [10_000 * (i + 1) for i in range(len(order))], order,
                                   flags, e, es, stream=side)
        fo.fo_chunk_reduce(dst[local], dst, fo.Schedule(nchunks=R, local=local, order=[local] + order,
                                                        arrived=flags, epoch=e, status=status,
                                                        timeout_ns=5_000_000_000))
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        check_exact(host(dst[local]), ref, f"emulated reduce rep {rep}")


def test_emulator_release_times(fo):
    """Flags are set no earlier than their release times (device clock)."""
    cus, lds, hz = fo.fo_device_info()
    R = 4
    src = torch.arange(4096, dtype=torch.float32, device="cuda")
    dsts = [torch.zeros(4096, device="cuda") for _ in range(R - 1)]
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    rel = [50_000, 100_000, 150_000]
    e = epoch()
    fo.fo_emulate_arrivals(dsts, [src] * 3, rel, [1, 2, 3], flags, e, es)
    torch.cuda.synchronize()
    st = host(es).astype(np.int64)
    for i, q in enumerate([1, 2, 3]):
        assert (st[1 + q] - st[0]) * 1e9 / hz >= rel[i] - 1000
        assert torch.equal(dsts[i], src)
    assert (host(flags)[1:] == e).all()
