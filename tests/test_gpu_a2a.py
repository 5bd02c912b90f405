"""GPU parity of fo_a2a_gemm (Flash All-to-All output projection) against the
fp64 oracle, through the C ABI: every piece order, ragged shapes and piece
widths, emulated SDMA arrivals into NaN-poisoned inboxes (pairwise-exchange
order and out of order), the flag timeout, and the Ulysses workload at full
size (16K tokens, d_model 4096, degree 8) unsampled on integer inputs."""
import itertools

import numpy as np
import pytest

import workloads as wl
from helpers import bf16_bits_to_f64, check_exact, check_tolerance, dev_bf16, host, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_EP = [40000]
_SIDE = []


def epoch():
    _EP[0] += 1
    return _EP[0]


def side_stream():
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


def case(m, k, n, P, mode, seed):
    x = wl.bf16_operand((m, k), mode, 1.0, seed)
    w = wl.bf16_operand((n, k), mode, 0.02 if mode == "gauss" else 1.0, seed + 1)
    kp = k // P
    return [np.ascontiguousarray(x[:, q * kp:(q + 1) * kp]) for q in range(P)], w


def run(fo, pieces_b, wb, P, y_dtype=torch.float32, ws=None, **sched):
    m = pieces_b[0].shape[0]
    n = wb.shape[0]
    pieces = [dev_bf16(p) for p in pieces_b]
    w = dev_bf16(wb)
    y = torch.full((m, n), float("nan"), dtype=y_dtype, device="cuda")
    if ws is None:
        ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    fo.fo_a2a_gemm(pieces, w, y, fo.Schedule(nchunks=P, epoch=epoch(), **sched), ws)
    torch.cuda.synchronize()
    return host(y), ws


def test_a2a_tiny_int_every_order(fo, orc):
    P = 4
    pieces, w = case(256, 512, 512, P, "int", 17001)
    ref = orc.a2a_gemm(pieces, w)
    flags = torch.full((P,), 1 << 30, dtype=torch.int32, device="cuda")
    for order in itertools.permutations(range(P)):
        for local in (0, 3):
            y, ws = run(fo, pieces, w, P, order=list(order), local=local, arrived=flags)
            check_exact(y, ref, f"order {order} local {local}")
            assert int(ws.sum()) == 0, "counters not returned to zero"
    y, _ = run(fo, pieces, w, P, y_dtype=torch.bfloat16)
    assert np.array_equal(y, orc.f64_to_bf16(ref)), "bf16 out"


@pytest.mark.parametrize("m,k,n,P", [(200, 360, 264, 3), (64, 40, 40, 5), (130, 64, 520, 1),
                                     (300, 576, 300, 4), (129, 1024, 257, 8)])
def test_a2a_ragged(fo, orc, m, k, n, P):
    """Partial row and column tiles, pieces narrower than one 64-wide stage or
    ending inside one, odd n (scalar stores)."""
    log(f"case: a2a ragged {m}x{n}x{k} P={P}")
    for mode in ("int", "gauss"):
        pieces, w = case(m, k, n, P, mode, 17100 + m + k)
        ref = orc.a2a_gemm(pieces, w)
        y, _ = run(fo, pieces, w, P, local=P // 2)
        if mode == "int":
            check_exact(y, ref, "int")
        else:
            check_tolerance(y, ref, what="gauss")
    y, _ = run(fo, pieces, w, P, y_dtype=torch.bfloat16)
    got = bf16_bits_to_f64(y)
    check_tolerance(got, ref, frob_ref=bf16_bits_to_f64(orc.f64_to_bf16(ref)), what="gauss bf16")


@pytest.mark.parametrize("grid", [8, 100, 0])
def test_a2a_grids_and_determinism(fo, orc, grid):
    pieces, w = case(1024, 2048, 1024, 8, "gauss", 17200)
    ref = orc.a2a_gemm(pieces, w)
    y1, _ = run(fo, pieces, w, 8, max_workgroups=grid)
    y2, _ = run(fo, pieces, w, 8, max_workgroups=grid)
    assert np.array_equal(y1, y2), "not run-to-run identical"
    check_tolerance(y1, ref, what=f"grid {grid}")
    pieces, w = case(1024, 2048, 1024, 8, "int", 17201)
    y, _ = run(fo, pieces, w, 8, max_workgroups=grid)
    check_exact(y, orc.a2a_gemm(pieces, w), f"int grid {grid}")


def a2a_emulated(fo, pieces_b, wb, P, local, arrival, release_ns, order=None, reps=1, gated=True):
    """fo_a2a_gemm with the peers' pieces copied by SDMA at release_ns[i]
    (piece arrival[i]) into inboxes filled with NaN first."""
    m, kp = pieces_b[0].shape
    n = wb.shape[0]
    staging = [dev_bf16(p) for p in pieces_b]
    inbox = [s.clone() for s in staging]
    w = dev_bf16(wb)
    flags = torch.zeros(P, dtype=torch.int32, device="cuda")
    es = torch.zeros(P + 2, dtype=torch.int64, device="cuda")
    gs = torch.zeros(2 * P + 2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    side = side_stream()
    outs = []
    for _ in range(reps):
        e = epoch()
        for q in arrival:
            inbox[q].fill_(float("nan"))
        y = torch.full((m, n), float("nan"), device="cuda")
        gs.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            fo.fo_emulate_arrivals([inbox[q] for q in arrival], [staging[q] for q in arrival],
                                   [int(t) for t in release_ns], arrival, flags, e, es, stream=side,
                                   gate=gs[2 * P:2 * P + 1] if gated else None)
        fo.fo_a2a_gemm(inbox, w, y, fo.Schedule(nchunks=P, local=local, order=order, arrived=flags, epoch=e,
                                                stamps=gs, status=status, timeout_ns=5_000_000_000), ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "flag wait timed out"
        assert int(ws.sum()) == 0
        st = host(gs).astype(np.int64)
        last = max(host(es).astype(np.int64)[1 + q] for q in arrival)
        assert st[2 * P + 1] >= last, "output completed before the last landing"
        outs.append(host(y))
    return outs


@pytest.mark.parametrize("local", [0, 5])
def test_a2a_emulated_pairwise_and_out_of_order(fo, orc, local):
    P = 8
    pieces, w = case(1024, 2048, 768, P, "int", 17300 + local)
    ref = orc.a2a_gemm(pieces, w)
    pairwise = [(local - s) % P for s in range(1, P)]
    log(f"case: a2a emulated pairwise arrivals, local {local}")
    for y in a2a_emulated(fo, pieces, w, P, local, pairwise, [10_000 * (i + 1) for i in range(P - 1)], reps=2):
        check_exact(y, ref, "pairwise")
    shuffled = wl.seeded_permutation(pairwise, 31 + local)
    log(f"case: a2a emulated out-of-order arrivals {shuffled}")
    (y,) = a2a_emulated(fo, pieces, w, P, local, shuffled, [8_000 * (i + 1) for i in range(P - 1)])
    check_exact(y, ref, "out of order")
    order = [local] + shuffled       # accumulation in landing order
    (y,) = a2a_emulated(fo, pieces, w, P, local, shuffled, [8_000 * (i + 1) for i in range(P - 1)], order=order)
    check_exact(y, ref, "landing order")


def test_a2a_timeout_from_unset_flag(fo):
    P = 4
    pieces, w = case(256, 512, 512, P, "int", 17400)
    flags = torch.zeros(P, dtype=torch.int32, device="cuda")
    e = epoch()
    flags.fill_(e)
    flags[2] = 0
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    y = torch.zeros((256, 512), device="cuda")
    dp = [dev_bf16(p) for p in pieces]
    dw = dev_bf16(w)
    fo.fo_a2a_gemm(dp, dw, y, fo.Schedule(nchunks=P, epoch=e, arrived=flags, status=status,
                                          timeout_ns=2_000_000), ws)
    torch.cuda.synchronize()
    assert int(status.item()) == fo.FO_ERR_TIMEOUT
    assert int(ws.sum()) == 0
    flags.fill_(epoch())
    fo.fo_a2a_gemm(dp, dw, y, fo.Schedule(nchunks=P, epoch=_EP[0], arrived=flags), ws)
    torch.cuda.synchronize()


def test_a2a_ulysses_full_size(fo, orc):
    """The Ulysses workload: int unsampled (all present and with emulated
    50 GB/s pairwise arrivals), Gaussian within the bar on sampled rows."""
    c = wl.CFG6
    pieces, w = wl.a2a_pieces(c, "int")
    log(f"oracle: ulysses a2a int {c.m}x{c.n}x{c.k} P={c.R}")
    ref = orc.a2a_gemm(pieces, w)
    y, _ = run(fo, pieces, w, c.R)
    check_exact(y, ref, "ulysses int")
    pairwise = [(c.local - s) % c.R for s in range(1, c.R)]
    rel = wl.ring_release_ns(c.m * (c.k // c.R) * 2, c.R - 1)
    log("case: ulysses int, emulated 50 GB/s pairwise arrivals")
    (y,) = a2a_emulated(fo, pieces, w, c.R, c.local, pairwise, rel)
    check_exact(y, ref, "ulysses emulated")
    pieces, w = wl.a2a_pieces(c, "gauss")
    y, _ = run(fo, pieces, w, c.R)
    rows = np.unique(np.concatenate([np.arange(0, c.m, 29), [c.m - 1]]))
    check_tolerance(y[rows], orc.a2a_gemm([p[rows] for p in pieces], w), what="ulysses gauss")
