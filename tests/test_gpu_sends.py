"""The send side of the decomposed reduce-scatter, emulated on one GPU: each
peer-destined partial chunk is copied by SDMA to its peer's inbox once the
GEMM-RS launch has released that chunk's done flag (fo_emulate_sends on a
side stream, enqueued before the launch).  Checked: every send starts after
its chunk's completion stamp and after its flag, the copied bytes equal the
oracle's partial exactly (integer inputs), and a send waits for the flag
(a flag that is never released times out without blocking the stream)."""
import numpy as np
import pytest

import workloads as wl
from helpers import check_exact, dev_bf16, host, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_SIDE = []


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


@pytest.mark.parametrize("form", ["gemm_rs", "fused"])
def test_sends_after_done_flags_int_exact(fo, orc, form):
    m, n, k, R, local = 1024, 512, 512, 8, 0
    xb = wl.bf16_operand((m, k), "int", 1.0, 19001)
    wb = wl.bf16_operand((n, k), "int", 1.0, 19002)
    ref = orc.gemm(xb, wb)
    x, w = dev_bf16(xb), dev_bf16(wb)
    mc = m // R
    part = torch.full((m, n), float("nan"), device="cuda")
    done = torch.zeros(R, dtype=torch.int32, device="cuda")
    gs = torch.zeros(2 * R + 2, dtype=torch.int64, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    peers = [(local - s) % R for s in range(1, R)]          # send order
    inbox = [torch.full((mc, n), float("nan"), device="cuda") for _ in peers]
    st = torch.zeros(2 * len(peers), dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    shard = torch.empty((mc, n), device="cuda")
    inc = [None if q == local else torch.zeros((mc, n), device="cuda") for q in range(R)]
    for rep in range(2):
        e = 100 + rep
        torch.cuda.synchronize()
        side = side_stream()
        with torch.cuda.stream(side):
            fo.fo_emulate_sends(done, e, inbox, [part[q * mc:(q + 1) * mc] for q in peers], peers,
                                [5_000] * len(peers), st, timeout_ns=5_000_000_000, status=status, stream=side)
        log(f"case: {form} with emulated sends, rep {rep}")
        if form == "fused":
            fo.fo_gemm_rs_reduce(x, w, part, done, shard, inc, fo.Schedule(nchunks=R, local=local, epoch=e,
                                                                          stamps=gs), ws)
        else:
            fo.fo_gemm_rs(x, w, part, done, fo.Schedule(nchunks=R, local=local, epoch=e, stamps=gs), ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a send waited out its timeout"
        g = host(gs).astype(np.int64)
        t = host(st).astype(np.int64)
        for i, q in enumerate(peers):
            assert t[2 * i] >= g[R + q], f"send of chunk {q} started before the chunk was complete"
            assert t[2 * i + 1] >= t[2 * i]
            check_exact(host(inbox[i]), ref[q * mc:(q + 1) * mc], f"sent partial of chunk {q}")
        assert all(t[2 * i + 2] >= t[2 * i + 1] for i in range(len(peers) - 1)), "sends overlapped on one link"


def test_send_waits_for_its_flag(fo):
    """A flag that is never released: the wait times out (status set), the
    stream moves on, and the other sends are unaffected."""
    done = torch.zeros(4, dtype=torch.int32, device="cuda")
    done[1] = 7
    done[3] = 7
    src = torch.arange(1024, dtype=torch.float32, device="cuda")
    dst = [torch.zeros(1024, device="cuda") for _ in range(3)]
    st = torch.zeros(6, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    fo.fo_emulate_sends(done, 7, dst, [src] * 3, [1, 2, 3], [1_000] * 3, st, timeout_ns=2_000_000, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == fo.FO_ERR_TIMEOUT
    for d in dst:
        assert torch.equal(d, src)
