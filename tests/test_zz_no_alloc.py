"""fo_ag_gemm_noalloc, the AG-GEMM entry point that allocates nothing (its
workspace is the library's per-GPU scratch array), against fo_ag_gemm with a
caller workspace: the same bits on two calls in a row, the second on a
smaller problem, through the C ABI."""
import numpy as np
import pytest

import workloads as wl
from helpers import check_exact, dev_bf16, host, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fo():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sp_rank_adaptive_amd as fo
    fo.lib()
    return fo


def both(fo, xb, wb, R, epoch, **kw):
    """(noalloc output, fo_ag_gemm output) on the same inputs and schedule."""
    m, k = xb.shape
    n = wb.shape[0]
    x, w = dev_bf16(xb), dev_bf16(wb)
    flags = torch.full((R,), epoch + 1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    y0 = torch.full((m, n), float("nan"), device="cuda")
    fo.fo_ag_gemm_noalloc(x, w, y0, fo.Schedule(nchunks=R, epoch=epoch, arrived=flags, status=status,
                                                timeout_ns=2_000_000_000, **kw))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    y1 = torch.full((m, n), float("nan"), device="cuda")
    fo.fo_ag_gemm(x, w, y1, fo.Schedule(nchunks=R, epoch=epoch + 1, arrived=flags, **kw), ws)
    torch.cuda.synchronize()
    return host(y0), host(y1)


def test_noalloc_matches_workspace_entry_point(fo, orc):
    # 1st call: TP=8 MLP up-projection share with preset flags and the
    # automatic split of the last peer (its split partials use the scratch)
    c = wl.CFG2
    for mode in ("int", "gauss"):
        xb, wb = wl.gemm_inputs(c, mode)
        log(f"case: noalloc {c.m}x{c.n}x{c.k} R={c.R} {mode}, automatic split")
        y0, y1 = both(fo, xb, wb, c.R, 100 + (mode == "gauss") * 10)
        assert np.array_equal(y0, y1), f"noalloc differs from fo_ag_gemm ({mode})"
        if mode == "int":
            rows = np.arange(0, c.m, 7)
            check_exact(y0[rows], orc.gemm(xb[rows], wb), "noalloc int")
    # 2nd call: a smaller, ragged problem with another split vector, on the
    # scratch the first call left behind
    m, n, k, R = 600, 264, 1000, 4
    xb = wl.bf16_operand((m, k), "int", 1.0, 16001)
    wb = wl.bf16_operand((n, k), "int", 1.0, 16002)
    log(f"case: noalloc {m}x{n}x{k} R={R} split [1, 3, 1, 2]")
    y0, y1 = both(fo, xb, wb, R, 200, split=[1, 3, 1, 2])
    assert np.array_equal(y0, y1), "noalloc differs from fo_ag_gemm (small)"
    check_exact(y0, orc.gemm(xb, wb), "noalloc small int")


def test_noalloc_refuses_problems_beyond_scratch(fo):
    m, n, k, R = 65536, 8192, 4096, 8       # workspace bound far above 64 MiB
    assert fo.fo_workspace_bytes(m, n, k, R) > fo.FO_NOALLOC_SCRATCH_BYTES
    x = torch.empty((8, 8), dtype=torch.bfloat16, device="cuda")   # never read
    st = fo.lib().fo_ag_gemm_noalloc(x.data_ptr(), x.data_ptr() + 4096, x.data_ptr() + 8192, fo.FO_F32,
                                     m, n, k, None, None)
    assert st == fo.FO_ERR_NULL                 # no schedule
    s, keep = fo.Schedule(nchunks=R, epoch=1)._c()
    import ctypes
    st = fo.lib().fo_ag_gemm_noalloc(x.data_ptr(), x.data_ptr() + 4096, x.data_ptr() + 8192, fo.FO_F32,
                                     m, n, k, ctypes.byref(s), None)
    assert st == fo.FO_ERR_WORKSPACE
