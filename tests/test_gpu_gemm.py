"""GPU parity of fo_ag_gemm / fo_gemm_rs against the fp64 oracle, through the C ABI."""
import itertools

import numpy as np
import pytest

import workloads as wl
from helpers import (bf16_bits_to_f64, check_exact, check_tolerance, dev_bf16, dev_f32, host,
                     log)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fo():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sp_rank_adaptive_amd as fo
    fo.lib()
    return fo


class Epochs:
    def __init__(self):
        self.e = 0

    def next(self):
        self.e += 1
        return self.e


EP = Epochs()


def workspace(fo, m, n, k, R):
    nb = fo.fo_workspace_bytes(m, n, k, R)
    assert nb > 0
    return torch.zeros(nb, dtype=torch.uint8, device="cuda")


def run_ag(fo, x, w, R, y_dtype=torch.float32, ws=None, **sched):
    m, k = x.shape
    n = w.shape[0]
    y = torch.full((m, n), float("nan"), dtype=y_dtype, device="cuda")
    if ws is None:
        ws = workspace(fo, m, n, k, R)
    s = fo.Schedule(nchunks=R, epoch=EP.next(), **sched)
    fo.fo_ag_gemm(x, w, y, s, ws)
    torch.cuda.synchronize()
    return y, ws


def gemm_case(cfg, mode, m=None):
    xb, wb = wl.gemm_inputs(cfg, mode, m=m)
    return xb, wb, dev_bf16(xb), dev_bf16(wb)


def test_ag_gemm_tiny_int_bitexact_all_orders(fo, orc):
    c = wl.CFG1
    log(f"case: cfg1 int {c.m}x{c.n}x{c.k} R={c.R}")
    xb, wb, x, w = gemm_case(c, "int")
    ref = orc.gemm(xb, wb)
    for order in itertools.permutations(range(c.R)):
        for mode in (fo.FO_SCHED_READY_FIRST, fo.FO_SCHED_STRICT):
            y, ws = run_ag(fo, x, w, c.R, order=list(order), mode=mode)
            check_exact(host(y), ref, f"order {order} mode {mode}")
            assert int(ws[:4096].sum()) == 0, "workspace not returned to zero"


@pytest.mark.parametrize("local", [0, 1, 2, 3])
def test_ag_gemm_tiny_every_local_rank(fo, orc, local):
    c = wl.CFG1
    xb, wb, x, w = gemm_case(c, "int")
    y, _ = run_ag(fo, x, w, c.R, local=local)
    check_exact(host(y), orc.gemm(xb, wb), f"local {local}")


@pytest.mark.parametrize("m,n,k,R", [(210, 200, 136, 3), (64, 40, 8, 1), (520, 136, 200, 5),
                                     (128, 128, 64, 2), (1024, 96, 1032, 4)])
def test_ag_gemm_ragged_shapes(fo, orc, m, n, k, R):
    log(f"case: ragged {m}x{n}x{k} R={R}")
    for mode in ("int", "gauss"):
        xb = wl.bf16_operand((m, k), mode, 1.0, 900 + m)
        wb = wl.bf16_operand((n, k), mode, 0.02 if mode == "gauss" else 1.0, 901 + n)
        ref = orc.gemm(xb, wb)
        y, _ = run_ag(fo, dev_bf16(xb), dev_bf16(wb), R)
        if mode == "int":
            check_exact(host(y), ref, "int")
        else:
            check_tolerance(host(y), ref, what="gauss")


# every compiled tile layout (FO_TILE=BMxBN picks one)
TILES = ["256x256", "256x160", "128x224", "128x128"]


@pytest.mark.parametrize("tile", TILES)
def test_every_tile_layout_ragged_int_exact(fo, orc, tile, monkeypatch):
    """Each layout on ragged shapes (partial row/column tiles, k not a
    multiple of the stage depth, odd n for the scalar store path, one and
    two k stages), unsplit and split, AG and GEMM-RS, fp32 and bf16 out."""
    monkeypatch.setenv("FO_TILE", tile)
    R = 2
    for m, n, k in [(600, 522, 200), (520, 264, 8), (520, 264, 40), (1040, 520, 1000)]:
        log(f"case: tile {tile} {m}x{n}x{k} R={R}")
        xb = wl.bf16_operand((m, k), "int", 1.0, 1200 + k)
        wb = wl.bf16_operand((n, k), "int", 1.0, 1201 + n)
        ref = orc.gemm(xb, wb)
        x, w = dev_bf16(xb), dev_bf16(wb)
        ws = torch.zeros(4 * fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
        for split in (None, [3, 1], [1, 2]):
            kw = {} if split is None else {"split": split}
            y, _ = run_ag(fo, x, w, R, ws=ws, **kw)
            check_exact(host(y), ref, f"{tile} {m}x{n}x{k} split {split}")
        part = torch.full((m, n), float("nan"), device="cuda")
        done = torch.zeros(R, dtype=torch.int32, device="cuda")
        e = EP.next()
        fo.fo_gemm_rs(x, w, part, done, fo.Schedule(nchunks=R, epoch=e), ws)
        torch.cuda.synchronize()
        assert (host(done) == e).all()
        check_exact(host(part), ref, f"{tile} {m}x{n}x{k} gemm_rs")
        y, _ = run_ag(fo, x, w, R, y_dtype=torch.bfloat16, ws=ws)
        assert np.array_equal(host(y), orc.f64_to_bf16(ref)), f"{tile} bf16 out"


def test_ag_gemm_bf16_output(fo, orc):
    c = wl.CFG1
    xb, wb, x, w = gemm_case(c, "gauss")
    ref = orc.gemm(xb, wb)
    y, _ = run_ag(fo, x, w, c.R, y_dtype=torch.bfloat16)
    got = bf16_bits_to_f64(host(y))
    check_tolerance(got, ref, frob_ref=bf16_bits_to_f64(orc.f64_to_bf16(ref)), what="bf16 out")
    # integer inputs: the fp32 sums are exact, so the bf16 result is RNE of the exact value
    xb, wb, x, w = gemm_case(c, "int")
    ref = orc.gemm(xb, wb)
    y, _ = run_ag(fo, x, w, c.R, y_dtype=torch.bfloat16)
    assert np.array_equal(host(y), orc.f64_to_bf16(ref))


def test_ag_gemm_split_k_exact_and_deterministic(fo, orc):
    m, n, k, R = 512, 256, 1024, 4
    xb = wl.bf16_operand((m, k), "int", 1.0, 950)
    wb = wl.bf16_operand((n, k), "int", 1.0, 951)
    ref = orc.gemm(xb, wb)
    x, w = dev_bf16(xb), dev_bf16(wb)
    # every chunk split 8-way needs more than the default partial-tile area
    nb = fo.fo_workspace_bytes(m, n, k, R)
    with pytest.raises(fo.FoError, match="workspace"):
        run_ag(fo, x, w, R, split=[8, 8, 8, 8])
    big = torch.zeros(4 * nb, dtype=torch.uint8, device="cuda")
    for split in ([1, 4, 1, 2], [8, 8, 8, 8], [3, 1, 5, 1], [4, 4, 1, 1]):
        y, ws = run_ag(fo, x, w, R, split=split, ws=big if split == [8, 8, 8, 8] else None)
        check_exact(host(y), ref, f"split {split}")
        assert int(ws[:4096].sum()) == 0, "counters not returned to zero"
        # a stale tile counter would pick the wrong split to write the tile
        y, _ = run_ag(fo, x, w, R, split=split, ws=ws)
        check_exact(host(y), ref, f"split {split}, reused workspace")
    xb = wl.bf16_operand((m, k), "gauss", 1.0, 952)
    wb = wl.bf16_operand((n, k), "gauss", 0.02, 953)
    ref = orc.gemm(xb, wb)
    x, w = dev_bf16(xb), dev_bf16(wb)
    y1, _ = run_ag(fo, x, w, R, split=[1, 4, 1, 2])
    y2, _ = run_ag(fo, x, w, R, split=[1, 4, 1, 2])
    assert torch.equal(y1, y2), "split-K result not run-to-run deterministic"
    check_tolerance(host(y1), ref, what="split gauss")
    # unsplit chunks are bitwise identical whatever the other chunks' splits
    y3, _ = run_ag(fo, x, w, R)
    assert torch.equal(y1[0:128], y3[0:128]) and torch.equal(y1[256:384], y3[256:384])


@pytest.mark.parametrize("R,split,grid", [
    (1, [4], 0), (1, [8], 0), (1, [4], 32), (1, [4], 40), (1, [8], 72),
    (4, [1, 4, 1, 8], 0), (4, [1, 4, 1, 8], 96),
    (1, [2], 0), (4, [1, 4, 1, 2], 56),
])
def test_split_units_reduce_own_slices_int_exact(fo, orc, R, split, grid):
    # With every split at least 4 and at least 8 x (sum of the splits)
    # workgroups, each split unit sums its own row slices of its tile once
    # the tile's splits are all written (no reduce units): static first
    # claims, static round-robin with tiles that span two rounds (grid 40: 5
    # workgroups per XCD, split 4) and dynamic claims over preset flags.  A
    # split of 2 goes through reduce units.  Every element is written once
    # and equals the oracle; the counters return to zero; two runs agree
    # bitwise.
    mc, n, k = 512, 1792, 1024
    m = mc * R
    xb = wl.bf16_operand((m, k), "int", 0.0, 12101 + R)
    wb = wl.bf16_operand((n, k), "int", 0.0, 12102)
    x, w = dev_bf16(xb), dev_bf16(wb)
    ref = orc.gemm(xb, wb)
    log(f"case: self-reduce {m}x{n}x{k} R={R} split={split} grid={grid}")
    # several split chunks need more than the default partial-tile area
    big = torch.zeros(4 * fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    y, ws = run_ag(fo, x, w, R, ws=big, split=split, max_workgroups=grid)
    assert not torch.isnan(y).any()
    check_exact(host(y), ref, f"split {split} grid {grid}")
    assert int(ws[:4096].sum()) == 0, "counters not returned to zero"
    flags = torch.full((R,), EP.e + 1, dtype=torch.int32, device="cuda")
    y2, _ = run_ag(fo, x, w, R, ws=ws, split=split, max_workgroups=grid, arrived=flags)
    assert not torch.isnan(y2).any()
    check_exact(host(y2), ref, f"preset flags, split {split} grid {grid}")
    assert int(ws[:4096].sum()) == 0, "counters not returned to zero (flags)"
    xg = wl.bf16_operand((m, k), "gauss", 1.0, 12111)
    wg = wl.bf16_operand((n, k), "gauss", 0.02, 12112)
    xd, wd = dev_bf16(xg), dev_bf16(wg)
    g1, _ = run_ag(fo, xd, wd, R, ws=ws, split=split, max_workgroups=grid)
    g2, _ = run_ag(fo, xd, wd, R, ws=ws, split=split, max_workgroups=grid)
    assert torch.equal(g1, g2), "self-reduced split-K not run-to-run deterministic"
    check_tolerance(host(g1), orc.gemm(xg, wg), what=f"gauss split {split}")


def test_ag_gemm_preset_flags_and_epoch_reuse(fo, orc):
    c = wl.CFG1
    xb, wb, x, w = gemm_case(c, "int")
    ref = orc.gemm(xb, wb)
    flags = torch.zeros(c.R, dtype=torch.int32, device="cuda")
    ws = workspace(fo, c.m, c.n, c.k, c.R)
    stamps = torch.zeros(2 * c.R + 2, dtype=torch.int64, device="cuda")
    for _ in range(3):      # flags are never reset: each call raises the epoch
        e = EP.next()
        flags.fill_(e)
        y = torch.full((c.m, c.n), float("nan"), device="cuda")
        s = fo.Schedule(nchunks=c.R, epoch=e, arrived=flags, stamps=stamps)
        fo.fo_ag_gemm(x, w, y, s, ws)
        torch.cuda.synchronize()
        check_exact(host(y), ref, "preset flags")
        assert int(ws[:4096].sum()) == 0
        st = host(stamps).astype(np.int64)
        assert st[2 * c.R + 1] >= st[2 * c.R] > 0


def test_ag_gemm_timeout_from_unset_flag(fo):
    """A flag the host never sets: the bounded wait ends with FO_ERR_TIMEOUT and
    the kernel exits; the workspace is clean afterwards."""
    c = wl.CFG1
    xb, wb, x, w = gemm_case(c, "int")
    flags = torch.zeros(c.R, dtype=torch.int32, device="cuda")
    e = EP.next()
    flags.fill_(e)
    flags[2] = 0                        # chunk 2 never lands
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = workspace(fo, c.m, c.n, c.k, c.R)
    y = torch.zeros((c.m, c.n), device="cuda")
    s = fo.Schedule(nchunks=c.R, epoch=e, arrived=flags, status=status, timeout_ns=2_000_000)
    fo.fo_ag_gemm(x, w, y, s, ws)
    torch.cuda.synchronize()
    assert int(status.item()) == fo.FO_ERR_TIMEOUT
    assert int(ws[:4096].sum()) == 0
    # the next call on the same workspace works
    flags.fill_(EP.next())
    s = fo.Schedule(nchunks=c.R, epoch=EP.e, arrived=flags)
    fo.fo_ag_gemm(x, w, y, s, ws)
    torch.cuda.synchronize()


def test_ag_gemm_full_size_sampled_rows(fo, orc):
    for cfg in (wl.CFG2, wl.CFG5):
        log(f"case: cfg{cfg.cfg} gauss {cfg.m}x{cfg.n}x{cfg.k} R={cfg.R}")
        xb, wb, x, w = gemm_case(cfg, "gauss")
        y, _ = run_ag(fo, x, w, cfg.R)
        assert not torch.isnan(y).any()   # every tile written (y starts as NaN)
        rows = np.sort(np.random.Generator(np.random.PCG64(7 + cfg.cfg)).choice(cfg.m, 48, replace=False))
        mc = cfg.m // cfg.R
        rows = np.unique(np.concatenate([rows, [0, mc - 1, mc, cfg.m - 1]]))
        ref = orc.gemm(xb[rows], wb)
        check_tolerance(host(y)[rows], ref, what=f"cfg{cfg.cfg}")


@pytest.mark.parametrize("grid", [8, 12, 96, 100, 256])
def test_claim_paths_cover_every_unit_int_exact(fo, orc, grid):
    # Static round-robin (no flags, 8 | grid, balanced groups), the static
    # first claim followed by dynamic claims (grid not a multiple of 8), and
    # dynamic claims over preset flags: every output element is written once
    # (the output starts as NaN) and equals the oracle exactly.
    m, n, k, R = 1024, 448, 512, 4
    xb = wl.bf16_operand((m, k), "int", 0.0, 12001)
    wb = wl.bf16_operand((n, k), "int", 0.0, 12002)
    x, w = dev_bf16(xb), dev_bf16(wb)
    ref = orc.gemm(xb, wb)
    log(f"case: claim paths {m}x{n}x{k} R={R} grid={grid}")
    y, ws = run_ag(fo, x, w, R, max_workgroups=grid)
    assert not torch.isnan(y).any()
    check_exact(host(y), ref, f"no flags, grid {grid}")
    flags = torch.full((R,), EP.e + 1, dtype=torch.int32, device="cuda")
    y2, _ = run_ag(fo, x, w, R, ws=ws, max_workgroups=grid, arrived=flags)
    assert not torch.isnan(y2).any()
    check_exact(host(y2), ref, f"preset flags, grid {grid}")


def test_ag_gemm_full_size_int_sampled_rows(fo, orc):
    cfg = wl.CFG2
    xb, wb, x, w = gemm_case(cfg, "int")
    y, _ = run_ag(fo, x, w, cfg.R, arrived=None)
    rows = np.arange(0, cfg.m, 97)
    check_exact(host(y)[rows], orc.gemm(xb[rows], wb), "cfg2 int")


def test_gemm_rs_parity_done_flags_and_order(fo, orc):
    cfg = wl.CFG3
    for mode in ("int", "gauss"):
        log(f"case: cfg3 gemm_rs {mode}")
        xb, wb, x, w = gemm_case(cfg, mode)
        part = torch.full((cfg.m, cfg.n), float("nan"), device="cuda")
        done = torch.zeros(cfg.R, dtype=torch.int32, device="cuda")
        stamps = torch.zeros(2 * cfg.R + 2, dtype=torch.int64, device="cuda")
        ws = workspace(fo, cfg.m, cfg.n, cfg.k, cfg.R)
        e = EP.next()
        s = fo.Schedule(nchunks=cfg.R, epoch=e, stamps=stamps)
        fo.fo_gemm_rs(x, w, part, done, s, ws)
        torch.cuda.synchronize()
        assert (host(done) == e).all()
        rows = np.unique(np.concatenate([np.arange(0, cfg.m, 131), [cfg.m - 1]]))
        ref = orc.gemm(xb[rows], wb)
        if mode == "int":
            check_exact(host(part)[rows], ref, "rs int")
        else:
            check_tolerance(host(part)[rows], ref, what="rs gauss")
    # Claim order: with fewer workgroups than units the units are taken in
    # rounds, in priority order (peers in send order, local last).  64
    # workgroups are 8 per XCD and each chunk holds 4 units per XCD group, so
    # a round covers two chunks and the local chunk (0) shares the last round
    # with chunk 1: it starts no earlier than every chunk of the earlier
    # rounds.  (With one unit per workgroup every chunk starts at once.)
    part = torch.full((cfg.m, cfg.n), float("nan"), device="cuda")
    stamps = torch.zeros(2 * cfg.R + 2, dtype=torch.int64, device="cuda")
    e = EP.next()
    fo.fo_gemm_rs(x, w, part, done, fo.Schedule(nchunks=cfg.R, epoch=e, stamps=stamps, max_workgroups=64), ws)
    torch.cuda.synchronize()
    assert (host(done) == e).all()
    check_tolerance(host(part)[rows], ref, what="rs gauss, 64 workgroups")
    first = host(stamps).astype(np.int64)[:cfg.R]
    assert first[0] >= first[2:].max()


def test_workspace_size_covers_padded_tiles(fo, orc):
    """m = 2048, R = 8, n = 2560, k = 8192 with arrival flags: the automatic
    split (8 ways, 128 x 224 tiles, n padded to 2688) needs more partial area
    than a 256-wide tile's padding; fo_workspace_bytes must cover it."""
    m, n, k, R = 2048, 2560, 8192, 8
    xb = wl.bf16_operand((m, k), "int", 1.0, 14001)
    wb = wl.bf16_operand((n, k), "int", 1.0, 14002)
    x, w = dev_bf16(xb), dev_bf16(wb)
    flags = torch.full((R,), EP.e + 1, dtype=torch.int32, device="cuda")
    log(f"case: workspace sizing {m}x{n}x{k} R={R}, automatic split")
    y, ws = run_ag(fo, x, w, R, arrived=flags)
    assert ws.numel() == fo.fo_workspace_bytes(m, n, k, R)
    check_exact(host(y), orc.gemm(xb, wb), "padded split tiles")


def test_grid_request_above_cus_is_capped(fo, orc):
    """A max_workgroups request above one per CU acts as the cap: a split
    chunk without flags (reduce units waiting for split tiles held by other
    workgroups) still completes, exactly."""
    cus, _, _ = fo.fo_device_info()
    m, n, k, R = 1024, 448, 2048, 4
    xb = wl.bf16_operand((m, k), "int", 1.0, 14101)
    wb = wl.bf16_operand((n, k), "int", 1.0, 14102)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    log(f"case: max_workgroups {4 * cus} on {cus} CUs, split [8, 8, 1, 2]")
    ws = torch.zeros(4 * fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    y, _ = run_ag(fo, dev_bf16(xb), dev_bf16(wb), R, ws=ws, split=[8, 8, 1, 2], max_workgroups=4 * cus,
                  status=status, timeout_ns=2_000_000_000)
    assert int(status.item()) == 0
    check_exact(host(y), orc.gemm(xb, wb), "capped grid")


@pytest.mark.parametrize("R", [24, 64])
@pytest.mark.parametrize("grid", [8, 100, 256])
def test_claim_walk_many_chunks_preset_flags(fo, orc, R, grid):
    """R = 24 and 64 chunks with arrival flags: the claim walk reads three and
    eight 64-lane batches of (position, XCD group) counters; a priority order
    that is a seeded permutation, the automatic split of its last peer, and
    every element written once and exact."""
    mc, n, k = 64, 264, 2048
    m = R * mc
    xb = wl.bf16_operand((m, k), "int", 1.0, 15000 + R)
    wb = wl.bf16_operand((n, k), "int", 1.0, 15001)
    x, w = dev_bf16(xb), dev_bf16(wb)
    ref = orc.gemm(xb, wb)
    order = wl.seeded_permutation(list(range(R)), R + grid)
    local = order[-1]
    flags = torch.full((R,), EP.e + 1, dtype=torch.int32, device="cuda")
    log(f"case: R={R} grid={grid} preset flags, order {order[:4]}..., local {local}")
    y, ws = run_ag(fo, x, w, R, arrived=flags, order=order, local=local, max_workgroups=grid)
    assert not torch.isnan(y).any()
    check_exact(host(y), ref, f"R={R} grid={grid}")
    assert int(ws[:4096].sum()) == 0
    y, _ = run_ag(fo, x, w, R, ws=ws, arrived=torch.full((R,), EP.e + 1, dtype=torch.int32, device="cuda"),
                  order=order, local=local, max_workgroups=grid, mode=fo.FO_SCHED_STRICT)
    check_exact(host(y), ref, f"R={R} grid={grid} strict")
