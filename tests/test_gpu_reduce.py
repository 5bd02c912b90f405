"""GPU parity of fo_chunk_reduce against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import workloads as wl
from helpers import bf16_bits_to_f64, check_exact, check_tolerance, dev_f32, host, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_EPOCH = [1000]


def next_epoch():
    _EPOCH[0] += 1
    return _EPOCH[0]


@pytest.fixture(scope="module")
def fo():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sp_rank_adaptive_amd as fo
    fo.lib()
    return fo


def reduce_case(R, n, mode, seed, std=1e-3, int_range=1 << 20):
    g = np.random.Generator(np.random.PCG64(seed))
    if mode == "int":
        return [g.integers(-int_range, int_range + 1, n).astype(np.float32) for _ in range(R)]
    return [(g.standard_normal(n, dtype=np.float32) * np.float32(std)) for _ in range(R)]


@pytest.mark.parametrize("R,n", [(1, 4096), (2, 1024), (3, 4100), (8, 1 << 21), (16, 12348)])
def test_reduce_fp32_parity(fo, orc, R, n):
    log(f"case: reduce fp32 R={R} n={n}")
    for mode in ("int", "gauss"):
        srcs = reduce_case(R, n, mode, 1000 + R + n)
        ref = orc.reduce(srcs)
        d = [dev_f32(s) for s in srcs]
        dst = torch.full((n,), float("nan"), device="cuda")
        s = fo.Schedule(nchunks=R, local=R // 2, epoch=next_epoch())
        fo.fo_chunk_reduce(dst, d, s)
        torch.cuda.synchronize()
        if mode == "int":
            check_exact(host(dst), ref, "int")
        else:
            check_tolerance(host(dst), ref, what="gauss")


def test_reduce_bf16_out_cfg3_shape(fo, orc):
    cfg = wl.CFG3
    n = cfg.m // cfg.R * cfg.n
    for mode in ("int", "gauss"):
        srcs = reduce_case(cfg.R, n, mode, 77, std=0.847, int_range=129024 // 8)
        ref = orc.reduce(srcs)
        d = [dev_f32(s) for s in srcs]
        dst = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        fo.fo_chunk_reduce(dst, d, fo.Schedule(nchunks=cfg.R, epoch=next_epoch()))
        torch.cuda.synchronize()
        got = host(dst)
        if mode == "int":
            assert np.array_equal(got, orc.f64_to_bf16(ref))
        else:
            check_tolerance(bf16_bits_to_f64(got), ref,
                            frob_ref=bf16_bits_to_f64(orc.f64_to_bf16(ref)), what="bf16")


def test_reduce_in_place_and_order_determinism(fo, orc):
    R, n = 8, 1 << 16
    srcs = reduce_case(R, n, "gauss", 91)
    ref = orc.reduce(srcs)
    order = [3, 1, 7, 0, 2, 6, 5, 4]
    outs = []
    for _ in range(2):
        d = [dev_f32(s) for s in srcs]
        fo.fo_chunk_reduce(d[0], d, fo.Schedule(nchunks=R, local=0, order=order, epoch=next_epoch()))
        torch.cuda.synchronize()
        outs.append(host(d[0]))
    assert np.array_equal(outs[0], outs[1])
    check_tolerance(outs[0], ref, what="in place")
    # the result is the left-to-right fp32 sum in the stated order
    acc = srcs[0].copy()
    for c in order:
        if c != 0:
            acc = (acc + srcs[c]).astype(np.float32)
    assert np.array_equal(outs[0], acc)


def test_reduce_preset_flags_and_timeout(fo, orc):
    R, n = 4, 1 << 14
    srcs = reduce_case(R, n, "int", 5)
    ref = orc.reduce(srcs)
    d = [dev_f32(s) for s in srcs]
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    e = next_epoch()
    flags.fill_(e)
    dst = torch.zeros(n, device="cuda")
    stamps = torch.zeros(2, dtype=torch.int64, device="cuda")
    fo.fo_chunk_reduce(dst, d, fo.Schedule(nchunks=R, epoch=e, arrived=flags, stamps=stamps))
    torch.cuda.synchronize()
    check_exact(host(dst), ref, "preset flags")
    st = host(stamps)
    assert st[1] >= st[0] > 0
    # a source the host never flags: bounded wait, FO_ERR_TIMEOUT
    e = next_epoch()
    flags.fill_(e)
    flags[3] = 0
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    fo.fo_chunk_reduce(dst, d, fo.Schedule(nchunks=R, epoch=e, arrived=flags, status=status,
                                           timeout_ns=2_000_000))
    torch.cuda.synchronize()
    assert int(status.item()) == fo.FO_ERR_TIMEOUT


def test_reduce_cfg4_full_size_sampled(fo, orc):
    cfg = wl.CFG4
    log("case: cfg4 full size")
    for mode in ("int", "gauss"):
        srcs = wl.reduce_sources(cfg, mode)
        idx = np.sort(np.random.Generator(np.random.PCG64(3)).choice(cfg.n, 1 << 16, replace=False))
        idx = np.unique(np.concatenate([idx, [0, cfg.n - 1]]))
        ref = orc.reduce([s[idx] for s in srcs])
        d = [dev_f32(s) for s in srcs]
        del srcs
        fo.fo_chunk_reduce(d[0], d, fo.Schedule(nchunks=cfg.R, epoch=next_epoch()))
        torch.cuda.synchronize()
        got = d[0][torch.from_numpy(idx).cuda()].cpu().numpy()
        if mode == "int":
            check_exact(got, ref, "cfg4 int")
        else:
            check_tolerance(got, ref, what="cfg4 gauss")
        del d
        torch.cuda.empty_cache()
