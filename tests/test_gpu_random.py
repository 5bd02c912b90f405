"""Seeded random parity cases for fo_ag_gemm and fo_gemm_rs: shapes, chunk
counts, local rank, priority order, STRICT or ready-first, preset flags,
per-chunk splits, workgroup caps, forced tile layouts and output types drawn
together, on integer inputs, every element bit-exact against the fp64 oracle."""
import os

import numpy as np
import pytest

import workloads as wl
from helpers import bf16_bits_to_f64, check_exact, check_tolerance, dev_bf16, host, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TILES = [None, "256x256", "256x160x3", "128x224", "128x128"]
# FO_RANDOM_SCALE multiplies the number of cases of every random test
# (default 1: a few seconds in all)
SCALE = int(os.environ.get("FO_RANDOM_SCALE", "1"))
SEEDS = list(range(48 * SCALE))


def seeds(n):
    return list(range(n * SCALE))


@pytest.fixture(scope="module")
def fo():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sp_rank_adaptive_amd as fo
    fo.lib()
    return fo


class _Epoch:
    e = 5000


def ws_bytes(fo, m, n, k, R, split):
    """fo_workspace_bytes covers the automatic split (one chunk split up to 8
    ways); an explicit vector needs partial slots for every split chunk."""
    extra = 0 if split is None else sum(s_ for s_ in split if s_ > 1) // 8
    return (2 + extra) * fo.fo_workspace_bytes(m, n, k, R)


def draw(seed: int) -> dict:
    g = np.random.Generator(np.random.PCG64(31337 + seed))
    R = int(g.choice([1, 2, 3, 4, 5, 8, 12]))
    mc = int(g.integers(1, 600 // R + 2)) * 8 if R > 4 else int(g.integers(8, 520))
    n = int(g.integers(8, 1100))
    k = int(g.choice([8, 64, 200, 520, 1024, 2000]))
    case = {
        "R": R, "m": R * mc, "n": n, "k": k,
        "local": int(g.integers(0, R)),
        "order": [int(v) for v in g.permutation(R)],
        "strict": bool(g.integers(0, 4) == 0),
        "flags": bool(g.integers(0, 2)),
        "split": [int(v) for v in g.choice([1, 1, 2, 3, 4, 8], size=R)] if g.integers(0, 2) else None,
        "grid": int(g.choice([0, 0, 1, 7, 40, 100, 300])),
        "tile": TILES[int(g.integers(0, len(TILES)))],
        "bf16": bool(g.integers(0, 3) == 0),
    }
    return case


@pytest.mark.parametrize("seed", SEEDS)
def test_random_ag_gemm_and_gemm_rs_int_exact(fo, orc, seed, monkeypatch):
    c = draw(seed)
    log(f"case: seed {seed} {c}")
    if c["tile"] is None:
        monkeypatch.delenv("FO_TILE", raising=False)
    else:
        monkeypatch.setenv("FO_TILE", c["tile"])
    m, n, k, R = c["m"], c["n"], c["k"], c["R"]
    xb = wl.bf16_operand((m, k), "int", 1.0, 17000 + 2 * seed)
    wb = wl.bf16_operand((n, k), "int", 1.0, 17001 + 2 * seed)
    x, w = dev_bf16(xb), dev_bf16(wb)
    ref = orc.gemm(xb, wb)
    ws = torch.zeros(ws_bytes(fo, m, n, k, R, c["split"]), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    _Epoch.e += 1
    e = _Epoch.e
    flags = torch.full((R,), e, dtype=torch.int32, device="cuda") if c["flags"] else None
    sched = dict(nchunks=R, local=c["local"], order=c["order"], epoch=e, arrived=flags,
                 mode=fo.FO_SCHED_STRICT if c["strict"] else fo.FO_SCHED_READY_FIRST,
                 split=c["split"], max_workgroups=c["grid"], status=status, timeout_ns=2_000_000_000)
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    y = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
    fo.fo_ag_gemm(x, w, y, fo.Schedule(**sched), ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    if c["bf16"]:
        assert np.array_equal(host(y), orc.f64_to_bf16(ref)), f"seed {seed} bf16"
    else:
        check_exact(host(y), ref, f"seed {seed} ag")

    # GEMM-RS on the same operands: no split, no arrival flags (the local
    # chunk last is the default order)
    _Epoch.e += 1
    e = _Epoch.e
    part = torch.full((m, n), float("nan"), device="cuda")
    done = torch.zeros(R, dtype=torch.int32, device="cuda")
    fo.fo_gemm_rs(x, w, part, done, fo.Schedule(nchunks=R, local=c["local"], epoch=e,
                                                max_workgroups=c["grid"], status=status), ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert (host(done) == e).all()
    check_exact(host(part), ref, f"seed {seed} gemm_rs")


def draw_a2a(seed: int) -> dict:
    g = np.random.Generator(np.random.PCG64(41000 + seed))
    P = int(g.choice([1, 2, 3, 4, 8]))
    return {
        "P": P, "m": int(g.integers(8, 1200)), "n": int(g.integers(8, 900)),
        "kp": int(g.choice([8, 64, 120, 256, 520])),
        "local": int(g.integers(0, P)),
        "order": [int(v) for v in g.permutation(P)],
        "flags": bool(g.integers(0, 2)),
        "grid": int(g.choice([0, 0, 1, 9, 64])),
        "bf16": bool(g.integers(0, 3) == 0),
    }


@pytest.mark.parametrize("seed", seeds(24))
def test_random_a2a_gemm_int_exact(fo, orc, seed):
    """Flash All-to-All GEMM: random piece count and width, m, n, local
    rank, piece order, preset flags, workgroup cap and output type; every
    element bit-exact on integer inputs."""
    c = draw_a2a(seed)
    log(f"case: a2a seed {seed} {c}")
    P, m, n, kp = c["P"], c["m"], c["n"], c["kp"]
    x = wl.bf16_operand((m, kp * P), "int", 1.0, 42000 + 2 * seed)
    wb = wl.bf16_operand((n, kp * P), "int", 1.0, 42001 + 2 * seed)
    pieces_b = [np.ascontiguousarray(x[:, q * kp:(q + 1) * kp]) for q in range(P)]
    ref = orc.a2a_gemm(pieces_b, wb)
    _Epoch.e += 1
    e = _Epoch.e
    flags = torch.full((P,), e, dtype=torch.int32, device="cuda") if c["flags"] else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    y = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    fo.fo_a2a_gemm([dev_bf16(p) for p in pieces_b], dev_bf16(wb), y,
                   fo.Schedule(nchunks=P, local=c["local"], order=c["order"], epoch=e, arrived=flags,
                               max_workgroups=c["grid"], status=status, timeout_ns=2_000_000_000), ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    if c["bf16"]:
        assert np.array_equal(host(y), orc.f64_to_bf16(ref)), f"seed {seed} bf16"
    else:
        check_exact(host(y), ref, f"seed {seed} a2a")


def draw_qsa(seed: int) -> dict:
    g = np.random.Generator(np.random.PCG64(43000 + seed))
    R = int(g.choice([1, 2, 3, 4, 6]))
    return {
        "R": R, "S": R * 128 * int(g.integers(1, 5 if R <= 3 else 3)), "H": int(g.integers(1, 4)),
        "causal": bool(g.integers(0, 2)),
        "order": [int(v) for v in g.permutation(R)],
        "flags": bool(g.integers(0, 2)),
        "grid": int(g.choice([0, 0, 1, 13, 100])),
        "bf16": bool(g.integers(0, 3) == 0),
    }


@pytest.mark.parametrize("seed", seeds(16))
def test_random_qsa_within_bar(fo, orc, seed):
    """Query-split attention: random sequence length, chunk count, heads,
    mask, stage order, preset flags, workgroup cap and output type; within
    the bar of the fp64 oracle, and the counters back to zero."""
    from oracle import attention
    c = draw_qsa(seed)
    log(f"case: qsa seed {seed} {c}")
    S, H, R, D = c["S"], c["H"], c["R"], 128
    qkv = wl.bf16_operand((S, 3 * H * D), "gauss", 1.0, 44000 + seed)
    ref = attention.attention(qkv, H, D, c["causal"])
    _Epoch.e += 1
    e = _Epoch.e
    flags = torch.full((R,), e, dtype=torch.int32, device="cuda") if c["flags"] else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    o = torch.full((S, H * D), float("nan"), dtype=dt, device="cuda")
    ws = torch.zeros(fo.fo_qsa_workspace_bytes(S, H, D, R), dtype=torch.uint8, device="cuda")
    fo.fo_qsa_attention(dev_bf16(qkv), o, H, D, c["causal"],
                        fo.Schedule(nchunks=R, order=c["order"], epoch=e, arrived=flags,
                                    max_workgroups=c["grid"], status=status, timeout_ns=2_000_000_000), ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    if c["bf16"]:
        check_tolerance(bf16_bits_to_f64(host(o)), ref, frob_ref=bf16_bits_to_f64(orc.f64_to_bf16(ref)),
                        what=f"seed {seed} bf16")
    else:
        check_tolerance(host(o), ref, what=f"seed {seed}")
    counters = (1024 + H * (S // 128) + R * H) * 4
    assert int(ws[:counters].sum()) == 0, "counters not returned to zero"


def draw_reduce(seed: int) -> dict:
    g = np.random.Generator(np.random.PCG64(45000 + seed))
    R = int(g.choice([1, 2, 3, 5, 8, 13, 16]))
    return {
        "R": R, "n": 4 * int(g.integers(1, 75000)), "local": int(g.integers(0, R)),   # n % 4 == 0 (16-byte rows)
        "order": [int(v) for v in g.permutation(R)],
        "flags": bool(g.integers(0, 2)),
        "grid": int(g.choice([0, 0, 1, 5, 77])),
        "out": str(g.choice(["f32", "bf16", "inplace"])),
    }


@pytest.mark.parametrize("seed", seeds(24))
def test_random_chunk_reduce_int_exact(fo, orc, seed):
    """Chunk reduce-add: random source count, length (ragged), local source,
    order, preset flags, workgroup cap and output (fp32, bf16, in place);
    integer sources, every element exact."""
    c = draw_reduce(seed)
    log(f"case: reduce seed {seed} {c}")
    R, n, local = c["R"], c["n"], c["local"]
    srcs = [wl.f32_operand((n,), "int", 1.0, 46000 + 64 * seed + q) for q in range(R)]
    ref = orc.reduce(srcs)
    d = [torch.from_numpy(a).cuda() for a in srcs]
    _Epoch.e += 1
    e = _Epoch.e
    flags = torch.full((R,), e, dtype=torch.int32, device="cuda") if c["flags"] else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if c["out"] == "inplace":
        dst = d[local]
    else:
        dst = torch.full((n,), float("nan"), dtype=torch.bfloat16 if c["out"] == "bf16" else torch.float32,
                         device="cuda")
    fo.fo_chunk_reduce(dst, d, fo.Schedule(nchunks=R, local=local, order=c["order"], epoch=e, arrived=flags,
                                           max_workgroups=c["grid"], status=status, timeout_ns=2_000_000_000))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    if c["out"] == "bf16":
        assert np.array_equal(host(dst), orc.f64_to_bf16(ref)), f"seed {seed} bf16"
    else:
        check_exact(host(dst), ref, f"seed {seed} reduce")


def draw_fused(seed: int) -> dict:
    g = np.random.Generator(np.random.PCG64(47000 + seed))
    R = int(g.choice([1, 2, 3, 4, 5, 8]))
    return {
        "R": R, "mc": int(g.integers(1, 80)) * 8, "n": 4 * int(g.integers(2, 225)),   # n % 4 == 0
        "k": int(g.choice([8, 64, 200, 1024])), "local": int(g.integers(0, R)),
        "flags": bool(g.integers(0, 2)), "grid": int(g.choice([0, 0, 3, 40])),
        "bf16": bool(g.integers(0, 2)), "ring": bool(g.integers(0, 2)),
    }


@pytest.mark.parametrize("seed", seeds(24))
def test_random_fused_and_ring_rs_int_exact(fo, orc, seed):
    """GEMM-RS with the reduce in the same launch, direct or ring form:
    random shape, chunks, local rank, preset incoming flags, workgroup cap
    and shard type; partials, shard (and the ring's forwarded sums) exact
    on integer inputs, done flags all released."""
    c = draw_fused(seed)
    log(f"case: fused seed {seed} {c}")
    R, mc, n, k, local = c["R"], c["mc"], c["n"], c["k"], c["local"]
    m = R * mc
    xb = wl.bf16_operand((m, k), "int", 1.0, 48000 + 2 * seed)
    wb = wl.bf16_operand((n, k), "int", 1.0, 48001 + 2 * seed)
    inc = [wl.f32_operand((mc, n), "int", 1.0, 48100 + 16 * seed + q) for q in range(R)]
    prod = orc.gemm(xb, wb)
    x, w = dev_bf16(xb), dev_bf16(wb)
    part = torch.full((m, n), float("nan"), device="cuda")
    sdt = torch.bfloat16 if c["bf16"] else torch.float32
    shard = torch.full((mc, n), float("nan"), dtype=sdt, device="cuda")
    done = torch.zeros(R, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    _Epoch.e += 1
    e = _Epoch.e
    flags = torch.full((R,), e, dtype=torch.int32, device="cuda") if c["flags"] else None
    s = fo.Schedule(nchunks=R, local=local, epoch=e, arrived=flags, status=status, max_workgroups=c["grid"],
                    timeout_ns=2_000_000_000)
    if c["ring"]:
        # ring form: every chunk but local - 1 receives an accumulated partial
        start = (local - 1) % R
        incoming = [None if (q == start and R > 1) else torch.from_numpy(inc[q]).cuda() for q in range(R)]
        fo.fo_gemm_rs_ring(x, w, part, done, shard, incoming, s, ws)
    else:
        incoming = [None if q == local else torch.from_numpy(inc[q]).cuda() for q in range(R)]
        fo.fo_gemm_rs_reduce(x, w, part, done, shard, incoming, s, ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert (host(done) == e).all()
    loc = slice(local * mc, (local + 1) * mc)
    if c["ring"]:
        want = prod.copy()
        for q in range(R):
            if incoming[q] is not None and q != local:
                want[q * mc:(q + 1) * mc] += inc[q]
        if R > 1:
            peers = np.r_[0:local * mc, (local + 1) * mc:m]
            check_exact(host(part)[peers], want[peers], f"seed {seed} forwarded sums")
        check_exact(host(part)[loc], prod[loc], f"seed {seed} local partial")
        ref = prod[loc] + (inc[local] if incoming[local] is not None else 0.0)
    else:
        check_exact(host(part), prod, f"seed {seed} partials")
        ref = orc.gemm_rs_shard(xb, wb, R, local, [None if q == local else inc[q] for q in range(R)])
    if c["bf16"]:
        assert np.array_equal(host(shard), orc.f64_to_bf16(ref)), f"seed {seed} bf16 shard"
    else:
        check_exact(host(shard), ref, f"seed {seed} shard")


def draw_emulated(seed: int) -> dict:
    g = np.random.Generator(np.random.PCG64(49000 + seed))
    R = int(g.choice([2, 3, 4, 6, 8, 12]))
    local = int(g.integers(0, R))
    peers = [q for q in range(R) if q != local]
    return {
        "R": R, "mc": int(g.integers(1, 64)) * 8, "n": int(g.integers(8, 700)),
        "k": int(g.choice([64, 512, 1024, 2048])), "local": local,
        "arrival": [int(v) for v in g.permutation(peers)],
        "gap_ns": int(g.choice([0, 3000, 20000, 60000])),
        "strict": bool(g.integers(0, 4) == 0),
        "split": [int(v) for v in g.choice([1, 1, 2, 4, 8], size=R)] if g.integers(0, 3) == 0 else None,
        "grid": int(g.choice([0, 0, 0, 16, 64])),
        "tile": TILES[int(g.integers(0, len(TILES)))],
    }


@pytest.mark.parametrize("seed", seeds(24))
def test_random_ag_gemm_emulated_arrivals_int_exact(fo, orc, seed, monkeypatch):
    """AG-GEMM with the peers' chunks copied by the copy engine into
    NaN-poisoned rows and released at modelled times, in a random landing
    order: random shape, chunks, local rank, gap between landings, STRICT or
    ready-first, splits (explicit or the automatic split of the last peer),
    workgroup cap and tile layout; every element exact."""
    from test_gpu_emulated import side_stream
    c = draw_emulated(seed)
    log(f"case: emulated seed {seed} {c}")
    if c["tile"] is None:
        monkeypatch.delenv("FO_TILE", raising=False)
    else:
        monkeypatch.setenv("FO_TILE", c["tile"])
    R, mc, n, k, local = c["R"], c["mc"], c["n"], c["k"], c["local"]
    m = R * mc
    xb = wl.bf16_operand((m, k), "int", 1.0, 50000 + 2 * seed)
    wb = wl.bf16_operand((n, k), "int", 1.0, 50001 + 2 * seed)
    ref = orc.gemm(xb, wb)
    staging = dev_bf16(xb)
    w = dev_bf16(wb)
    x = staging.clone()
    for q in c["arrival"]:
        x[q * mc:(q + 1) * mc].fill_(float("nan"))
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(ws_bytes(fo, m, n, k, R, c["split"]), dtype=torch.uint8, device="cuda")
    y = torch.full((m, n), float("nan"), device="cuda")
    _Epoch.e += 1
    e = _Epoch.e
    side = side_stream()
    torch.cuda.synchronize()
    rel = [c["gap_ns"] * (i + 1) for i in range(len(c["arrival"]))]
    with torch.cuda.stream(side):
        fo.fo_emulate_arrivals([x[q * mc:(q + 1) * mc] for q in c["arrival"]],
                               [staging[q * mc:(q + 1) * mc] for q in c["arrival"]],
                               rel, c["arrival"], flags, e, es, stream=side)
    fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=R, local=local, arrived=flags, epoch=e, status=status,
                                       mode=fo.FO_SCHED_STRICT if c["strict"] else fo.FO_SCHED_READY_FIRST,
                                       split=c["split"], max_workgroups=c["grid"], timeout_ns=5_000_000_000), ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "flag wait timed out"
    check_exact(host(y), ref, f"seed {seed} emulated")


def draw_qsa_emulated(seed: int) -> dict:
    g = np.random.Generator(np.random.PCG64(51000 + seed))
    R = int(g.choice([2, 3, 4, 6]))
    local = int(g.integers(0, R))
    peers = [q for q in range(R) if q != local]
    return {
        "R": R, "S": R * 128 * int(g.integers(1, 4 if R <= 3 else 3)), "H": int(g.integers(1, 4)),
        "causal": bool(g.integers(0, 2)), "local": local,
        "arrival": [int(v) for v in g.permutation(peers)],
        "order": [int(v) for v in g.permutation(R)] if g.integers(0, 2) else None,
        "gap_ns": int(g.choice([0, 5000, 30000])),
        "grid": int(g.choice([0, 0, 16, 64])),
    }


@pytest.mark.parametrize("seed", seeds(16))
def test_random_qsa_emulated_arrivals_same_bits(fo, orc, seed):
    """Query-split attention with the peers' QKV rows copied into NaN-poisoned
    rows and released in a random order: random length, chunks, heads, mask,
    stage order, gap and workgroup cap.  The output equals, bit for bit, the
    run with every flag preset, and is within the bar of the oracle."""
    from oracle import attention
    from test_gpu_emulated import side_stream
    c = draw_qsa_emulated(seed)
    log(f"case: qsa emulated seed {seed} {c}")
    S, H, R, D, local = c["S"], c["H"], c["R"], 128, c["local"]
    cs = S // R
    qkv_b = wl.bf16_operand((S, 3 * H * D), "gauss", 1.0, 52000 + seed)
    ref = attention.attention(qkv_b, H, D, c["causal"])
    staging = dev_bf16(qkv_b)
    ws = torch.zeros(fo.fo_qsa_workspace_bytes(S, H, D, R), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def sched(flags, e):
        return fo.Schedule(nchunks=R, local=local, order=c["order"], arrived=flags, epoch=e, status=status,
                           max_workgroups=c["grid"], timeout_ns=5_000_000_000)

    _Epoch.e += 1
    base = torch.full((S, H * D), float("nan"), device="cuda")
    fo.fo_qsa_attention(staging, base, H, D, c["causal"],
                        sched(torch.full((R,), _Epoch.e, dtype=torch.int32, device="cuda"), _Epoch.e), ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    qkv = staging.clone()
    for q in c["arrival"]:
        qkv[q * cs:(q + 1) * cs].fill_(float("nan"))
    flags = torch.zeros(R, dtype=torch.int32, device="cuda")
    es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
    o = torch.full((S, H * D), float("nan"), device="cuda")
    _Epoch.e += 1
    e = _Epoch.e
    side = side_stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        fo.fo_emulate_arrivals([qkv[q * cs:(q + 1) * cs] for q in c["arrival"]],
                               [staging[q * cs:(q + 1) * cs] for q in c["arrival"]],
                               [c["gap_ns"] * (i + 1) for i in range(R - 1)], c["arrival"], flags, e, es,
                               stream=side)
    fo.fo_qsa_attention(qkv, o, H, D, c["causal"], sched(flags, e), ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "flag wait timed out"
    got = host(o)
    assert np.array_equal(got.view(np.uint32), host(base).view(np.uint32)), f"seed {seed}: landings changed the bits"
    check_tolerance(got, ref, what=f"seed {seed} emulated")


@pytest.mark.parametrize("seed", seeds(8))
def test_random_ag_gemm_bits_independent_of_landings(fo, orc, seed, monkeypatch):
    """Gaussian inputs, a fixed split vector: the output bits do not depend
    on when or in which order the chunks land (two emulated landing orders
    and gaps, and every flag preset, give the same bits), and are within the
    bar of the oracle."""
    from test_gpu_emulated import side_stream
    monkeypatch.delenv("FO_TILE", raising=False)
    g = np.random.Generator(np.random.PCG64(53000 + seed))
    R = int(g.choice([3, 4, 8]))
    local = int(g.integers(0, R))
    mc, n, k = int(g.integers(4, 40)) * 16, int(g.integers(64, 900)), int(g.choice([512, 1024, 2048]))
    m = R * mc
    split = [int(v) for v in g.choice([1, 2, 4, 8], size=R)]
    log(f"case: determinism seed {seed} R={R} local={local} {m}x{n}x{k} split {split}")
    xb = wl.bf16_operand((m, k), "gauss", 1.0, 54000 + 2 * seed)
    wb = wl.bf16_operand((n, k), "gauss", 0.02, 54001 + 2 * seed)
    staging = dev_bf16(xb)
    w = dev_bf16(wb)
    ws = torch.zeros(ws_bytes(fo, m, n, k, R, split), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    peers = [q for q in range(R) if q != local]
    outs = []
    for run in range(3):
        x = staging.clone()
        y = torch.full((m, n), float("nan"), device="cuda")
        _Epoch.e += 1
        e = _Epoch.e
        if run == 0:
            flags = torch.full((R,), e, dtype=torch.int32, device="cuda")
        else:
            arrival = [int(v) for v in g.permutation(peers)]
            for q in arrival:
                x[q * mc:(q + 1) * mc].fill_(float("nan"))
            flags = torch.zeros(R, dtype=torch.int32, device="cuda")
            es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
            side = side_stream()
            torch.cuda.synchronize()
            gap = int(g.choice([0, 4000, 25000]))
            with torch.cuda.stream(side):
                fo.fo_emulate_arrivals([x[q * mc:(q + 1) * mc] for q in arrival],
                                       [staging[q * mc:(q + 1) * mc] for q in arrival],
                                       [gap * (i + 1) for i in range(len(arrival))], arrival, flags, e, es,
                                       stream=side)
        fo.fo_ag_gemm(x, w, y, fo.Schedule(nchunks=R, local=local, arrived=flags, epoch=e, status=status,
                                           split=split, timeout_ns=5_000_000_000), ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "flag wait timed out"
        outs.append(host(y))
    for i in (1, 2):
        assert np.array_equal(outs[i].view(np.uint32), outs[0].view(np.uint32)), f"seed {seed} run {i}"
    rows = np.arange(0, m, 7)
    check_tolerance(outs[0][rows], orc.gemm(xb[rows], wb), what=f"seed {seed}")


def draw_fused_emulated(seed: int) -> dict:
    g = np.random.Generator(np.random.PCG64(55000 + seed))
    R = int(g.choice([2, 3, 4, 8]))
    local = int(g.integers(0, R))
    return {
        "R": R, "mc": int(g.integers(1, 48)) * 8, "n": 4 * int(g.integers(2, 200)),
        "k": int(g.choice([64, 512, 1024])), "local": local,
        "gap_ns": int(g.choice([0, 5000, 30000])), "grid": int(g.choice([0, 0, 40])),
        "ring": bool(g.integers(0, 2)), "perm_seed": int(g.integers(0, 1 << 30)),
    }


@pytest.mark.parametrize("seed", seeds(16))
def test_random_fused_and_ring_rs_emulated_incoming_int_exact(fo, orc, seed):
    """GEMM-RS with the reduce in the same launch (direct or ring form), the
    incoming partials copied by the copy engine into NaN-poisoned inboxes in
    a random order at a random gap: the shard (and the ring's forwarded sums)
    exact on integer inputs, the same bits as with every partial present."""
    from test_gpu_emulated import side_stream
    c = draw_fused_emulated(seed)
    log(f"case: fused emulated seed {seed} {c}")
    R, mc, n, k, local = c["R"], c["mc"], c["n"], c["k"], c["local"]
    m = R * mc
    xb = wl.bf16_operand((m, k), "int", 1.0, 56000 + 2 * seed)
    wb = wl.bf16_operand((n, k), "int", 1.0, 56001 + 2 * seed)
    inc = [wl.f32_operand((mc, n), "int", 1.0, 56100 + 16 * seed + q) for q in range(R)]
    x, w = dev_bf16(xb), dev_bf16(wb)
    if c["ring"]:
        start = (local - 1) % R
        has = [not (q == start and R > 1) for q in range(R)]
    else:
        has = [q != local for q in range(R)]
    staging = [torch.from_numpy(inc[q]).cuda() if has[q] else None for q in range(R)]
    senders = [q for q in range(R) if has[q]]
    arrival = [senders[i] for i in np.random.Generator(np.random.PCG64(c["perm_seed"])).permutation(len(senders))]
    ws = torch.zeros(fo.fo_workspace_bytes(m, n, k, R), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = []
    for emulated in (False, True):
        inbox = [None if a is None else (torch.full_like(a, float("nan")) if emulated else a.clone()) for a in staging]
        part = torch.full((m, n), float("nan"), device="cuda")
        shard = torch.full((mc, n), float("nan"), device="cuda")
        done = torch.zeros(R, dtype=torch.int32, device="cuda")
        _Epoch.e += 1
        e = _Epoch.e
        flags = torch.zeros(R, dtype=torch.int32, device="cuda") if emulated else \
            torch.full((R,), e, dtype=torch.int32, device="cuda")
        if emulated:
            es = torch.zeros(R + 2, dtype=torch.int64, device="cuda")
            side = side_stream()
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                fo.fo_emulate_arrivals([inbox[q] for q in arrival], [staging[q] for q in arrival],
                                       [c["gap_ns"] * (i + 1) for i in range(len(arrival))], arrival, flags, e, es,
                                       stream=side)
        s = fo.Schedule(nchunks=R, local=local, epoch=e, arrived=flags, status=status, max_workgroups=c["grid"],
                        timeout_ns=5_000_000_000)
        if c["ring"]:
            fo.fo_gemm_rs_ring(x, w, part, done, shard, inbox, s, ws)
        else:
            fo.fo_gemm_rs_reduce(x, w, part, done, shard, inbox, s, ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "flag wait timed out"
        assert (host(done) == e).all()
        outs.append((host(part), host(shard)))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32)), f"seed {seed} partials"
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32)), f"seed {seed} shard"
    prod = orc.gemm(xb, wb)
    loc = slice(local * mc, (local + 1) * mc)
    if c["ring"]:
        ref = prod[loc] + (inc[local] if has[local] else 0.0)
    else:
        ref = orc.gemm_rs_shard(xb, wb, R, local, [None if q == local else inc[q] for q in range(R)])
    check_exact(outs[1][1], ref, f"seed {seed} shard")


@pytest.mark.parametrize("seed", seeds(16))
def test_random_a2a_and_reduce_emulated_int_exact(fo, orc, seed):
    """All-to-all GEMM pieces and reduce sources copied into NaN-poisoned
    buffers by the copy engine in a random order at a random gap: every
    element exact on integer inputs."""
    from test_gpu_emulated import side_stream
    g = np.random.Generator(np.random.PCG64(57000 + seed))
    P = int(g.choice([2, 3, 4, 8]))
    local = int(g.integers(0, P))
    m, n, kp = int(g.integers(8, 900)), int(g.integers(8, 700)), int(g.choice([8, 64, 200, 520]))
    gap = int(g.choice([0, 4000, 30000]))
    peers = [q for q in range(P) if q != local]
    arrival = [int(v) for v in g.permutation(peers)]
    log(f"case: a2a/reduce emulated seed {seed} P={P} local={local} m={m} n={n} kp={kp} gap={gap} {arrival}")
    side = side_stream()
    # all-to-all GEMM
    x = wl.bf16_operand((m, kp * P), "int", 1.0, 58000 + 2 * seed)
    wb = wl.bf16_operand((n, kp * P), "int", 1.0, 58001 + 2 * seed)
    pieces_b = [np.ascontiguousarray(x[:, q * kp:(q + 1) * kp]) for q in range(P)]
    staging = [dev_bf16(p_) for p_ in pieces_b]
    inbox = [staging[q].clone() if q == local else torch.full_like(staging[q], float("nan")) for q in range(P)]
    flags = torch.zeros(P, dtype=torch.int32, device="cuda")
    es = torch.zeros(P + 2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    _Epoch.e += 1
    e = _Epoch.e
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        fo.fo_emulate_arrivals([inbox[q] for q in arrival], [staging[q] for q in arrival],
                               [gap * (i + 1) for i in range(len(arrival))], arrival, flags, e, es, stream=side)
    y = torch.full((m, n), float("nan"), device="cuda")
    fo.fo_a2a_gemm(inbox, dev_bf16(wb), y, fo.Schedule(nchunks=P, local=local, arrived=flags, epoch=e, status=status,
                                                       timeout_ns=5_000_000_000),
                   torch.zeros(4096, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "flag wait timed out"
    check_exact(host(y), orc.a2a_gemm(pieces_b, wb), f"seed {seed} a2a")
    # reduce-add of the same peers' sources into the local one
    nn = 4 * int(g.integers(1, 40000))
    srcs = [wl.f32_operand((nn,), "int", 1.0, 59000 + 16 * seed + q) for q in range(P)]
    src_st = [torch.from_numpy(a).cuda() for a in srcs]
    dsts = [src_st[q].clone() if q == local else torch.full_like(src_st[q], float("nan")) for q in range(P)]
    flags.zero_()
    _Epoch.e += 1
    e = _Epoch.e
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        fo.fo_emulate_arrivals([dsts[q] for q in arrival], [src_st[q] for q in arrival],
                               [gap * (i + 1) for i in range(len(arrival))], arrival, flags, e, es, stream=side)
    out = torch.full((nn,), float("nan"), device="cuda")
    fo.fo_chunk_reduce(out, dsts, fo.Schedule(nchunks=P, local=local, arrived=flags, epoch=e, status=status,
                                              timeout_ns=5_000_000_000))
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "flag wait timed out"
    check_exact(host(out), orc.reduce(srcs), f"seed {seed} reduce")
