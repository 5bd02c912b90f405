"""Pins for the CPU oracle, against things other than the oracle itself.

Each test fixes the oracle to an independent fact: a library routine
(numpy fp64 matmul, Python's math.fsum, torch's bf16 decode), exact rational
brute force, integer arithmetic, closed forms (identity, one-hot), the
invariants that the pages' "exact algorithm" implies (any chunk order, chunked
equals unchunked, the ring decomposition equals the collective), and hand
worked values in tests/golden/.
"""
import itertools
import math
import os

import numpy as np
import pytest

import workloads as wl
from oracle import brute, ring

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---- bf16 decode / encode -------------------------------------------------

def test_bf16_decode_known_patterns(orc):
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x4049: 3.140625,
             0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
             0xBF40: -0.75, 0x3C00: 2.0 ** -7}
    bits = np.array(list(cases), dtype=np.uint16)
    got = orc.bf16_to_f64(bits)
    assert list(got) == list(cases.values())


def test_bf16_decode_all_finite_patterns_vs_torch_and_fraction(orc):
    import torch
    allb = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[((allb >> 7) & 0xFF) != 0xFF]
    t = torch.from_numpy(finite.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    sample = finite[:: 97]
    got = orc.bf16_to_f64(sample)
    assert np.array_equal(got, t[:: 97])
    for b, g in zip(sample[:: 7], got[:: 7]):
        assert brute.bf16_fraction(int(b)) == g


def test_f64_to_bf16_rne_ties_and_library(orc):
    # closed-form ties: 1 + 2^-8 lies half way between 1 and 1 + 2^-7
    tie_cases = [(1.0 + 2 ** -8, 0x3F80),            # tie -> even (1.0)
                 (1.0 + 3 * 2 ** -8, 0x3F82),        # tie -> even (1 + 2^-6)
                 (1.0 + 2 ** -8 + 2 ** -40, 0x3F81),  # just above tie -> up
                 (-(1.0 + 2 ** -8), 0xBF80),
                 (2.0 ** -134, 0x0000),              # half the smallest subnormal -> 0
                 (3 * 2.0 ** -134, 0x0002),          # 1.5 quanta -> 2
                 (0.0, 0x0000), (-0.0, 0x8000)]
    vals = np.array([v for v, _ in tie_cases], dtype=np.float64)
    got = orc.f64_to_bf16(vals)
    assert [int(g) for g in got] == [b for _, b in tie_cases]
    # a value whose float32 rounding would create a false tie: one rounding only
    v = 1.0 + 2 ** -8 + 2 ** -30     # rounds to 1+2^-8 in fp32, then to 1.0
    assert int(orc.f64_to_bf16(np.array([v]))[0]) == 0x3F81
    # against torch for values exactly representable in fp32 (single rounding)
    import torch
    x = rng(5).standard_normal(20000).astype(np.float32).astype(np.float64) * 37.0
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f64_to_bf16(x), ref)


# ---- exact summation --------------------------------------------------------

def _hard_sums(n_cases=400, seed=11):
    g = rng(seed)
    out = []
    for _ in range(n_cases):
        R = int(g.integers(1, 17))
        e = g.integers(-60, 60, size=R)
        v = g.standard_normal(R) * np.exp2(e)
        if R > 2 and g.random() < 0.5:         # add catastrophic cancellation
            v[-1] = -np.sum(v[:-1])
        out.append(v)
    # half-way cases for the final rounding
    out.append(np.array([1.0, 2.0 ** -53, 2.0 ** -106]))
    out.append(np.array([1.0, 2.0 ** -53, -(2.0 ** -106)]))
    out.append(np.array([1.0, -(2.0 ** -54), 2.0 ** -107, 1e-300]))
    out.append(np.array([1e308, 1e308 * 0.5, -1e308]))
    return out


def test_sum_exact_matches_math_fsum(orc):
    for v in _hard_sums():
        assert orc.sum_exact(v) == math.fsum(v)


def test_sum_exact_matches_fraction(orc):
    for v in _hard_sums(120, seed=12):
        assert orc.sum_exact(v) == float(brute.sum_exact(v))


def test_reduce_order_invariant_and_exact(orc):
    g = rng(13)
    for R in (1, 2, 3, 4):
        srcs = [(g.standard_normal(257) * np.exp2(g.integers(-20, 20, 257))).astype(np.float32)
                for _ in range(R)]
        ref = orc.reduce(srcs)
        for perm in itertools.permutations(range(R)):
            assert np.array_equal(orc.reduce([srcs[p] for p in perm]), ref)
        fs = np.array([math.fsum(float(s[e]) for s in srcs) for e in range(257)])
        assert np.array_equal(ref, fs)


def test_reduce_integer_equals_int64(orc):
    c = wl.CFG4
    srcs = wl.reduce_sources(c, "int", n=4096)
    ref = np.sum(np.stack([s.astype(np.int64) for s in srcs]), axis=0)
    assert np.array_equal(orc.reduce(srcs), ref.astype(np.float64))


# ---- GEMM -------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k", [(37, 23, 19), (64, 48, 128), (5, 130, 33)])
def test_gemm_vs_numpy(orc, m, n, k):
    x = wl.bf16_operand((m, k), "gauss", 1.0, 101)
    w = wl.bf16_operand((n, k), "gauss", 0.02, 102)
    xf = orc.bf16_to_f64(x)
    wf = orc.bf16_to_f64(w)
    y = orc.gemm(x, w)
    ref = xf @ wf.T
    scale = np.abs(xf) @ np.abs(wf).T
    assert np.all(np.abs(y - ref) <= 1e-12 * scale + 1e-300)
    # a transposed operand would not even have this shape, and a wrong index
    # would break the comparison
    assert y.shape == (m, n)


@pytest.mark.parametrize("mode", ["int", "gauss"])
def test_gemm_vs_fraction_bruteforce(orc, mode):
    for (m, n, k), seed in zip([(3, 4, 5), (7, 5, 16), (16, 9, 13)], (1, 2, 3)):
        x = wl.bf16_operand((m, k), mode, 1.0, 200 + seed)
        w = wl.bf16_operand((n, k), mode, 0.5, 300 + seed)
        exact = brute.gemm(x, w)
        y = orc.gemm(x, w)
        if mode == "int":
            assert np.array_equal(y, brute.to_float(exact))
        else:
            ex = brute.to_float(exact)
            absx = np.abs(orc.bf16_to_f64(x)) @ np.abs(orc.bf16_to_f64(w)).T
            assert np.all(np.abs(y - ex) <= k * 2.0 ** -53 * absx)


def test_gemm_integer_equals_int64_cfg1(orc):
    c = wl.CFG1
    x, w = wl.gemm_inputs(c, "int")
    xi = orc.bf16_to_f64(x).astype(np.int64)
    wi = orc.bf16_to_f64(w).astype(np.int64)
    ref = xi @ wi.T
    assert np.array_equal(orc.gemm(x, w), ref.astype(np.float64))
    assert np.abs(ref).max() <= 9 * c.k


def test_gemm_identity_and_one_hot(orc):
    k = 24
    x = wl.bf16_operand((10, k), "gauss", 1.0, 401)
    eye = wl.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    assert np.array_equal(orc.gemm(x, eye), orc.bf16_to_f64(x))
    w = wl.bf16_operand((7, k), "gauss", 1.0, 402)          # stored [n, k]
    idx = [3, 0, 23, 11]
    onehot = np.zeros((len(idx), k), dtype=np.float32)
    onehot[np.arange(len(idx)), idx] = 1.0
    y = orc.gemm(wl.f32_to_bf16_bits(onehot), w)
    assert np.array_equal(y, orc.bf16_to_f64(w)[:, idx].T)


def test_chunked_equals_unchunked_every_order(orc):
    m, n, k = 48, 20, 36
    x = wl.bf16_operand((m, k), "gauss", 1.0, 501)
    w = wl.bf16_operand((n, k), "gauss", 0.02, 502)
    full = orc.gemm(x, w)
    for R in (1, 2, 3, 4):
        for order in itertools.permutations(range(R)):
            assert np.array_equal(orc.ag_gemm(x, w, R, list(order)), full)
    g = rng(503)
    for R in (8, 16):
        for _ in range(8):
            o = list(g.permutation(R))
            assert np.array_equal(orc.ag_gemm(x, w, R, o), full)


def test_gemm_rs_shard_vs_fraction_and_int64(orc):
    m, n, k, R = 16, 6, 10, 4
    for mode in ("int", "gauss"):
        x = wl.bf16_operand((m, k), mode, 1.0, 601)
        w = wl.bf16_operand((n, k), mode, 0.3, 602)
        inc = [None if q == 1 else wl.f32_operand((m // R, n), mode, 0.7, 610 + q, 4096)
               for q in range(R)]
        s = orc.gemm_rs_shard(x, w, R, 1, inc)
        P = brute.gemm(x, w)
        mc = m // R
        ex = [[P[mc + i][j] + sum((brute.f32_fraction(inc[q][i, j]) for q in range(R) if q != 1), 0)
               for j in range(n)] for i in range(mc)]
        assert np.array_equal(s, brute.to_float(ex))


def test_ring_ag_equals_collective(orc):
    R, mc, n, k = 4, 8, 12, 20
    chunks = [wl.bf16_operand((mc, k), "int", 1.0, 700 + r) for r in range(R)]
    ws = [wl.bf16_operand((n + r, k), "int", 1.0, 710 + r) for r in range(R)]
    ys, done = ring.ring_ag(chunks, ws)
    X = np.concatenate(chunks)
    for r in range(R):
        assert np.array_equal(ys[r], orc.gemm(X, ws[r]))
        # local slice first, then received slices from predecessors
        assert done[r] == [(r - s) % R for s in range(R)]


@pytest.mark.parametrize("mode", ["int", "gauss"])
def test_ring_rs_equals_collective(orc, mode):
    R, m, n = 4, 16, 10
    ks = [6, 9, 5, 12]
    xs = [wl.bf16_operand((m, ks[r]), mode, 1.0, 800 + r) for r in range(R)]
    ws = [wl.bf16_operand((n, ks[r]), mode, 0.5, 810 + r) for r in range(R)]
    shards, done = ring.ring_rs(xs, ws)
    mc = m // R
    for r in range(R):
        exact = [[sum((brute.gemm(xs[q][r * mc:(r + 1) * mc], ws[q])[i][j] for q in range(R)), 0)
                  for j in range(n)] for i in range(mc)]
        ex = brute.to_float(exact)
        if mode == "int":
            assert np.array_equal(shards[r], ex)
        else:
            assert np.allclose(shards[r], ex, rtol=1e-13, atol=1e-13)
        assert done[r][-1] == r       # the local chunk is computed last


@pytest.mark.parametrize("mode", ["int", "gauss"])
def test_ring_rs_rank_composes_to_collective(orc, mode):
    """ring_rs_rank run on every rank, each rank's incoming partial of chunk
    c being its predecessor's forwarded sum (none where the chunk starts, at
    rank c+1), gives every rank the collective's shard: exactly on integers,
    and equal to the message-passing simulation in ring.py bit for bit."""
    R, m, n = 4, 16, 10
    ks = [6, 9, 5, 12]
    xs = [wl.bf16_operand((m, ks[r]), mode, 1.0, 820 + r) for r in range(R)]
    ws = [wl.bf16_operand((n, ks[r]), mode, 0.5, 830 + r) for r in range(R)]
    mc = m // R
    fwd = [None] * R
    shards = [None] * R
    for _ in range(R):          # R rounds settle every chain of R - 1 hops
        new = []
        for r in range(R):
            prev = (r - 1) % R
            inc = [None if (c == prev or fwd[prev] is None) else fwd[prev][c * mc:(c + 1) * mc]
                   for c in range(R)]
            f, sh = orc.ring_rs_rank(xs[r], ws[r], R, r, inc)
            new.append(f)
            shards[r] = sh
        fwd = new
    ref, _ = ring.ring_rs(xs, ws)
    for r in range(R):
        assert np.array_equal(shards[r], ref[r])
        if mode == "int":
            exact = [[sum((brute.gemm(xs[q][r * mc:(r + 1) * mc], ws[q])[i][j] for q in range(R)), 0)
                      for j in range(n)] for i in range(mc)]
            assert np.array_equal(shards[r], brute.to_float(exact))


def test_ring_rs_rank_single_rank(orc):
    """One chunk, no incoming partial: the shard is the product itself."""
    x = wl.bf16_operand((8, 16), "int", 1.0, 840)
    w = wl.bf16_operand((6, 16), "int", 1.0, 841)
    f, sh = orc.ring_rs_rank(x, w, 1, 0, [None])
    assert np.array_equal(sh, orc.gemm(x, w)) and np.array_equal(f, sh)


def test_golden_worked_example(orc):
    """Hand-worked 4x2 example (tests/golden/worked_example.txt)."""
    vals = {}
    with open(os.path.join(GOLDEN, "worked_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                key, rest = line.split("=")
                vals[key.strip()] = np.array(eval(rest, {"__builtins__": {}}), dtype=np.float64)
    x = wl.f32_to_bf16_bits(vals["X"].astype(np.float32))
    w = wl.f32_to_bf16_bits(vals["W_stored"].astype(np.float32))
    assert np.array_equal(orc.gemm(x, w), vals["Y"])
    assert np.array_equal(orc.ag_gemm(x, w, 2, [1, 0]), vals["Y"])
    inc = [None, vals["IN1"].astype(np.float32)]
    assert np.array_equal(orc.gemm_rs_shard(x, w, 2, 0, inc), vals["SHARD0"])
    srcs = [vals["SRC0"].astype(np.float32), vals["SRC1"].astype(np.float32),
            vals["SRC2"].astype(np.float32)]
    assert np.array_equal(orc.reduce(srcs), vals["SUM"])


# ---- Flash All-to-All (Ulysses output projection) ----------------------------

def a2a_case(m, k, n, P, mode, seed):
    x = wl.bf16_operand((m, k), mode, 1.0, seed)
    w = wl.bf16_operand((n, k), mode, 0.02 if mode == "gauss" else 1.0, seed + 1)
    kp = k // P
    pieces = [np.ascontiguousarray(x[:, q * kp:(q + 1) * kp]) for q in range(P)]
    return x, w, pieces


@pytest.mark.parametrize("m,k,n,P", [(37, 48, 23, 4), (64, 128, 40, 8), (5, 30, 7, 3)])
def test_a2a_gemm_vs_numpy_block_sum(orc, m, k, n, P):
    """Y against numpy fp64 as a sum of per-piece block products (a different
    formula from the oracle's assembled product): block q of the gathered
    rows must meet columns block q of W."""
    x, w, pieces = a2a_case(m, k, n, P, "gauss", 700 + m)
    kp = k // P
    wf = orc.bf16_to_f64(w)
    ref = sum(orc.bf16_to_f64(pieces[q]) @ wf[:, q * kp:(q + 1) * kp].T for q in range(P))
    scale = np.abs(orc.bf16_to_f64(x)) @ np.abs(wf).T
    y = orc.a2a_gemm(pieces, w)
    assert np.all(np.abs(y - ref) <= 1e-12 * scale + 1e-300)
    xi, wi, pi = a2a_case(m, k, n, P, "int", 800 + m)
    ri = sum(orc.bf16_to_f64(pi[q]).astype(np.int64) @ orc.bf16_to_f64(wi[:, q * kp:(q + 1) * kp]).astype(np.int64).T
             for q in range(P))
    assert np.array_equal(orc.a2a_gemm(pi, wi), ri.astype(np.float64))


@pytest.mark.parametrize("mode", ["int", "gauss"])
def test_a2a_gemm_vs_fraction_bruteforce(orc, mode):
    for (m, k, n, P), seed in zip([(3, 8, 4, 2), (4, 12, 5, 3), (2, 16, 3, 4)], (1, 2, 3)):
        x, w, pieces = a2a_case(m, k, n, P, mode, 900 + seed)
        kp = k // P
        exact = None
        for q in range(P):
            part = brute.gemm(pieces[q], np.ascontiguousarray(w[:, q * kp:(q + 1) * kp]))
            exact = part if exact is None else [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(exact, part)]
        ex = brute.to_float(exact)
        y = orc.a2a_gemm(pieces, w)
        if mode == "int":
            assert np.array_equal(y, ex)
        else:
            absx = np.abs(orc.bf16_to_f64(x)) @ np.abs(orc.bf16_to_f64(w)).T
            assert np.all(np.abs(y - ex) <= k * 2.0 ** -53 * absx)


def test_a2a_gemm_special_cases(orc):
    x, w, pieces = a2a_case(9, 16, 6, 1, "gauss", 1001)
    assert np.array_equal(orc.a2a_gemm(pieces, w), orc.gemm(x, w))        # one rank
    k, P = 24, 4
    x, _, pieces = a2a_case(10, k, 1, P, "gauss", 1002)
    eye = wl.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    assert np.array_equal(orc.a2a_gemm(pieces, eye), orc.bf16_to_f64(x))  # W = I
    # a zero piece contributes nothing: the others' block products alone
    x, w, pieces = a2a_case(8, k, 5, P, "int", 1003)
    pieces[2] = np.zeros_like(pieces[2])
    kp = k // P
    keep = [q for q in range(P) if q != 2]
    ref = sum(orc.gemm(pieces[q], np.ascontiguousarray(w[:, q * kp:(q + 1) * kp])) for q in keep)
    assert np.array_equal(orc.a2a_gemm(pieces, w), ref)


@pytest.mark.parametrize("P", [2, 4, 8])
@pytest.mark.parametrize("mode", ["int", "gauss"])
def test_ulysses_all_to_all_equals_collective(orc, P, mode):
    """Every rank's pairwise-exchange all-to-all and piece-by-piece output
    projection (oracle/ulysses.py) against the undistributed product of the
    whole attention output with W (numpy); each rank's result also equals the
    oracle's a2a_gemm over the pieces it received."""
    from oracle import ulysses
    S, k, n = 8 * P, 16 * P, 24
    o = wl.bf16_operand((S, k), mode, 1.0, 1100 + P)
    w = wl.bf16_operand((n, k), mode, 0.02 if mode == "gauss" else 1.0, 1101 + P)
    ys, received = ulysses.ulysses_out_proj(o, w, P)
    of, wf = orc.bf16_to_f64(o), orc.bf16_to_f64(w)
    full = of @ wf.T
    sp, kp = S // P, k // P
    for r in range(P):
        assert received[r] == [(r - s) % P for s in range(P)]
        rows = full[r * sp:(r + 1) * sp]
        pieces = [np.ascontiguousarray(o[r * sp:(r + 1) * sp, q * kp:(q + 1) * kp]) for q in range(P)]
        if mode == "int":
            ri = (of.astype(np.int64) @ wf.astype(np.int64).T)[r * sp:(r + 1) * sp]
            assert np.array_equal(ys[r], ri.astype(np.float64))
            assert np.array_equal(orc.a2a_gemm(pieces, w), ys[r])
        else:
            scale = (np.abs(of) @ np.abs(wf).T)[r * sp:(r + 1) * sp]
            assert np.all(np.abs(ys[r] - rows) <= 1e-12 * scale + 1e-300)
            assert np.all(np.abs(orc.a2a_gemm(pieces, w) - rows) <= 1e-12 * scale + 1e-300)


# ---- Query-Split Attention -----------------------------------------------------

def qkv_case(S, H, d, seed, std=1.0):
    return wl.bf16_operand((S, 3 * H * d), "gauss", std, seed)


def test_bf16_fast_decode_matches_c_decode(orc):
    allb = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[((allb >> 7) & 0xFF) != 0xFF][::13]
    assert np.array_equal(orc.bf16_to_f64_fast(finite), orc.bf16_to_f64(finite))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,H,d", [(64, 2, 16), (48, 1, 128), (96, 3, 32)])
def test_attention_vs_torch_sdpa_float64(orc, causal, S, H, d):
    """The plain definition against torch's scaled_dot_product_attention on
    the CPU in float64 (an independent library routine)."""
    import torch
    from oracle import attention as at
    qkv = qkv_case(S, H, d, 1300 + S + d)
    x = orc.bf16_to_f64(qkv)
    t = torch.from_numpy(x)
    q = t[:, :H * d].reshape(S, H, d).transpose(0, 1)
    k = t[:, H * d:2 * H * d].reshape(S, H, d).transpose(0, 1)
    v = t[:, 2 * H * d:].reshape(S, H, d).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    ref = ref.transpose(0, 1).reshape(S, H * d).numpy()
    got = at.attention(qkv, H, d, causal)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_attention_closed_forms(orc):
    """Zero queries give equal weights: every output row is the mean of the
    value rows it sees (all of them, or the prefix 0..i when causal); one key
    whose score dominates selects its value row."""
    from oracle import attention as at
    S, H, d = 40, 2, 16
    qkv = qkv_case(S, H, d, 1401)
    qkv[:, :H * d] = 0
    v = orc.bf16_to_f64(qkv[:, 2 * H * d:])
    full = at.attention(qkv, H, d, False)
    assert np.allclose(full, np.broadcast_to(v.mean(axis=0), (S, H * d)), rtol=0, atol=1e-14)
    cum = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
    assert np.allclose(at.attention(qkv, H, d, True), cum, rtol=0, atol=1e-14)
    qkv = np.zeros((S, 3 * H * d), dtype=np.uint16)
    one = wl.f32_to_bf16_bits(np.array([4.0], dtype=np.float32))[0]
    big = wl.f32_to_bf16_bits(np.array([64.0], dtype=np.float32))[0]
    qkv[:, 0] = one                       # head 0 queries: 4 e_0
    qkv[17, H * d] = big                  # head 0, key 17: 64 e_0 (score 64)
    qkv[:, 2 * H * d:] = wl.bf16_operand((S, H * d), "gauss", 1.0, 1402)
    got = at.attention(qkv, H, d, False)
    vrow = orc.bf16_to_f64(qkv[17, 2 * H * d:2 * H * d + d])
    assert np.allclose(got[:, :d], np.broadcast_to(vrow, (S, d)), rtol=1e-20, atol=1e-20)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_query_split_blocks_equal_plain(orc, causal):
    """The query-split decomposition (per query chunk, per key chunk blocks
    merged with their maxima and sums) equals the plain definition, whatever
    order the key chunks are merged in."""
    from oracle import attention as at
    S, H, d, R = 64, 2, 32, 4
    qkv = qkv_case(S, H, d, 1501 + causal)
    plain = at.attention(qkv, H, d, causal)
    for order in itertools.permutations(range(R)):
        got = at.attention_blocks(qkv, H, d, causal, R, order)
        assert np.max(np.abs(got - plain)) <= 1e-13


def test_attention_key_permutation_invariance(orc):
    """Without a mask, permuting the tokens of K and V together leaves every
    output row unchanged (softmax attention is a set function of the keys)."""
    from oracle import attention as at
    S, H, d = 32, 2, 16
    qkv = qkv_case(S, H, d, 1601)
    perm = rng(1602).permutation(S)
    moved = qkv.copy()
    moved[:, H * d:] = qkv[perm][:, H * d:]
    a = at.attention(qkv, H, d, False)
    b = at.attention(moved, H, d, False)
    assert np.max(np.abs(a - b)) <= 1e-13
