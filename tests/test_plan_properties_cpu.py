"""Property tests of the host-only schedule model over random valid inputs
(hypothesis): whatever the shape, chunk count, local rank and landing
times, the plans are valid schedules and the predictions are consistent
with the landings.  (Later landings do not always predict a later
completion: the model replays greedy ready-first claims, and a greedy list
schedule can finish earlier when a job is released later.)"""
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st

import sp_rank_adaptive_amd as fo

SPLITS = (1, 2, 4, 8)


@st.composite
def problems(draw):
    R = draw(st.integers(1, 16))
    mc = draw(st.integers(1, 64)) * 64
    n = draw(st.integers(1, 64)) * 64
    k = draw(st.integers(1, 128)) * 64
    local = draw(st.integers(0, R - 1))
    arr = [0 if q == local else draw(st.integers(0, 5_000_000)) for q in range(R)]
    grid = draw(st.sampled_from([8, 64, 256]))   # (0 would ask the device for its CU count)
    return R * mc, n, k, R, local, arr, grid


@settings(max_examples=300, deadline=None)
@given(problems())
def test_ag_schedule_is_valid_and_consistent(p):
    m, n, k, R, local, arr, grid = p
    order, split, pred = fo.fo_plan_ag_schedule(m, n, k, R, local, arr, num_workgroups=grid)
    assert sorted(order) == list(range(R)) and order[-1] == local
    times = [arr[c] for c in order[:-1]]
    assert times == sorted(times)                              # peers by landing time
    assert all(s in SPLITS for s in split)
    last = order[-2] if R > 1 else local
    assert all(s == 1 for c, s in enumerate(split) if c != last)  # only the last-landing chunk splits
    assert any(v > 0 for v in pred)
    assert all(v > max(arr) for v in pred if v > 0)            # nothing completes before the last landing
    chosen = pred[SPLITS.index(split[last])]
    assert chosen > 0 and chosen <= min(v for v in pred if v > 0) + 500   # the earliest, up to the 0.5 us margin


@settings(max_examples=150, deadline=None)
@given(problems(), st.sampled_from([10.0, 50.0, 153.0, 400.0, 1000.0, 2000.0]), st.sampled_from([0, 1]))
def test_stream_plan_is_valid(p, bw, topo):
    m, n, k, R, local, _, grid = p
    sub, order, split, pred = fo.fo_plan_ag_stream(m, n, k, R, local, bw, topo, num_workgroups=grid)
    assert sub in SPLITS
    R2 = R * sub
    assert sorted(order) == list(range(R2)) and len(split) == R2
    assert order[R2 - sub:] == list(range(local * sub, (local + 1) * sub))   # the local pieces last
    land = fo.fo_plan_link_arrivals(R, local, (m // R) * k * 2, bw, topo, sub)
    t = [land[q] for q in order[:R2 - sub]]
    assert t == sorted(t)
    if R > 1:
        last = order[R2 - sub - 1]
        assert all(s == 1 for q, s in enumerate(split) if q != last)
        chosen = pred[SPLITS.index(sub)][SPLITS.index(split[last])]
        assert chosen > max(land)
