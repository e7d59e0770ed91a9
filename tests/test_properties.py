"""Property tests (hypothesis) on random tiny shapes, CPU only.

Invariants that hold for any input, checked on generated cases:
  - the oracle's residency split partitions the picks: every valid pick lands
    in exactly one bank row, invalid picks are counted, rows ascend, slots
    ascend within a row, and the split of the identity map is a permutation
    of the split of any other map relabelled through it;
  - the oracle's finalize with k = 1 and weight 1 returns its input, with
    weight 0 returns +0 for every finite row (fmaf(0, y, +0) = +0, also for
    negative y), and scales by powers of two exactly (no rounding);
  - the usage counter adds T*k per decode-sized step and nothing above 256
    tokens;
  - a fitted map's cold set carries no more selections than any other cold
    set of its size, and the swaps to it leave exactly its hot set.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import synth
from expert_weight_residency_amd import mapfit
from expert_weight_residency_amd.policy import swaps_to

SETTINGS = settings(max_examples=80, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def split_case(draw):
    E = draw(st.integers(1, 24))
    k = draw(st.integers(1, min(E, 4)))
    T = draw(st.integers(0, 12))
    n_cold = draw(st.integers(0, E))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    row_map, ho, co = synth.random_map(E, n_cold, seed)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, k), np.int32)
    if T and draw(st.booleans()):
        ids[rng.integers(T), rng.integers(k)] = draw(st.sampled_from([-1, E, E + 7]))
    return E, k, T, row_map, len(ho), len(co), ids


@SETTINGS
@given(split_case())
def test_split_partitions_picks(case):
    E, k, T, row_map, n_hot, n_cold, ids = case
    res = oracle.route_split(ids, row_map, n_hot, n_cold)
    flat = ids.reshape(-1)
    seen = np.zeros(T * k, np.int64)
    for name, n_rows, sign in (("hot", n_hot, 1), ("cold", n_cold, -1)):
        active, off, slots = res[name]
        assert np.all(np.diff(active) > 0) and np.all((active >= 0) & (active < max(n_rows, 1)))
        assert off[0] == 0 and np.all(np.diff(off) > 0) and off[-1] == len(slots)
        for a, r in enumerate(active):
            sl = slots[off[a]:off[a + 1]]
            assert np.all(np.diff(sl) > 0)
            for s in sl:
                m = row_map[flat[s]]
                assert (m == r) if sign > 0 else (m == -1 - r)
            seen[sl] += 1
    valid = (flat >= 0) & (flat < E)
    assert np.all(seen[valid] == 1) and np.all(seen[~valid] == 0)
    assert res["n_invalid"] == int(np.count_nonzero(~valid))


@SETTINGS
@given(split_case())
def test_split_under_relabelled_map(case):
    """The picks each expert receives do not depend on where the map puts it."""
    E, k, T, row_map, n_hot, n_cold, ids = case
    all_map, _, _ = synth.all_hot_map(E)
    a = oracle.route_split(ids, row_map, n_hot, n_cold)
    b = oracle.route_split(ids, all_map, E, 0)
    per_expert_a, per_expert_b = {}, {}
    for name, sign in (("hot", 1), ("cold", -1)):
        active, off, slots = a[name]
        for i, r in enumerate(active):
            e = int(np.nonzero(row_map == (r if sign > 0 else -1 - r))[0][0])
            per_expert_a[e] = slots[off[i]:off[i + 1]].tolist()
    active, off, slots = b["hot"]
    for i, r in enumerate(active):
        per_expert_b[int(r)] = slots[off[i]:off[i + 1]].tolist()
    assert per_expert_a == per_expert_b


@SETTINGS
@given(st.integers(1, 6), st.integers(1, 40), st.integers(0, 2**31 - 1))
def test_finalize_identities(T, H, seed):
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal((T, 1, H)) * 10.0 ** rng.integers(-3, 4, (T, 1, 1))).astype(np.float32)
    Yb = oracle.f32_to_bf16(y)
    one = np.ones((T, 1), np.float32)
    assert np.array_equal(oracle.finalize(Yb, one), Yb.reshape(T, H))
    zero = oracle.finalize(Yb, np.zeros((T, 1), np.float32))
    assert np.all(zero == 0)  # fmaf(0, y, +0) is +0 for every finite y
    e = int(rng.integers(-4, 5))
    scaled = oracle.finalize(Yb, np.full((T, 1), 2.0 ** e, np.float32))
    expect = oracle.f32_to_bf16(oracle.bf16_to_f32(Yb.reshape(T, H)) * np.float32(2.0 ** e))
    assert np.array_equal(scaled, expect)


@SETTINGS
@given(st.integers(1, 300), st.integers(1, 6), st.integers(0, 2**31 - 1))
def test_usage_counter_totals(T, k, seed):
    E = 24
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    before = rng.integers(-2**31, 2**31 - 1, E).astype(np.int32)
    after = oracle.usage_count(before, ids, E)
    delta = (after.astype(np.int64) - before.astype(np.int64)) & 0xFFFFFFFF
    assert int(delta.sum()) == (T * k if T <= 256 else 0)


@SETTINGS
@given(st.integers(2, 10), st.integers(0, 2**31 - 1), st.data())
def test_fitted_map_minimal_and_reachable(E, seed, data):
    n_cold = data.draw(st.integers(0, E))
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 6, size=(2, E))
    maps = mapfit.fit_maps(counts, n_cold)
    for layer, m in enumerate(maps):
        load = counts[layer, m.cold_owner].sum()
        other = rng.choice(E, n_cold, replace=False)
        assert load <= counts[layer, other].sum()
        assert load == np.sort(counts[layer])[:n_cold].sum()
    rm, ho, co = synth.random_map(E, n_cold, seed)
    hot = [ho.copy(), ho.copy()]
    cold = [co.copy(), co.copy()]
    for sw in swaps_to(hot, cold, [m.hot_owner for m in maps]):
        hot[sw.layer][sw.hot_row], cold[sw.layer][sw.cold_row] = \
            sw.expect_cold_expert, sw.expect_hot_expert
    for layer, m in enumerate(maps):
        assert sorted(hot[layer].tolist()) == m.hot_owner.tolist()
