"""Off-line map fitting (expert_weight_residency_amd/mapfit.py), CPU only.

Pins: brute force over every cold set of tiny layers (the fitted cold set
carries the fewest selections, ties broken by expert id), the row-map
encoding of the input generators' independent map builder, the exact map
from expected counts of the skewed routing distribution (the generators'
fitted map), the 32-bit wrap of counter snapshots, weighted mixing, the
token floor, and swaps that turn live banks into the fitted hot sets."""
import itertools

import numpy as np
import pytest

import synth
from expert_weight_residency_amd import mapfit
from expert_weight_residency_amd.policy import swaps_to


def _apply(ho, co, swaps):
    ho, co = [h.copy() for h in ho], [c.copy() for c in co]
    for sw in swaps:
        l = sw.layer
        assert ho[l][sw.hot_row] == sw.expect_hot_expert
        assert co[l][sw.cold_row] == sw.expect_cold_expert
        ho[l][sw.hot_row], co[l][sw.cold_row] = sw.expect_cold_expert, sw.expect_hot_expert
    return ho, co


def test_brute_force_tiny_layers():
    rng = np.random.default_rng(5)
    for trial in range(200):
        E = int(rng.integers(2, 8))
        n_cold = int(rng.integers(0, E + 1))
        c = rng.integers(0, 4, size=(1, E))  # small values: many ties
        m = mapfit.fit_maps(c, n_cold)[0]
        best = None
        for cold in itertools.combinations(range(E), n_cold):
            load = int(c[0, list(cold)].sum())
            # among equal loads prefer the cold set whose ids are highest
            key = (load, tuple(sorted((-e for e in cold))))
            if best is None or key < best[0]:
                best = (key, cold)
        assert sorted(m.cold_owner.tolist()) == sorted(best[1]), (c, n_cold)
        assert m.hot_owner.size + m.cold_owner.size == E


def test_row_map_encoding_matches_generator_builder():
    rng = np.random.default_rng(7)
    c = rng.integers(0, 1000, size=(3, 384))
    for m in mapfit.fit_maps(c, 89):
        rm, ho, co = synth.map_from_cold_set(384, m.cold_owner)
        assert np.array_equal(rm, m.row_map)
        assert np.array_equal(ho, m.hot_owner) and np.array_equal(co, m.cold_owner)
        assert np.all(np.diff(m.hot_owner) > 0) and np.all(np.diff(m.cold_owner) > 0)


def test_expected_counts_give_the_generators_fitted_map():
    """Counts proportional to the routing pmf (distinct per expert) put the
    n_cold least probable experts cold, which is what the input generators'
    fitted map holds."""
    E, n_cold, seed = 384, 89, 20260917
    pmf = synth.rank_pmf(E)
    for layer in range(4):
        perm = synth.layer_permutation(E, seed, layer)
        expected = np.empty(E)
        expected[perm] = pmf * 1e6
        m = mapfit.fit_maps(expected[None, :], n_cold)[0]
        rm, _, _ = synth.fitted_map(E, n_cold, seed, layer)
        assert np.array_equal(m.row_map, rm), layer


def test_counts_between_wraps():
    before = np.array([[0x7FFFFFF0, -16, 5]], np.int32)
    after = np.array([[-0x7FFFFFF0, 16, 5]], np.int32)  # both first entries wrapped
    d = mapfit.counts_between(before, after)
    assert d.tolist() == [[0x20, 32, 0]]


def test_weighted_mix():
    a = np.array([[10, 0, 5, 1]])
    b = np.array([[0, 40, 1, 1]])
    assert mapfit.score([a, b], [1.0, 0.25]).tolist() == [[10, 10, 5.25, 1.25]]
    # 0.25 of b: expert 1 ties expert 0 at 10, experts 2 and 3 go cold
    assert mapfit.fit_maps(mapfit.score([a, b], [1.0, 0.25]), 2)[0].cold_owner.tolist() == [2, 3]
    # the tie at 10 sends the higher id (1) cold
    assert mapfit.fit_maps(mapfit.score([a, b], [1.0, 0.25]), 3)[0].cold_owner.tolist() == [1, 2, 3]
    # b alone: expert 0 cold, then the tie of 2 and 3 at 1 sends 3
    assert mapfit.fit_maps(b, 2)[0].cold_owner.tolist() == [0, 3]
    with pytest.raises(ValueError):
        mapfit.score([a, b], [1.0])
    with pytest.raises(ValueError):
        mapfit.score([a, b], [1.0, -1.0])


def test_token_floor():
    c = np.full((2, 8), 600)  # 4800 selections = 800 tokens of top-6 per layer
    mapfit.fit_maps(c, 2, top_k=6, min_tokens=800)
    c[1, 0] -= 1
    with pytest.raises(mapfit.ProfileTooSmall):
        mapfit.fit_maps(c, 2, top_k=6, min_tokens=800)
    assert mapfit.MIN_TOKENS_PER_LAYER == 50_000


def test_cold_share_and_leave_one_out_on_sampled_traffic():
    """Four slices of 2,000 decode tokens of one layer: the fitted map's
    in-sample cold share is the least any 89-expert cold set can give, and
    each held-out slice sees more cold picks than in-sample (small samples
    misjudge the tail), but far fewer than a positional map's."""
    E, k, n_cold, seed = 384, 6, 89, 3
    slices = []
    for i in range(4):
        c = np.zeros((1, E), np.int64)
        for step in range(10):
            ids, _ = synth.skewed_routing(200, k, E, seed, 0, 100 * i + step)
            np.add.at(c[0], ids.ravel(), 1)
        slices.append(c)
    total = mapfit.score(slices)
    maps = mapfit.fit_maps(total, n_cold)
    ins = mapfit.overall_cold_share(total, maps)
    srt = np.sort(total[0])
    assert ins == pytest.approx(srt[:n_cold].sum() / srt.sum())
    loo = mapfit.leave_one_out(slices, n_cold)
    rm_pos, _, co_pos = synth.positional_map(E, n_cold)
    pos = total[0, co_pos].sum() / total.sum()
    assert all(ins <= x < 0.5 * pos for x in loo), (ins, loo, pos)
    assert mapfit.cold_share(total, maps)[0] == pytest.approx(ins)


def test_swaps_to_fitted_map():
    rng = np.random.default_rng(11)
    E, n_cold, L = 64, 16, 3
    rm0, ho0, co0 = synth.random_map(E, n_cold, 1)
    ho = [rng.permutation(ho0).astype(np.int32) for _ in range(L)]  # rows in any order
    co = [rng.permutation(co0).astype(np.int32) for _ in range(L)]
    maps = mapfit.fit_maps(rng.integers(0, 100, size=(L, E)), n_cold)
    props = swaps_to(ho, co, [m.hot_owner for m in maps])
    for l in range(L):
        n = sum(1 for p in props if p.layer == l)
        assert n == mapfit.changed_cold(co[l], maps[l].cold_owner)
    ho2, co2 = _apply(ho, co, props)
    for l in range(L):
        assert set(ho2[l].tolist()) == set(maps[l].hot_owner.tolist())
        assert set(co2[l].tolist()) == set(maps[l].cold_owner.tolist())
    assert swaps_to(ho2, co2, [m.hot_owner for m in maps]) == []
    # a limit takes a prefix; the rest follows on the next call
    first = swaps_to(ho, co, [m.hot_owner for m in maps], limit=5)
    assert len(first) == min(5, len(props))
    with pytest.raises(ValueError):
        swaps_to(ho, co, [m.hot_owner[:-1] for m in maps])
