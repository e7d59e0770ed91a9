"""The synthetic generators: determinism and the routing statistics they are
shaped after."""
import json
import os

import numpy as np

import synth


def test_weight_streams_deterministic_and_keyed():
    a = synth.make_bank_host([3, 5], seed=1, layer=2, H=256, I=128)
    b = synth.make_bank_host([5, 3], seed=1, layer=2, H=256, I=128)
    for t in synth.TENSORS:
        assert np.array_equal(a[t][0], b[t][1]) and np.array_equal(a[t][1], b[t][0])
        assert not np.array_equal(a[t][0], a[t][1])
    c = synth.make_bank_host([3], seed=1, layer=3, H=256, I=128)
    assert not np.array_equal(a["w13"][0], c["w13"][0])


def test_weight_byte_distributions():
    bank = synth.make_bank_host([0, 1, 2, 3], seed=7, layer=0, H=1024, I=512)
    w = bank["w13"].reshape(-1)
    counts = np.bincount(w, minlength=256)
    assert counts.min() > 0.8 * w.size / 256 and counts.max() < 1.2 * w.size / 256
    s = np.concatenate([bank["s13"].reshape(-1), bank["s2"].reshape(-1)])
    assert set(np.unique(s).tolist()) == {124, 125, 126, 127, 128}
    frac = np.bincount(s, minlength=129)[124:] / s.size
    assert np.all(np.abs(frac - 0.2) < 0.01)


def test_wide_scale_window():
    bank = synth.make_bank_host([0], seed=7, layer=0, H=4096, I=256, scale_lo=0, scale_cnt=255)
    s = bank["s13"].reshape(-1)
    assert s.min() == 0 and s.max() == 254


def test_activation_stats():
    x = synth.activations(64, 4096, seed=3)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(xf.mean()) < 0.01 and abs(xf.std() - 1) < 0.01
    assert np.array_equal(x, synth.activations(64, 4096, seed=3))


def test_routing_skew_matches_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "routing_skew.json")))
    E, k = 384, 6
    ginis, tops, cold, pos = [], [], [], []
    rp, _, _ = synth.positional_map(E, 89)
    for layer in range(3):
        rm, _, _ = synth.fitted_map(E, 89, 1, layer)
        cnt = np.zeros(E)
        for step in range(120):
            ids, _ = synth.skewed_routing(16, k, E, 1, layer, step)
            cnt += np.bincount(ids.ravel(), minlength=E)
            cold.append((rm[ids] < 0).mean())
            pos.append((rp[ids] < 0).mean())
        ginis.append(synth.gini(cnt))
        tops.append([synth.top_share(cnt, f) for f in (0.25, 0.5, 0.73)])
    assert abs(np.mean(ginis) - g["mean_gini"]) < 0.03
    t = np.mean(tops, axis=0)
    assert abs(t[0] - g["top_25pct_share"]) < 0.05
    assert abs(t[1] - g["top_50pct_share"]) < 0.03
    assert abs(t[2] - g["top_73pct_share"]) < 0.02
    lo, hi = g["fitted_cold_share_range"]
    assert lo <= np.mean(cold) <= hi
    # positional share varies by layer (the permutation decides which ranks land
    # on the last ids); its expectation over the 40 layers is exact from the pmf
    pmf = synth.rank_pmf(E)
    shares = []
    for layer in range(40):
        rank_of = np.empty(E, int)
        rank_of[synth.layer_permutation(E, 1, layer)] = np.arange(E)
        shares.append(pmf[rank_of[E - 89:]].sum())
    lo, hi = g["positional_cold_share_range"]
    assert lo <= np.mean(shares) <= hi
    assert abs(np.mean(pos) - np.mean(shares[:3])) < 0.02   # sampling agrees with the pmf


def test_verify_window_routing_matches_pages(golden_dir):
    """The verify-window generator touches as many experts per window as the
    pages measured (within 6%), independent tokens touch far more, and its
    pick distribution keeps the decode skew (Gini, fitted cold share)."""
    g = json.load(open(os.path.join(golden_dir, "verify_window_touched_set.json")))
    skew = json.load(open(os.path.join(golden_dir, "routing_skew.json")))
    E, k = 384, g["top_k"]
    want = {int(w): v for w, v in g["unique_experts_by_window_tokens"].items()}
    for w, v in want.items():
        got = np.mean([len(np.unique(synth.window_routing(w, k, E, 3, 0, step, window=w)[0]))
                       for step in range(400)])
        assert abs(got - v) <= 0.06 * v, (w, got, v)
        if w >= 4:  # independent tokens: at least 25% more
            iid = np.mean([len(np.unique(synth.skewed_routing(w, k, E, 3, 0, step)[0]))
                           for step in range(200)])
            assert iid > 1.25 * v, (w, iid)
    rm, _, _ = synth.fitted_map(E, 89, 3, 0)
    cnt, cold = np.zeros(E), []
    for step in range(300):
        ids, wts = synth.window_routing(112, k, E, 3, 0, step)
        cnt += np.bincount(ids.ravel(), minlength=E)
        cold.append((rm[ids] < 0).mean())
        assert ids.shape == (112, k) and np.allclose(wts.sum(axis=1), 1, atol=1e-6)
        assert all(len(set(r)) == k for r in ids)  # distinct picks per token
    assert abs(synth.gini(cnt) - skew["mean_gini"]) < 0.04
    lo, hi = skew["fitted_cold_share_range"]
    assert lo <= np.mean(cold) <= hi
    a, _ = synth.window_routing(14, k, E, 3, 0, 5)
    b, _ = synth.window_routing(14, k, E, 3, 0, 5)
    assert np.array_equal(a, b)  # deterministic


def test_maps_are_bijections():
    for rm, ho, co in (synth.fitted_map(384, 89, 1, 0), synth.positional_map(384, 89),
                       synth.random_map(16, 4, 3), synth.all_hot_map(8)):
        E = len(rm)
        assert len(ho) + len(co) == E
        assert np.all(np.diff(ho) > 0) and (len(co) < 2 or np.all(np.diff(co) > 0))
        assert np.array_equal(rm[ho], np.arange(len(ho)))
        assert np.array_equal(-1 - rm[co], np.arange(len(co)))
