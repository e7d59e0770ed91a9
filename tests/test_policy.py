"""Host-side swap policy and runtime control ("We Built the Counter", sections
2 and 9): the decaying average against its closed form, counter wrap-around,
the proposal rules (minimum average, hysteresis, per-layer and per-barrier
budgets, largest gain first, rows and experts named for the stale check),
freeze, the restore to the boot-time hot sets, the JSON control file and the
JSONL telemetry. CPU only."""
import json

import numpy as np
import pytest

from expert_weight_residency_amd.policy import (AdaptivePolicy, PolicyConfig, RuntimeControl,
                                                Telemetry, restore_swaps)


def apply_swap(hot_owner, cold_owner, sw):
    """What moe_swap_rows does to the owner mirrors (after its stale check)."""
    ho, co = hot_owner[sw.layer], cold_owner[sw.layer]
    assert ho[sw.hot_row] == sw.expect_hot_expert and co[sw.cold_row] == sw.expect_cold_expert
    ho[sw.hot_row], co[sw.cold_row] = sw.expect_cold_expert, sw.expect_hot_expert


def test_average_matches_closed_form():
    pol = AdaptivePolicy(1, 4)
    d = pol.decay
    assert d == pytest.approx(0.5 ** (64 / 500))
    counts = np.zeros((1, 4), np.int64)
    pol.observe(counts)  # first read only sets the reference
    assert not pol.avg.any()
    delta = np.array([[10, 0, 3, 7]])
    for n in range(1, 21):
        counts = counts + delta
        pol.observe(counts)
        np.testing.assert_allclose(pol.avg, delta * (1 - d ** n), rtol=1e-12)


def test_half_life():
    cfg = PolicyConfig(read_every=50, half_life=500)
    pol = AdaptivePolicy(1, 1, cfg)
    pol.observe(np.zeros((1, 1)))
    pol.avg[:] = 64.0
    for _ in range(10):  # 10 reads x 50 steps = one half-life, no new counts
        pol.observe(np.zeros((1, 1)))
    assert pol.avg[0, 0] == pytest.approx(32.0)


def test_counter_wraps_modulo_2_32():
    pol = AdaptivePolicy(1, 2)
    pol.observe(np.array([[2**31 - 3, 5]], np.int64).astype(np.int32))
    nxt = np.array([[-2**31 + 4, 5]], np.int64).astype(np.int32)  # +7 across the int32 wrap
    pol.observe(nxt)
    assert pol.avg[0, 0] == pytest.approx(7 * (1 - pol.decay))
    assert pol.avg[0, 1] == 0


def _policy_with(avgs, cfg=None):
    pol = AdaptivePolicy(len(avgs), len(avgs[0]), cfg)
    pol.avg[:] = np.array(avgs, np.float64)
    return pol


def test_decide_rules():
    # experts 0..5; hot rows hold 0,1,2; cold rows hold 3,4,5
    pol = _policy_with([[0.0, 10.0, 50.0, 20.0, 9.0, 3.0]])
    ho, co = [np.array([0, 1, 2])], [np.array([3, 4, 5])]
    props = pol.decide(ho, co)
    # busiest cold (3: 20) vs idlest hot (0: 0): promoted; next pair (4: 9 vs 1: 10) fails
    # the 1.5x hysteresis
    assert len(props) == 1
    sw = props[0]
    assert (sw.layer, sw.hot_row, sw.cold_row, sw.expect_hot_expert, sw.expect_cold_expert) == \
        (0, 0, 0, 0, 3)
    assert sw.gain == pytest.approx(20.0)
    # minimum average: a cold expert below 8 is never promoted, however idle the hot one
    pol = _policy_with([[0.0, 0.0, 7.9, 7.0]])
    assert pol.decide([np.array([0, 1])], [np.array([2, 3])]) == []


def test_budgets_and_gain_order():
    cfg = PolicyConfig(swaps_per_layer=2, swaps_per_barrier=3)
    # two layers, experts 0..7: hot rows 0..3 idle, cold rows hold busy 4..7
    a0 = [0, 0, 0, 0, 100, 90, 80, 70]
    a1 = [0, 0, 0, 0, 60, 95, 50, 40]
    pol = _policy_with([a0, a1], cfg)
    ho = [np.array([0, 1, 2, 3]), np.array([0, 1, 2, 3])]
    co = [np.array([4, 5, 6, 7]), np.array([4, 5, 6, 7])]
    props = pol.decide(ho, co)
    assert len(props) == 3  # per barrier
    assert [s.gain for s in props] == sorted([s.gain for s in props], reverse=True)
    per_layer = [sum(1 for s in props if s.layer == l) for l in (0, 1)]
    assert max(per_layer) <= 2
    assert [(s.layer, s.expect_cold_expert) for s in props] == [(0, 4), (1, 5), (0, 5)]
    # no row is used twice within a layer
    for l in (0, 1):
        rows = [(s.hot_row, s.cold_row) for s in props if s.layer == l]
        assert len({r for r, _ in rows}) == len(rows) and len({c for _, c in rows}) == len(rows)


def test_freeze():
    pol = _policy_with([[0.0, 50.0]])
    ctl = RuntimeControl(pol)
    ctl.apply({"freeze": True})
    assert pol.decide([np.array([0])], [np.array([1])]) == []
    ctl.apply({"freeze": False})
    assert len(pol.decide([np.array([0])], [np.array([1])])) == 1


def test_restore_to_boot_hot_sets():
    rng = np.random.default_rng(3)
    L, E, R = 3, 24, 18
    boot_hot = [np.sort(rng.permutation(E)[:R]) for _ in range(L)]
    hot = [b.copy() for b in boot_hot]
    cold = [np.setdiff1d(np.arange(E), b) for b in boot_hot]
    # a run of random swaps moves the hot sets away from boot
    for _ in range(40):
        l = int(rng.integers(L))
        r, c = int(rng.integers(R)), int(rng.integers(E - R))
        hot[l][r], cold[l][c] = cold[l][c], hot[l][r]
    moved = sum(len(set(hot[l]) - set(boot_hot[l])) for l in range(L))
    assert moved > 0
    # limited batches, applied and recomputed until none is left
    rounds = 0
    while True:
        props = restore_swaps(hot, cold, boot_hot, limit=4)
        if not props:
            break
        assert len(props) <= 4
        for sw in props:
            apply_swap(hot, cold, sw)
        rounds += 1
    assert rounds >= (moved + 3) // 4
    for l in range(L):
        assert set(hot[l]) == set(boot_hot[l])
        assert set(cold[l]) == set(range(E)) - set(boot_hot[l])
    assert restore_swaps(hot, cold, boot_hot) == []


def test_control_file_and_dump(tmp_path):
    pol = AdaptivePolicy(2, 4)
    path = tmp_path / "ctrl.json"
    ctl = RuntimeControl(pol, str(path))
    assert ctl.poll() is None  # no file yet
    path.write_text(json.dumps({"freeze": True, "swaps_per_barrier": "5", "min_avg": 2,
                                "counting": False, "bogus": 1}))
    assert ctl.poll() == ["bogus"]
    assert pol.frozen and not ctl.counting
    assert pol.cfg.swaps_per_barrier == 5 and isinstance(pol.cfg.swaps_per_barrier, int)
    assert pol.cfg.min_avg == 2.0
    assert ctl.poll() is None  # unchanged file is not re-read
    dump = tmp_path / "counts.json"
    ctl.apply({"dump_counts": str(dump), "restore_map": True})
    assert ctl.restore_pending
    snap = np.arange(8, dtype=np.int32).reshape(2, 4)
    assert ctl.maybe_dump(snap)
    assert json.loads(dump.read_text()) == snap.tolist()
    assert not ctl.maybe_dump(snap)  # one dump per request


def test_telemetry_jsonl(tmp_path):
    path = tmp_path / "t.jsonl"
    tel = Telemetry(str(path))
    tel.log(step=64, swaps=2, stale=0)
    tel.log(step=128, swaps=0, stale=1, frozen=True)
    lines = [json.loads(x) for x in path.read_text().splitlines()]
    assert lines == [{"step": 64, "swaps": 2, "stale": 0},
                     {"step": 128, "swaps": 0, "stale": 1, "frozen": True}]
    assert tel.records == lines
