"""GPU row swaps at the pages' dry-run geometry (384 experts, 295 hot / 89
cold; small expert shapes so the test is quick): five ordered swaps leave the
layer output bit-identical and every expert's bytes where the map says; a map
flip without the copies diverges; a stale swap is refused with nothing
enqueued; a long swap sequence undone in reverse restores the banks byte for
byte. Every step is mirrored on host byte arrays by the oracle's swap."""
import numpy as np
import pytest
import torch

import expert_weight_residency_amd as moe
import oracle
import synth
from gpu_util import device_bank, host_bank, pinned_bank, run_layer

pytestmark = pytest.mark.gpu

E, N_COLD, K, H, I, SEED = 384, 89, 6, 256, 128, 77


def _setup(cold_at="pinned"):
    rm, ho, co = synth.fitted_map(E, N_COLD, SEED, 0)
    hot_h, cold_h = host_bank(ho, SEED, 0, H, I), host_bank(co, SEED, 0, H, I)
    hot = device_bank(hot_h)
    if cold_at == "pinned":
        cold = pinned_bank(cold_h)
    elif cold_at == "device":
        cold = device_bank(cold_h)
    else:  # weights pinned on the host, scales in HBM
        w, s = pinned_bank(cold_h), device_bank(cold_h)
        cold = moe.Bank(w.w13, s.s13, w.w2, s.s2, on_host=moe.BANK_HOST_WEIGHTS)
    ob_hot, ob_cold = oracle.Bank(**{k: v.copy() for k, v in hot_h.items()}), \
        oracle.Bank(**{k: v.copy() for k, v in cold_h.items()})
    rm_dev = torch.from_numpy(rm.copy()).cuda()
    staging = torch.empty(moe.moe_expert_bytes(H, I), dtype=torch.uint8, device="cuda")
    return rm, ho.copy(), co.copy(), hot, cold, ob_hot, ob_cold, rm_dev, staging


def _bank_equals(gbank, obank):
    return all(np.array_equal(getattr(gbank, t).cpu().numpy(), getattr(obank, t))
               for t in synth.TENSORS)


def _layer(hot, cold, rm_np, ids, w, x):
    return run_layer(hot, cold, rm_np, ids, w, x, H, I)[1]


@pytest.mark.parametrize("cold_at", ["pinned", "device", "host_weights"],
                         ids=["cold_pinned", "cold_device", "cold_host_weights"])
def test_five_ordered_swaps(cold_at):
    rm, ho, co, hot, cold, ob_hot, ob_cold, rm_dev, staging = _setup(cold_at)
    rng = np.random.default_rng(1)
    pairs = [(int(rng.integers(len(ho))), int(rng.integers(len(co)))) for _ in range(5)]
    ids, w = synth.skewed_routing(16, K, E, SEED, 0, 0)
    for n, (a, b) in enumerate(pairs):          # the swapped experts are routed to
        ids[n, 0], ids[n, 1] = ho[a], co[b]
    x = synth.activations(16, H, SEED)
    out0 = _layer(hot, cold, rm, ids, w, x)
    rm_host = rm.copy()
    for n, (a, b) in enumerate(pairs):
        e_h, e_c = int(ho[a]), int(co[b])
        moe.moe_swap_rows(hot, cold, a, b, e_h, e_c, rm_dev, ho, co, staging, H, I)
        oracle.swap_rows(ob_hot, ob_cold, a, b, e_h, e_c, rm_host, *_mirrors(ho, co, a, b, e_h, e_c))
        torch.cuda.synchronize()
        assert np.array_equal(rm_dev.cpu().numpy(), rm_host), n
        assert _bank_equals(hot, ob_hot) and _bank_equals(cold, ob_cold), n
        assert ho[a] == e_c and co[b] == e_h
        out = _layer(hot, cold, rm_dev.cpu().numpy(), ids, w, x)
        assert np.array_equal(out, out0), n


def _mirrors(ho, co, a, b, e_h, e_c):
    """The oracle swap checks and updates its own owner mirrors; give it copies
    holding the pre-swap owners (the ABI call already updated ho / co)."""
    oh, oc = ho.copy(), co.copy()
    oh[a], oc[b] = e_h, e_c
    return oh, oc


def test_misordered_flip_diverges():
    rm, ho, co, hot, cold, _, _, rm_dev, _ = _setup()
    ids, w = synth.skewed_routing(16, K, E, SEED, 0, 1)
    ids[0, 0], ids[1, 0] = ho[3], co[2]
    x = synth.activations(16, H, SEED, step=1)
    out0 = _layer(hot, cold, rm, ids, w, x)
    bad = rm.copy()
    bad[ho[3]], bad[co[2]] = -1 - 2, 3          # flip the map, skip the copies
    out1 = _layer(hot, cold, bad, ids, w, x)
    assert not np.array_equal(out0, out1)


def test_stale_swap_refused_nothing_enqueued():
    rm, ho, co, hot, cold, ob_hot, ob_cold, rm_dev, staging = _setup()
    ho_before, co_before = ho.copy(), co.copy()
    with pytest.raises(moe.MoeStale):
        moe.moe_swap_rows(hot, cold, 4, 7, int(ho[5]), int(co[7]), rm_dev, ho, co, staging, H, I)
    torch.cuda.synchronize()
    assert np.array_equal(ho, ho_before) and np.array_equal(co, co_before)
    assert np.array_equal(rm_dev.cpu().numpy(), rm)
    assert _bank_equals(hot, ob_hot) and _bank_equals(cold, ob_cold)


def test_swap_round_trip_restores_banks():
    rm, ho, co, hot, cold, ob_hot, ob_cold, rm_dev, staging = _setup()
    rng = np.random.default_rng(2)
    log = []
    for _ in range(60):
        a, b = int(rng.integers(len(ho))), int(rng.integers(len(co)))
        log.append((a, b, int(ho[a]), int(co[b])))
        moe.moe_swap_rows(hot, cold, a, b, int(ho[a]), int(co[b]), rm_dev, ho, co, staging, H, I)
    for a, b, e_h, e_c in reversed(log):
        moe.moe_swap_rows(hot, cold, a, b, e_c, e_h, rm_dev, ho, co, staging, H, I)
    torch.cuda.synchronize()
    assert np.array_equal(rm_dev.cpu().numpy(), rm)
    assert _bank_equals(hot, ob_hot) and _bank_equals(cold, ob_cold)


def test_usage_counts_snapshot():
    table = torch.arange(40 * E, dtype=torch.int32, device="cuda").reshape(40, E)
    dst = torch.empty((40, E), dtype=torch.int32, pin_memory=True)
    moe.moe_usage_counts(table, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.numpy(), table.cpu().numpy())
    assert dst.numel() * 4 == 61_440


def test_refit_from_device_counts():
    """A count-only profile on the positional boot map (~23% of picks cold),
    counted on the device by moe_route_split, equals the host's count of the
    same picks; the map fitted to it (mapfit) is applied with moe_swap_rows
    and leaves the layer output bit-identical, the banks byte-equal to the
    oracle's swaps, and far fewer picks cold."""
    from expert_weight_residency_amd import mapfit
    from expert_weight_residency_amd.layer import LayerBuffers
    from expert_weight_residency_amd.policy import swaps_to
    rm, ho, co = synth.positional_map(E, N_COLD)
    hot_h, cold_h = host_bank(ho, SEED, 0, H, I), host_bank(co, SEED, 0, H, I)
    hot, cold = device_bank(hot_h), pinned_bank(cold_h)
    ob_hot = oracle.Bank(**{k: v.copy() for k, v in hot_h.items()})
    ob_cold = oracle.Bank(**{k: v.copy() for k, v in cold_h.items()})
    rm_dev = torch.from_numpy(rm.copy()).cuda()
    staging = torch.empty(moe.moe_expert_bytes(H, I), dtype=torch.uint8, device="cuda")
    counts = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    snap = torch.empty((1, E), dtype=torch.int32, pin_memory=True)
    T, steps = 16, 40
    bufs = LayerBuffers.allocate(T, K, H, I, len(ho), len(co))
    host_counts = np.zeros((1, E), np.int64)
    moe.moe_usage_counts(counts, snap)
    torch.cuda.synchronize()
    before = snap.numpy().copy()
    for s in range(steps):
        ids, _ = synth.skewed_routing(T, K, E, SEED, 0, 100 + s)
        np.add.at(host_counts[0], ids.ravel(), 1)
        moe.moe_route_split(torch.from_numpy(ids).cuda(), rm_dev, len(ho), len(co),
                            bufs.hot_split, bufs.cold_split, bufs.n_invalid, counts[0], 256)
    moe.moe_usage_counts(counts, snap)
    torch.cuda.synchronize()
    prof = mapfit.counts_between(before, snap.numpy())
    assert np.array_equal(prof, host_counts)
    fitted = mapfit.fit_maps(prof, N_COLD, top_k=K, min_tokens=T * steps)[0]
    boot_share = host_counts[0, co].sum() / host_counts.sum()

    ids, w = synth.skewed_routing(T, K, E, SEED, 0, 1)
    x = synth.activations(T, H, SEED, step=1)
    out0 = _layer(hot, cold, rm, ids, w, x)
    rm_host = rm.copy()
    props = swaps_to([ho], [co], [fitted.hot_owner])
    assert len(props) == mapfit.changed_cold(co, fitted.cold_owner) > 0
    for sw in props:
        a, b, e_h, e_c = sw.hot_row, sw.cold_row, sw.expect_hot_expert, sw.expect_cold_expert
        moe.moe_swap_rows(hot, cold, a, b, e_h, e_c, rm_dev, ho, co, staging, H, I)
        oracle.swap_rows(ob_hot, ob_cold, a, b, e_h, e_c, rm_host, *_mirrors(ho, co, a, b, e_h, e_c))
    torch.cuda.synchronize()
    assert np.array_equal(rm_dev.cpu().numpy(), rm_host)
    assert set(ho.tolist()) == set(fitted.hot_owner.tolist())
    assert _bank_equals(hot, ob_hot) and _bank_equals(cold, ob_cold)
    assert np.array_equal(_layer(hot, cold, rm_host, ids, w, x), out0)
    fitted_share = host_counts[0, co].sum() / host_counts.sum()
    print(f"refit: {len(props)} swaps, cold share {boot_share:.3f} -> {fitted_share:.3f}",
          flush=True)
    assert fitted_share < 0.25 * boot_share


def test_five_swaps_full_expert_size():
    """Five ordered swaps at full expert size (H = 4096, I = 2880: 18,800,640
    bytes per expert) between a 295-row hot bank in HBM and an 89-row cold bank
    in pinned host memory, the 384-expert fitted map of the pages' dry run
    ("vLLM: Pin Hot Experts", "Closed, September 17 evening", E4/E4b at real
    geometry). After each swap both swapped experts' bytes are exactly the
    generator's bytes for those experts at the rows the map names, the rows'
    neighbours are untouched, and the device map equals the host's. Prints the
    time per swap (12 copies through the staging row + the map write)."""
    Hf, If = 4096, 2880
    rm, ho, co = synth.fitted_map(E, N_COLD, SEED, 0)
    shapes = synth.tensor_shapes(len(ho), Hf, If)
    hot = moe.Bank(*[torch.empty(s, dtype=torch.uint8, device="cuda") for s in shapes.values()])
    synth.fill_bank_device(hot.tensors(), torch.from_numpy(ho).cuda(), SEED, 0, Hf, If)
    cshapes = synth.tensor_shapes(len(co), Hf, If)
    cold = moe.Bank(*[torch.empty(s, dtype=torch.uint8, pin_memory=True)
                      for s in cshapes.values()], on_host=True)
    synth.fill_bank_host(cold.tensors(), co, SEED, 0, Hf, If)
    rm_dev = torch.from_numpy(rm.copy()).cuda()
    rm_host = rm.copy()
    staging = torch.empty(moe.moe_expert_bytes(Hf, If), dtype=torch.uint8, device="cuda")
    assert staging.numel() == 18_800_640
    torch.cuda.synchronize()

    def row_bytes(e):
        m = int(rm_host[e])
        b, r = (hot, m) if m >= 0 else (cold, -1 - m)
        return [getattr(b, t)[r].cpu().numpy().tobytes() for t in synth.TENSORS]

    def expected(e):
        one = synth.make_bank_host([e], SEED, 0, Hf, If)
        return [one[t][0].tobytes() for t in synth.TENSORS]

    rng = np.random.default_rng(11)
    times = []
    for n in range(5):
        a, b = int(rng.integers(len(ho))), int(rng.integers(len(co)))
        e_h, e_c = int(ho[a]), int(co[b])
        nb_h = hot.w13[(a + 1) % len(ho)].cpu().numpy().tobytes()
        nb_c = cold.w2[(b + 1) % len(co)].numpy().tobytes()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        moe.moe_swap_rows(hot, cold, a, b, e_h, e_c, rm_dev, ho, co, staging, Hf, If)
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1) * 1e3)
        rm_host[e_h], rm_host[e_c] = -1 - b, a
        assert np.array_equal(rm_dev.cpu().numpy(), rm_host), n
        assert ho[a] == e_c and co[b] == e_h
        assert row_bytes(e_h) == expected(e_h), (n, e_h)
        assert row_bytes(e_c) == expected(e_c), (n, e_c)
        assert hot.w13[(a + 1) % len(ho)].cpu().numpy().tobytes() == nb_h
        assert cold.w2[(b + 1) % len(co)].numpy().tobytes() == nb_c
    print(f"full-size swap: {np.round(times, 1)} us each "
          f"({2 * 18_800_640 / (np.median(times) * 1e-6) / 1e9:.1f} GB/s over the host link "
          "counting both directions)", flush=True)
