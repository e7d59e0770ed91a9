"""GPU parity at the full expert shapes: 384 experts, top-6, H=4096, I=2880,
295 hot rows in HBM and 89 cold rows in pinned host memory read in place.
Decode (16 and 7 tokens) is checked on every slot; 112 tokens with the
positional map (staged == in place bitwise) and the 4096-token prefill chunk
on sampled slots and tokens."""
import numpy as np
import pytest
import torch

import expert_weight_residency_amd as moe
import oracle
import synth
from gpu_util import MAX_REL, REL_L2, empty_bank_host, oracle_bank, rel_errors, run_layer

pytestmark = pytest.mark.gpu

E, K, H, I = 384, 6, 4096, 2880
SEED = 20260917


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def banks():
    assert torch.cuda.is_available()
    rm, ho, co = synth.fitted_map(E, 89, SEED, 0)
    hot = empty_bank_host(len(ho), H, I, device="cuda")
    owners = torch.from_numpy(ho).cuda()
    synth.fill_bank_device(hot.tensors(), owners, SEED, 0, H, I)
    cold = empty_bank_host(len(co), H, I, pinned=True)
    synth.fill_bank_host(cold.tensors(), co, SEED, 0, H, I)
    torch.cuda.synchronize()
    log("full-shape banks filled")
    yield rm, ho, co, hot, cold
    del hot, cold
    torch.cuda.empty_cache()


def _oracle_for(ids, w, x, tokens=None):
    """Oracle rows for the given tokens (all if None): builds host copies of
    just the experts those tokens touch."""
    if tokens is None:
        tokens = np.arange(ids.shape[0])
    sub_ids = ids[tokens]
    U = np.unique(sub_ids)
    ob = oracle_bank(synth.make_bank_host(U, SEED, 0, H, I))
    rm_o = np.full(E, -(10 ** 6), np.int32)
    rm_o[U] = np.arange(len(U), dtype=np.int32)
    Yr, outr, bad = oracle.moe_layer(ob, None, rm_o, sub_ids, w[tokens], x[tokens], H, I)
    assert bad == 0
    return Yr, outr


def test_device_fill_matches_host_generator(banks):
    rm, ho, co, hot, cold = banks
    for r in (0, 147, len(ho) - 1):
        ref = synth.make_bank_host([ho[r]], SEED, 0, H, I)
        for t in synth.TENSORS:
            assert np.array_equal(getattr(hot, t)[r].cpu().numpy(), ref[t][0]), (r, t)


def test_decode_T16_every_slot(banks):
    rm, ho, co, hot, cold = banks
    ids, w = synth.skewed_routing(16, K, E, SEED, 0, 0)
    x = synth.activations(16, H, SEED)
    log(f"T=16: {len(np.unique(ids[rm[ids] >= 0]))} hot, {len(np.unique(ids[rm[ids] < 0]))} cold experts")
    Y, out, ninv = run_layer(hot, cold, rm, ids, w, x, H, I)
    assert ninv == 0
    Yr, outr = _oracle_for(ids, w, x)
    e_y, e_o = rel_errors(Y, Yr.reshape(-1, H)), rel_errors(out, outr)
    log(f"  Y {e_y}  out {e_o}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL


def test_decode_split_equals_all_hot_at_full_shape(banks):
    rm, ho, co, hot, cold = banks
    ids, w = synth.skewed_routing(16, K, E, SEED, 0, 1)
    # make sure several picks are cold
    ids[0, :3] = co[:3]
    ids[5, 1] = co[10]
    x = synth.activations(16, H, SEED, step=1)
    Ys, outs, _ = run_layer(hot, cold, rm, ids, w, x, H, I)
    allb = empty_bank_host(E, H, I, device="cuda")
    synth.fill_bank_device(allb.tensors(), torch.arange(E, dtype=torch.int32, device="cuda"), SEED,
                           0, H, I)
    all_map, _, _ = synth.all_hot_map(E)
    Yu, outu, _ = run_layer(allb, None, all_map, ids, w, x, H, I)
    del allb
    torch.cuda.empty_cache()
    assert np.array_equal(Ys, Yu)
    assert np.array_equal(outs, outu)


@pytest.mark.parametrize("routing", ["independent", "window"])
def test_decode_T7_every_slot(banks, routing):
    """One layer call of the 40-layer step (7 tokens: a verify window), with
    tokens routed independently or correlated within the window (fewer
    distinct experts, more tokens per expert)."""
    rm, ho, co, hot, cold = banks
    gen = synth.window_routing if routing == "window" else synth.skewed_routing
    ids, w = gen(7, K, E, SEED, 0, 3)
    x = synth.activations(7, H, SEED, step=3)
    Y, out, ninv = run_layer(hot, cold, rm, ids, w, x, H, I)
    assert ninv == 0
    Yr, outr = _oracle_for(ids, w, x)
    e_y, e_o = rel_errors(Y, Yr.reshape(-1, H)), rel_errors(out, outr)
    log(f"T=7 {routing}: {len(np.unique(ids))} experts, Y {e_y}  out {e_o}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL
    for s in range(7 * K):
        assert rel_errors(Y[s], Yr.reshape(-1, H)[s])[0] <= REL_L2, s


def test_decode_T112_positional_map_staged(banks):
    """High-concurrency step (112 tokens) with the positional map (the last 89
    ids cold, ~23% of picks): the token-tiled kernels for both banks (2.3
    and 7.6 picks per row); the cold path staged into HBM on a side stream
    gives the bits of the in-place cold path; sampled tokens (incl. cold
    picks) against the oracle."""
    _, ho, co, hot, cold = banks
    T = 112
    rm, ho_p, co_p = synth.positional_map(E, 89)
    # the fixture's banks hold the fitted map's rows: refill for the positional one
    hot_p = empty_bank_host(len(ho_p), H, I, device="cuda")
    synth.fill_bank_device(hot_p.tensors(), torch.from_numpy(ho_p).cuda(), SEED, 0, H, I)
    cold_p = empty_bank_host(len(co_p), H, I, pinned=True)
    synth.fill_bank_host(cold_p.tensors(), co_p, SEED, 0, H, I)
    ids, w = synth.skewed_routing(T, K, E, SEED, 0, 11)
    x = synth.activations(T, H, SEED, step=11)
    n_cold_picks = int((rm[ids] < 0).sum())
    log(f"T=112 positional: {n_cold_picks} cold picks, "
        f"{len(np.unique(ids[rm[ids] < 0]))} cold experts")
    assert n_cold_picks > 0
    Y0, o0, ninv = run_layer(hot_p, cold_p, rm, ids, w, x, H, I)
    assert ninv == 0
    from expert_weight_residency_amd.layer import ColdStage, LayerBuffers, ResidencyLayer
    from gpu_util import routing_tensors
    ids_d, w_d, x_d = routing_tensors(ids, w, x)
    bufs = LayerBuffers.allocate(T, K, H, I, hot_p.n_rows, cold_p.n_rows)
    layer = ResidencyLayer(hot_p, cold_p, torch.from_numpy(rm).cuda(), H, I,
                           stage=ColdStage(min(89, T * K), H, I))
    layer.forward(x_d, ids_d, w_d, bufs, hot_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    Y1 = bufs.Y[: T * K].cpu().numpy().view(np.uint16)
    o1 = bufs.out[:T].cpu().numpy().view(np.uint16)
    assert np.array_equal(Y0, Y1) and np.array_equal(o0, o1)
    t_cold = np.nonzero((rm[ids] < 0).any(axis=1))[0]
    tokens = np.unique(np.concatenate([t_cold[:4], [0, 57, T - 1]]))
    Yr, outr = _oracle_for(ids, w, x, tokens)
    e_y = rel_errors(Y0.reshape(T, K, H)[tokens], Yr)
    e_o = rel_errors(o0[tokens], outr)
    log(f"  sampled {len(tokens)} tokens: Y {e_y} out {e_o}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL
    del hot_p, cold_p
    torch.cuda.empty_cache()


def test_decode_T112_fitted_map_verify_windows(banks):
    """The high-concurrency workload as benchmarked: 112 tokens in 16 verify
    windows of 7 (correlated routing: experts with tens of tokens), the
    fitted map; the cold bank read in place and staged into HBM give the same
    bits; sampled tokens (every token with a cold pick among them) against the
    oracle."""
    rm, ho, co, hot, cold = banks
    T = 112
    ids, w = synth.window_routing(T, K, E, SEED, 0, 13)
    x = synth.activations(T, H, SEED, step=13)
    load = np.bincount(ids.ravel(), minlength=E)
    log(f"T=112 windows: {np.count_nonzero(load)} experts, max {load.max()} tokens/expert, "
        f"{int((rm[ids] < 0).sum())} cold picks")
    Y0, o0, ninv = run_layer(hot, cold, rm, ids, w, x, H, I)
    assert ninv == 0
    from expert_weight_residency_amd.layer import ColdStage, LayerBuffers, ResidencyLayer
    from gpu_util import routing_tensors
    ids_d, w_d, x_d = routing_tensors(ids, w, x)
    bufs = LayerBuffers.allocate(T, K, H, I, hot.n_rows, cold.n_rows)
    layer = ResidencyLayer(hot, cold, torch.from_numpy(rm).cuda(), H, I,
                           stage=ColdStage(min(len(co), T * K), H, I))
    layer.forward(x_d, ids_d, w_d, bufs, hot_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert np.array_equal(Y0, bufs.Y[: T * K].cpu().numpy().view(np.uint16))
    assert np.array_equal(o0, bufs.out[:T].cpu().numpy().view(np.uint16))
    t_cold = np.nonzero((rm[ids] < 0).any(axis=1))[0]
    busiest = int(np.argmax(load))
    t_busy = np.nonzero((ids == busiest).any(axis=1))[0]
    tokens = np.unique(np.concatenate([t_cold[:6], t_busy[:2], [0, T - 1]]))
    Yr, outr = _oracle_for(ids, w, x, tokens)
    e_y = rel_errors(Y0.reshape(T, K, H)[tokens], Yr)
    e_o = rel_errors(o0[tokens], outr)
    log(f"  sampled {len(tokens)} tokens: Y {e_y} out {e_o}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL


def test_prefill_T4096_sampled(banks):
    """Counter skipped (T > 256), nearly every expert touched, experts with
    hundreds of tokens; sampled tokens checked against the oracle."""
    rm, ho, co, hot, cold = banks
    T = 4096
    ids, w = synth.skewed_routing(T, K, E, SEED, 0, 7)
    x = synth.activations(T, H, SEED, step=7)
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    Y, out, ninv = run_layer(hot, cold, rm, ids, w, x, H, I, counts_layer=counts)
    assert ninv == 0
    assert not counts.cpu().numpy().any()
    load = np.bincount(ids.ravel(), minlength=E)
    log(f"T=4096: {np.count_nonzero(load)} experts touched, max {load.max()} tokens/expert")
    rng = np.random.default_rng(3)
    busiest = int(np.argmax(load))
    t_busy = np.nonzero((ids == busiest).any(axis=1))[0]
    t_cold = np.nonzero((rm[ids] < 0).any(axis=1))[0]
    tokens = np.unique(np.concatenate([rng.choice(T, 6, replace=False), t_busy[[0, -1]],
                                       t_cold[:3], [T - 1]]))
    Yr, outr = _oracle_for(ids, w, x, tokens)
    Yg = Y.reshape(T, K, H)[tokens]
    e_y, e_o = rel_errors(Yg, Yr), rel_errors(out[tokens], outr)
    log(f"  sampled {len(tokens)} tokens: Y {e_y} out {e_o}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL
