"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: the residency split (active rows, offsets, slots), n_invalid, the
usage counter (also under HIP-graph capture), the finalize given the same
rows, and split vs unsplit. Within tolerance (relative L2 <= 1e-2, max
relative <= 3e-2): the expert rows Y and the layer output."""
import numpy as np
import pytest
import torch

import expert_weight_residency_amd as moe
import oracle
import synth
from gpu_util import (MAX_REL, REL_L2, device_bank, empty_bank_host, host_bank, oracle_bank,
                      pinned_bank, rel_errors, routing_tensors, run_layer)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield


def log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ split --

def _gpu_split(ids, row_map, n_hot, n_cold, counts=None, count_tmax=256):
    T, k = ids.shape
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    rm = torch.from_numpy(np.ascontiguousarray(row_map, np.int32)).cuda()
    hs, cs = moe.Split.empty(n_hot, T, k), moe.Split.empty(n_cold, T, k)
    ninv = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    moe.moe_route_split(ids_d, rm, n_hot, n_cold, hs, cs, ninv, counts, count_tmax)
    torch.cuda.synchronize()
    return hs.to_host(), cs.to_host(), int(ninv.item())


def _split_cases():
    rng = np.random.default_rng(5)
    cases = []
    rm, ho, co = synth.random_map(16, 4, 1)
    ids, _ = synth.gaussian_routing(8, 2, 16, seed=1)
    cases.append(("tiny", ids, rm, len(ho), len(co)))
    rm, ho, co = synth.fitted_map(384, 89, 2, 0)
    for T in (1, 7, 16, 112, 256, 300, 4096):
        ids, _ = synth.skewed_routing(T, 6, 384, 2, 0, T)
        cases.append((f"fitted_T{T}", ids, rm, len(ho), len(co)))
    rm, ho, co = synth.positional_map(384, 89)
    ids, _ = synth.skewed_routing(112, 6, 384, 2, 1, 0)
    cases.append(("positional_T112", ids, rm, len(ho), len(co)))
    bad = ids.copy()
    bad[3, 2], bad[7, 0], bad[50, 5] = 384, -1, 10_000
    cases.append(("invalid_ids", bad, rm, len(ho), len(co)))
    rm_bad = rm.copy()
    rm_bad[int(bad[9, 1])] = 295           # hot row past the bank
    cases.append(("invalid_rows", bad, rm_bad, len(ho), len(co)))
    cases.append(("empty", np.zeros((0, 6), np.int32), rm, len(ho), len(co)))
    rm, ho, co = synth.all_hot_map(384)
    cases.append(("all_hot", synth.skewed_routing(64, 6, 384, 3, 0, 0)[0], rm, len(ho), 0))
    rm, ho, co = synth.map_from_cold_set(384, np.arange(384))
    cases.append(("all_cold", synth.skewed_routing(64, 6, 384, 3, 0, 0)[0], rm, 0, len(co)))
    # a single expert takes every token (long slot list for one row), k = 1
    ids = np.zeros((3000, 1), np.int32) + 17
    rm, ho, co = synth.fitted_map(384, 89, 2, 0)
    cases.append(("one_expert_T3000_k1", ids, rm, len(ho), len(co)))
    return cases


@pytest.mark.parametrize("name,ids,row_map,n_hot,n_cold", _split_cases(),
                         ids=[c[0] for c in _split_cases()])
def test_route_split_bit_exact(name, ids, row_map, n_hot, n_cold):
    log(f"split case {name} T={ids.shape[0]}")
    ref = oracle.route_split(ids, row_map, n_hot, n_cold)
    h, c, ninv = _gpu_split(ids, row_map, n_hot, n_cold)
    assert ninv == ref["n_invalid"]
    for got, want in ((h, ref["hot"]), (c, ref["cold"])):
        for g, w in zip(got, want):
            assert np.array_equal(g, w)


@pytest.mark.parametrize("T", [1, 16, 256, 257, 4096])
def test_usage_counter_bit_exact(T):
    E = 384
    rm, ho, co = synth.fitted_map(E, 89, 4, 3)
    ids, _ = synth.skewed_routing(T, 6, E, 4, 3, 1)
    ids[0, 0] = -5                          # invalid ids are not counted
    table = torch.zeros((40, E), dtype=torch.int32, device="cuda")
    table[3] = torch.arange(E, dtype=torch.int32)
    _gpu_split(ids, rm, len(ho), len(co), counts=table[3])
    want = oracle.usage_count(np.arange(E, dtype=np.int32), ids, E)
    got = table.cpu().numpy()
    assert np.array_equal(got[3], want)
    assert not got[np.arange(40) != 3].any()
    if T <= 256:
        assert int(got[3].sum() - np.arange(E).sum()) == T * 6 - 1


def test_usage_counter_in_graph_capture():
    """The counter inside a captured graph: every replay adds the histogram
    once, and the split outputs stay correct (device tensors are read at replay
    time)."""
    E, T, k = 384, 16, 6
    rm_np, ho, co = synth.fitted_map(E, 89, 6, 0)
    ids_np, _ = synth.skewed_routing(T, k, E, 6, 0, 0)
    ids = torch.from_numpy(ids_np).cuda()
    rm = torch.from_numpy(rm_np).cuda()
    table = torch.zeros((40, E), dtype=torch.int32, device="cuda")
    hs, cs = moe.Split.empty(len(ho), T, k), moe.Split.empty(len(co), T, k)
    ninv = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up outside capture
        moe.moe_route_split(ids, rm, len(ho), len(co), hs, cs, ninv, table[5], stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_route_split(ids, rm, len(ho), len(co), hs, cs, ninv, table[5])
    torch.cuda.synchronize()
    ref = oracle.route_split(ids_np, rm_np, len(ho), len(co))
    hist = np.bincount(ids_np.ravel(), minlength=E)
    for rep in range(1, 4):
        junk = torch.randn(1024, device="cuda").sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(table[5].cpu().numpy(), (rep + 1) * hist), rep
        for got, want in ((hs.to_host(), ref["hot"]), (cs.to_host(), ref["cold"])):
            for a, b in zip(got, want):
                assert np.array_equal(a, b)
        del junk


# --------------------------------------------------------------- finalize --

@pytest.mark.parametrize("T,k,H", [(16, 6, 4096), (3, 1, 64), (33, 8, 264), (7, 6, 4096)])
def test_finalize_bit_exact(T, k, H):
    rng = np.random.default_rng(T * 100 + k)
    Yf = (rng.standard_normal((T, k, H)) * 10.0 ** rng.integers(-3, 4, (T, k, 1))).astype(np.float32)
    Y = torch.from_numpy(Yf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    want = oracle.finalize(Y, w)
    Yd = torch.from_numpy(Y.reshape(T * k, H).view(np.int16)).cuda()
    wd = torch.from_numpy(w).cuda()
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    moe.moe_finalize(Yd, wd, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)


def test_finalize_crafted_fma_and_order():
    # The oracle-pinned crafted inputs, through the GPU kernel.
    def b16(x):
        return torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
    w = np.array([[-(1 + 2.0 ** -7 + 2.0 ** -20), 1 + 2.0 ** -20],
                  [1 + 2.0 ** -8, 2.0 ** -24]], np.float32)
    Y = np.array([[[b16(1.0)] * 8, [b16(1 + 2.0 ** -7)] * 8],
                  [[b16(1.0)] * 8, [b16(1.0)] * 8]], np.uint16)
    want = oracle.finalize(Y, w)
    out = torch.empty((2, 8), dtype=torch.int16, device="cuda")
    moe.moe_finalize(torch.from_numpy(Y.reshape(4, 8).view(np.int16)).cuda(), torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert oracle.bf16_to_f32(got)[0, 0] == 2.0 ** -27


# -------------------------------------------------------------------- FFN --

def _layer_case(E, k, H, I, T, n_cold, seed, routing="skewed", scale_lo=124, scale_cnt=5,
                force_expert=None):
    rm, ho, co = synth.random_map(E, n_cold, seed)
    hot = host_bank(ho, seed, 0, H, I, scale_lo=scale_lo, scale_cnt=scale_cnt)
    cold = host_bank(co, seed, 0, H, I, scale_lo=scale_lo, scale_cnt=scale_cnt)
    if routing == "gaussian":
        ids, w = synth.gaussian_routing(T, k, E, seed)
    else:
        ids, w = synth.skewed_routing(T, k, E, seed, 0, 0)
    if force_expert is not None:   # one expert in every token's picks: a long slot list
        for t in range(T):
            if force_expert not in ids[t]:
                ids[t, t % k] = force_expert
    x = synth.activations(T, H, seed)
    return rm, ho, co, hot, cold, ids, w, x


FFN_CASES = [
    # name, E, k, H, I, T, n_cold, routing, force
    ("tiny", 16, 2, 256, 128, 8, 4, "gaussian", None),
    ("mid", 64, 4, 1024, 512, 32, 16, "skewed", None),
    ("ragged_I320", 24, 3, 512, 320, 40, 6, "skewed", 5),
    ("many_tokens_one_expert", 32, 2, 256, 192, 100, 8, "skewed", 3),
    ("k1_T1", 16, 1, 256, 128, 1, 4, "gaussian", None),
    ("H4096_I2880_small_E", 8, 2, 4096, 2880, 6, 2, "gaussian", None),
    # 40 picks: the hot bank (48 rows) on the decode kernels, the cold (16) tiled
    ("decode_family_T20", 64, 2, 1024, 512, 20, 16, "skewed", None),
]


@pytest.mark.parametrize("case", FFN_CASES, ids=[c[0] for c in FFN_CASES])
def test_ffn_layer_matches_oracle(case):
    name, E, k, H, I, T, n_cold, routing, force = case
    log(f"ffn case {name}")
    rm, ho, co, hot, cold, ids, w, x = _layer_case(E, k, H, I, T, n_cold, 11, routing,
                                                    force_expert=force)
    Yr, outr, bad = oracle.moe_layer(oracle_bank(hot), oracle_bank(cold), rm, ids, w, x, H, I)
    assert bad == 0
    Y, out, ninv = run_layer(device_bank(hot), device_bank(cold), rm, ids, w, x, H, I)
    assert ninv == 0
    e_y = rel_errors(Y, Yr.reshape(T * k, H))
    e_o = rel_errors(out, outr)
    log(f"  Y rel-L2 {e_y[0]:.2e} max-rel {e_y[1]:.2e}; out rel-L2 {e_o[0]:.2e} max-rel {e_o[1]:.2e}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL
    # every slot individually, so one bad row cannot hide in the norm
    for s in range(T * k):
        r = rel_errors(Y[s], Yr.reshape(T * k, H)[s])
        assert r[0] <= REL_L2, (s, r)


def test_ffn_wide_scale_range():
    """E8M0 bytes spread over 112..142 (2^-15 .. 2^15) instead of the default window."""
    E, k, H, I, T = 16, 2, 256, 128, 8
    rm, ho, co, hot, cold, ids, w, x = _layer_case(E, k, H, I, T, 4, 21, "gaussian", 112, 31)
    Yr, outr, _ = oracle.moe_layer(oracle_bank(hot), oracle_bank(cold), rm, ids, w, x, H, I)
    Y, out, _ = run_layer(device_bank(hot), device_bank(cold), rm, ids, w, x, H, I)
    e = rel_errors(Y, Yr.reshape(T * k, H))
    assert e[0] <= REL_L2 and e[1] <= MAX_REL, e


@pytest.mark.parametrize("cold_where", ["device", "pinned_host", "pinned_host_two_streams"])
def test_split_equals_unsplit_bit_exact(cold_where):
    """Split (12 hot / 4 cold) and unsplit (all 16 in one bank, identity map)
    give the same bits for every row and every output."""
    E, k, H, I, T, seed = 16, 2, 256, 128, 8, 31
    rm, ho, co, hot, cold, ids, w, x = _layer_case(E, k, H, I, T, 4, seed, "gaussian")
    cold_bank = device_bank(cold) if cold_where == "device" else pinned_bank(cold)
    cs = torch.cuda.Stream() if cold_where.endswith("two_streams") else None
    Ys, outs, _ = run_layer(device_bank(hot), cold_bank, rm, ids, w, x, H, I, cold_stream=cs)
    all_map, all_owner, _ = synth.all_hot_map(E)
    allb = host_bank(all_owner, seed, 0, H, I)
    Yu, outu, _ = run_layer(device_bank(allb), None, all_map, ids, w, x, H, I)
    assert np.array_equal(Ys, Yu)
    assert np.array_equal(outs, outu)


def test_split_equals_unsplit_many_tokens():
    """Same at a size where experts get several 16-token tiles (T = 100)."""
    E, k, H, I, T, seed = 32, 4, 512, 256, 100, 41
    rm, ho, co, hot, cold, ids, w, x = _layer_case(E, k, H, I, T, 8, seed, "skewed")
    Ys, outs, _ = run_layer(device_bank(hot), pinned_bank(cold), rm, ids, w, x, H, I)
    all_map, all_owner, _ = synth.all_hot_map(E)
    Yu, outu, _ = run_layer(device_bank(host_bank(all_owner, seed, 0, H, I)), None, all_map, ids,
                            w, x, H, I)
    assert np.array_equal(Ys, Yu) and np.array_equal(outs, outu)


@pytest.mark.parametrize("T", [16, 17, 255, 256])
def test_family_boundaries(T):
    """Steps on either side of the kernel-family thresholds, H = 1024, I = 512,
    24 hot rows in HBM and 8 cold rows in pinned host memory: 16 tokens run the
    resident kernels, 17 the decode kernels (too few picks per row for the
    token tiles), 255 the token-tiled bf16 kernels and 256 the FP4 kernels.
    Each against the oracle (every slot on its own), and split == unsplit
    bitwise (the family depends on T alone, not on the bank)."""
    E, k, H, I, seed = 32, 2, 1024, 512, 57
    log(f"family boundary T={T}")
    rm, ho, co, hot, cold, ids, w, x = _layer_case(E, k, H, I, T, 8, seed, "skewed")
    Yr, outr, bad = oracle.moe_layer(oracle_bank(hot), oracle_bank(cold), rm, ids, w, x, H, I)
    assert bad == 0
    Ys, outs, ninv = run_layer(device_bank(hot), pinned_bank(cold), rm, ids, w, x, H, I)
    assert ninv == 0
    Yr = Yr.reshape(T * k, H)
    e_y, e_o = rel_errors(Ys, Yr), rel_errors(outs, outr)
    log(f"  Y rel-L2 {e_y[0]:.2e} max-rel {e_y[1]:.2e}; out rel-L2 {e_o[0]:.2e} max-rel {e_o[1]:.2e}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL
    for s in range(T * k):
        r = rel_errors(Ys[s], Yr[s])
        assert r[0] <= REL_L2, (s, r)
    all_map, all_owner, _ = synth.all_hot_map(E)
    Yu, outu, _ = run_layer(device_bank(host_bank(all_owner, seed, 0, H, I)), None, all_map, ids,
                            w, x, H, I)
    assert np.array_equal(Ys, Yu) and np.array_equal(outs, outu)


def test_empty_step_writes_nothing():
    E, k, H, I = 16, 2, 256, 128
    rm, ho, co, hot, cold, ids, w, x = _layer_case(E, k, H, I, 4, 4, 3, "gaussian")
    Y, out, ninv = run_layer(device_bank(hot), device_bank(cold), rm, ids[:0], w[:0], x[:0], H, I)
    assert ninv == 0 and Y.size == 0 and out.size == 0


def test_stage_calls_equal_fused_call():
    """moe_expert_gate_up_mxfp4 then moe_expert_down_mxfp4 == moe_expert_ffn_mxfp4, bitwise."""
    E, k, H, I, T = 24, 3, 512, 320, 20
    rm, ho, co, hot, cold, ids, w, x = _layer_case(E, k, H, I, T, 6, 13, "skewed")
    bank = device_bank(hot)
    ids_d, w_d, x_d = routing_tensors(ids, w, x)
    rm_d = torch.from_numpy(rm).cuda()
    hs, cs = moe.Split.empty(len(ho), T, k), moe.Split.empty(len(co), T, k)
    ninv = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_route_split(ids_d, rm_d, len(ho), len(co), hs, cs, ninv)
    ws = torch.empty(moe.moe_ffn_workspace_bytes(T, k, H, I), dtype=torch.uint8, device="cuda")
    Y1 = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    Y2 = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    moe.moe_expert_ffn_mxfp4(bank, hs, x_d, k, I, ws, Y1)
    moe.moe_expert_gate_up_mxfp4(bank, hs, x_d, k, I, ws)
    moe.moe_expert_down_mxfp4(bank, hs, T, k, H, I, ws, Y2)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    assert int((Y1 != 0).any(dim=1).sum()) == int(hs.to_host()[1][-1])
