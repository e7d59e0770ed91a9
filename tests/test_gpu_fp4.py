"""GPU parity of the FP4 path (steps of MOE_FP4_MIN_TOKENS = 256 tokens and more).

From 256 tokens per step the expert FFN runs on the block-scaled FP4 matrix
instruction, the activations carried as two E4M3 terms. Checked here:
  - against the oracle (relative L2 <= 1e-2, max relative <= 3e-2, every slot
    on its own) on shapes with reduction tails (K = 320, 192, 64), experts of
    1..130 tokens (partial column groups, several tiles per expert), a cold
    bank read in place from pinned host memory, and H = 4096, I = 2880;
  - that the two-term activations keep the bf16 path's accuracy: the same
    picks through the bf16 kernel families (a step of fewer than 256 tokens)
    agree with the FP4 rows to ~5e-4 relative L2 (bf16 rounding flips), far
    inside the oracle tolerance (one E4M3 term alone would be ~1e-2 off);
  - split == unsplit, bitwise, and gate/up then down == the fused call,
    bitwise; a cold bank staged into HBM == the same bank read in place.
"""
import numpy as np
import pytest
import torch

import expert_weight_residency_amd as moe
import oracle
import synth
from expert_weight_residency_amd.layer import ColdStage, LayerBuffers, ResidencyLayer
from gpu_util import (MAX_REL, REL_L2, device_bank, host_bank, oracle_bank, pinned_bank,
                      rel_errors, routing_tensors, run_layer)

pytestmark = pytest.mark.gpu

FP4_MIN_TOKENS = 256


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield


def log(msg):
    print(msg, flush=True)


def _case(E, k, H, I, T, n_cold, seed, routing):
    rm, ho, co = synth.random_map(E, n_cold, seed)
    hot = host_bank(ho, seed, 0, H, I)
    cold = host_bank(co, seed, 0, H, I)
    if routing == "gaussian":
        ids, w = synth.gaussian_routing(T, k, E, seed)
    else:
        ids, w = synth.skewed_routing(T, k, E, seed, 0, 0)
    x = synth.activations(T, H, seed)
    return rm, ho, co, hot, cold, ids, w, x


def _check_vs_oracle(rm, hot, cold, ids, w, x, H, I, cold_pinned):
    T, k = ids.shape
    assert T >= FP4_MIN_TOKENS
    Yr, outr, bad = oracle.moe_layer(oracle_bank(hot), oracle_bank(cold), rm, ids, w, x, H, I)
    assert bad == 0
    cb = pinned_bank(cold) if cold_pinned else device_bank(cold)
    Y, out, ninv = run_layer(device_bank(hot), cb, rm, ids, w, x, H, I)
    assert ninv == 0
    Yr = Yr.reshape(T * k, H)
    e_y, e_o = rel_errors(Y, Yr), rel_errors(out, outr)
    log(f"  Y rel-L2 {e_y[0]:.2e} max-rel {e_y[1]:.2e}; out rel-L2 {e_o[0]:.2e} max-rel {e_o[1]:.2e}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL
    for s in range(T * k):
        r = rel_errors(Y[s], Yr[s])
        assert r[0] <= REL_L2, (s, r)
    return Y, out


FP4_CASES = [
    # name, E, k, H, I, T, n_cold, routing, cold pinned
    ("small", 16, 2, 256, 128, 256, 4, "gaussian", False),
    ("ragged_K320_I192", 8, 2, 320, 192, 300, 2, "skewed", True),
    ("K64", 4, 1, 64, 64, 300, 1, "gaussian", False),
    ("mid_skewed", 64, 4, 1024, 512, 400, 16, "skewed", True),
]


@pytest.mark.parametrize("case", FP4_CASES, ids=[c[0] for c in FP4_CASES])
def test_fp4_matches_oracle(case):
    name, E, k, H, I, T, n_cold, routing, pinned = case
    log(f"fp4 case {name}")
    rm, ho, co, hot, cold, ids, w, x = _case(E, k, H, I, T, n_cold, 61, routing)
    _check_vs_oracle(rm, hot, cold, ids, w, x, H, I, pinned)


def test_fp4_tile_sizes():
    """Experts with 1, 15, 16, 17, 63, 64, 65, 127, 128, 129 and 257 tokens
    (k = 1, 891 tokens): partial column groups, exact tiles, experts spanning
    up to five tiles."""
    counts = [9, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 257]
    H, I, seed = 512, 256, 71
    E = len(counts)
    rm, ho, co = synth.map_from_cold_set(E, [0])
    hot, cold = host_bank(ho, seed, 0, H, I), host_bank(co, seed, 0, H, I)
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])[:, None]
    w = np.ones_like(ids, dtype=np.float32)
    x = synth.activations(len(ids), H, seed)
    log(f"fp4 tile sizes {counts}")
    _check_vs_oracle(rm, hot, cold, ids, w, x, H, I, True)


def test_fp4_full_shape():
    """H = 4096, I = 2880 (the I axis ends inside its 12th chunk), 4 experts,
    256 tokens of top-2."""
    E, k, H, I, T = 4, 2, 4096, 2880, 256
    rm, ho, co, hot, cold, ids, w, x = _case(E, k, H, I, T, 1, 81, "gaussian")
    log("fp4 full shape")
    _check_vs_oracle(rm, hot, cold, ids, w, x, H, I, True)


@pytest.mark.parametrize("shape", [(16, 2, 512, 256), (8, 2, 4096, 2880)], ids=["H512", "H4096"])
def test_fp4_close_to_bf16_families(shape):
    """The first 200 tokens of a 256-token step through the bf16 families (a
    200-token step) and through the FP4 path: within 1e-3 relative L2 overall
    and 5e-3 for every row. Both outputs are rounded to bf16 (unit 2^-8), so
    rows differ by single rounding flips; one E4M3 term per activation
    instead of two would put them ~1e-2 apart."""
    E, k, H, I = shape
    T, small = 256, 200
    rm, ho, co, hot, cold, ids, w, x = _case(E, k, H, I, T, 2, 93, "gaussian")
    hb, cb = device_bank(hot), device_bank(cold)
    Yf, _, _ = run_layer(hb, cb, rm, ids, w, x, H, I)
    Yb, _, _ = run_layer(hb, cb, rm, ids[:small], w[:small], x[:small], H, I)
    e = rel_errors(Yf[: small * k], Yb)
    worst = max(rel_errors(Yf[s], Yb[s])[0] for s in range(small * k))
    log(f"  fp4 vs bf16 families: rel-L2 {e[0]:.2e}, worst row {worst:.2e}")
    assert not np.array_equal(Yf[: small * k], Yb)  # the FP4 path ran
    assert e[0] <= 1e-3 and worst <= 5e-3


def test_fp4_split_equals_unsplit():
    """Bitwise split (hot in HBM + cold pinned, read in place) == unsplit (all
    rows in one HBM bank)."""
    E, k, H, I, T, seed = 16, 2, 512, 256, 400, 101
    rm, ho, co, hot, cold, ids, w, x = _case(E, k, H, I, T, 4, seed, "skewed")
    Ys, outs, _ = run_layer(device_bank(hot), pinned_bank(cold), rm, ids, w, x, H, I)
    all_map, all_owner, _ = synth.all_hot_map(E)
    Yu, outu, _ = run_layer(device_bank(host_bank(all_owner, seed, 0, H, I)), None, all_map, ids,
                            w, x, H, I)
    assert np.array_equal(Ys, Yu) and np.array_equal(outs, outu)


def test_fp4_stage_calls_equal_fused_call():
    """moe_expert_gate_up_mxfp4 then moe_expert_down_mxfp4 == moe_expert_ffn_mxfp4."""
    E, k, H, I, T = 24, 3, 512, 320, 260
    rm_np, ho, co = synth.random_map(E, 0, 5)
    bank = device_bank(host_bank(ho, 5, 0, H, I))
    ids, w = synth.gaussian_routing(T, k, E, 5)
    x = synth.activations(T, H, 5)
    ids_d, w_d, x_d = routing_tensors(ids, w, x)
    rm = torch.from_numpy(rm_np).cuda()
    bufs = LayerBuffers.allocate(T, k, H, I, E, 0)
    moe.moe_route_split(ids_d, rm, E, 0, bufs.hot_split, bufs.cold_split, bufs.n_invalid)
    moe.moe_expert_ffn_mxfp4(bank, bufs.hot_split, x_d, k, I, bufs.workspace, bufs.Y)
    torch.cuda.synchronize()
    Y1 = bufs.Y[: T * k].cpu().numpy().copy()
    bufs.Y.zero_()
    moe.moe_expert_gate_up_mxfp4(bank, bufs.hot_split, x_d, k, I, bufs.workspace)
    moe.moe_expert_down_mxfp4(bank, bufs.hot_split, T, k, H, I, bufs.workspace, bufs.Y)
    torch.cuda.synchronize()
    assert np.array_equal(Y1, bufs.Y[: T * k].cpu().numpy())


def test_fp4_staged_equals_in_place():
    """The cold bank staged into HBM (moe_stage_rows) gives the bits of the
    same bank read in place from pinned host memory."""
    E, k, H, I, T, seed = 32, 4, 512, 320, 300, 17
    rm_np, ho, co, hot, cold, ids, w, x = _case(E, k, H, I, T, 10, seed, "skewed")
    rm = torch.from_numpy(rm_np).cuda()
    hb, cb = device_bank(hot), pinned_bank(cold)
    ids_d, w_d, x_d = routing_tensors(ids, w, x)
    res = []
    for stage in (None, ColdStage(min(len(co), T * k), H, I)):
        bufs = LayerBuffers.allocate(T, k, H, I, hb.n_rows, cb.n_rows)
        ResidencyLayer(hb, cb, rm, H, I, stage=stage).forward(x_d, ids_d, w_d, bufs)
        torch.cuda.synchronize()
        res.append((bufs.Y[: T * k].cpu().numpy().copy(), bufs.out[:T].cpu().numpy().copy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
