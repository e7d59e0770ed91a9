"""GPU parity at the longest reduction axes the entry points accept.

H and I may each be up to 32768 elements (the bf16 decode kernels stage one
token's x row of H elements, 64 KB, in LDS). Here H = 32768 (the gate/up
reduction at its maximum, down over 128) and I = 32768 (down's reduction at
its maximum, gate/up over 256), each through the bf16 families (8 tokens) and
the FP4 family (256 tokens: 128 quantized chunks per row), 3 rows in HBM and 1
in pinned host memory read in place; every slot against the oracle.
"""
import numpy as np
import pytest
import torch

import expert_weight_residency_amd as moe
import oracle
import synth
from gpu_util import (MAX_REL, REL_L2, device_bank, host_bank, oracle_bank, pinned_bank,
                      rel_errors, run_layer)

pytestmark = pytest.mark.gpu

MAX_K = 32768


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield


def log(msg):
    print(msg, flush=True)


CASES = [
    # name, H, I, T, k
    ("H32768_bf16", MAX_K, 128, 8, 2),
    ("H32768_fp4", MAX_K, 128, 256, 1),
    ("I32768_bf16", 256, MAX_K, 8, 2),
    ("I32768_fp4", 256, MAX_K, 256, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_longest_reduction_matches_oracle(case):
    name, H, I, T, k = case
    E, seed = 4, 91
    log(f"max-size case {name}")
    rm, ho, co = synth.random_map(E, 1, seed)
    hot, cold = host_bank(ho, seed, 0, H, I), host_bank(co, seed, 0, H, I)
    ids, w = synth.gaussian_routing(T, k, E, seed)
    x = synth.activations(T, H, seed)
    Yr, outr, bad = oracle.moe_layer(oracle_bank(hot), oracle_bank(cold), rm, ids, w, x, H, I)
    assert bad == 0
    Y, out, ninv = run_layer(device_bank(hot), pinned_bank(cold), rm, ids, w, x, H, I)
    assert ninv == 0
    Yr = Yr.reshape(T * k, H)
    e_y, e_o = rel_errors(Y, Yr), rel_errors(out, outr)
    log(f"  Y rel-L2 {e_y[0]:.2e} max-rel {e_y[1]:.2e}; out rel-L2 {e_o[0]:.2e} max-rel {e_o[1]:.2e}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL
    for s in range(T * k):
        r = rel_errors(Y[s], Yr[s])
        assert r[0] <= REL_L2, (s, r)
    assert np.isfinite(oracle.bf16_to_f32(Y)).all()


def test_fp4_largest_step_sampled():
    """The largest step the FP4 path accepts at H = 4096: T*k = 524,286 slots,
    whose quantized x rows end 16 KB below 4 GB (the kernels address them with
    32-bit offsets; one more token of 6 picks is refused). 8 experts, top-6,
    I = 256; sampled tokens, the last one holding the highest slots, against
    the oracle."""
    from expert_weight_residency_amd.layer import LayerBuffers, ResidencyLayer
    from gpu_util import routing_tensors
    H, I, E, k, seed = 4096, 256, 8, 6, 93
    T = ((1 << 32) // (16 * 512) - 1) // k          # 87,381 tokens: 524,286 slots
    assert moe.moe_ffn_workspace_bytes(T, k, H, I) > 0
    assert moe.moe_ffn_workspace_bytes(T + 1, k, H, I) == 0
    rm, ho, co = synth.random_map(E, 1, seed)
    hb, cb = host_bank(ho, seed, 0, H, I), host_bank(co, seed, 0, H, I)
    ids, w = synth.gaussian_routing(T, k, E, seed)
    x = synth.activations(T, H, seed)
    log(f"largest FP4 step: T={T}, {T * k} slots")
    ids_d, w_d, x_d = routing_tensors(ids, w, x)
    bufs = LayerBuffers.allocate(T, k, H, I, len(ho), len(co))
    layer = ResidencyLayer(device_bank(hb), device_bank(cb),
                           torch.from_numpy(np.ascontiguousarray(rm, np.int32)).cuda(), H, I)
    layer.forward(x_d, ids_d, w_d, bufs)
    torch.cuda.synchronize()
    assert int(bufs.n_invalid.item()) == 0
    rng = np.random.default_rng(5)
    tokens = np.unique(np.concatenate([[0, T // 2, T - 2, T - 1], rng.choice(T, 4, replace=False)]))
    tok_d = torch.from_numpy(tokens).cuda()
    Y = bufs.Y.view(T, k, H)[tok_d].cpu().numpy().view(np.uint16)
    out = bufs.out[:T][tok_d].cpu().numpy().view(np.uint16)
    del bufs, layer
    torch.cuda.empty_cache()
    Yr, outr, bad = oracle.moe_layer(oracle_bank(hb), oracle_bank(cb), rm, ids[tokens], w[tokens],
                                     x[tokens], H, I)
    assert bad == 0
    e_y, e_o = rel_errors(Y, Yr.reshape(len(tokens), k, H)), rel_errors(out, outr)
    log(f"  sampled {len(tokens)} tokens: Y {e_y} out {e_o}")
    assert e_y[0] <= REL_L2 and e_y[1] <= MAX_REL
    assert e_o[0] <= REL_L2 and e_o[1] <= MAX_REL
    for i in range(len(tokens)):
        for j in range(k):
            r = rel_errors(Y[i, j], Yr.reshape(len(tokens), k, H)[i, j])
            assert r[0] <= REL_L2, (tokens[i], j, r)


@pytest.mark.parametrize("T", [8, 64, 256], ids=["T8_decode", "T64_decode", "T256_fp4"])
def test_most_experts_rows_and_picks(T):
    """The count limits at once: 4096 experts (MOE_MAX_EXPERTS), 3072 rows in
    HBM and 1024 in pinned host memory, one 4096-row bank (MOE_MAX_ROWS) for
    the unsplit run, top-32 (MOE_MAX_TOPK); H = I = 64 keeps the banks small.
    Every slot against the oracle, split == unsplit bitwise, and the usage
    counter against the oracle's (steps of at most 256 tokens count)."""
    E, k, H, I, seed = 4096, 32, 64, 64, 97
    log(f"count limits T={T}")
    rm, ho, co = synth.random_map(E, 1024, seed)
    hot, cold = host_bank(ho, seed, 0, H, I), host_bank(co, seed, 0, H, I)
    ids, w = synth.gaussian_routing(T, k, E, seed)
    x = synth.activations(T, H, seed)
    Yr, outr, bad = oracle.moe_layer(oracle_bank(hot), oracle_bank(cold), rm, ids, w, x, H, I)
    assert bad == 0
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    Ys, outs, ninv = run_layer(device_bank(hot), pinned_bank(cold), rm, ids, w, x, H, I,
                               counts_layer=counts)
    assert ninv == 0
    assert np.array_equal(counts.cpu().numpy(), oracle.usage_count(np.zeros(E, np.int32), ids, E))
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
