"""The host-bank kernels (decode-sized steps with the bank in pinned host
memory: each item's weights copied over the host link in the linear pattern,
then multiplied out of LDS) against the same bank in HBM, bit for bit, and
against the oracle within the FFN tolerance: several H and I (an I ending
inside its last chunk), 1 to 16 tokens, an expert whose slots need two
16-slot passes (duplicate ids), and a step whose slots exceed the LDS rows of
one phase (every pick cold)."""
import numpy as np
import pytest
import torch

import expert_weight_residency_amd as moe
import oracle
import synth
from gpu_util import (MAX_REL, REL_L2, device_bank, host_bank, oracle_bank, pinned_bank,
                      rel_errors, routing_tensors)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield


def _ffn(bank, ids, x, E, k, H, I):
    """One bank holding every expert (row e = expert e), identity map."""
    T = ids.shape[0]
    rm = torch.arange(E, dtype=torch.int32, device="cuda")
    ids_d, _, x_d = routing_tensors(ids, np.ones(ids.shape, np.float32), x)
    hs, cs = moe.Split.empty(E, T, k), moe.Split.empty(0, T, k)
    ninv = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_route_split(ids_d, rm, E, 0, hs, cs, ninv)
    ws = torch.empty(moe.moe_ffn_workspace_bytes(T, k, H, I), dtype=torch.uint8, device="cuda")
    Y = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    moe.moe_expert_ffn_mxfp4(bank, hs, x_d, k, I, ws, Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy().view(np.uint16)


CASES = [
    # name, E, k, H, I, T, routing
    ("h1024_i512_t7", 12, 4, 1024, 512, 7, "skewed"),
    ("h2048_i320_t16", 10, 3, 2048, 320, 16, "skewed"),
    ("h4096_i2880_t1", 8, 6, 4096, 2880, 1, "skewed"),
    ("h4096_i2880_t16", 12, 6, 4096, 2880, 16, "skewed"),
    ("h4096_i1472_t5", 8, 2, 4096, 1472, 5, "skewed"),
    ("two_passes_dup_ids", 6, 4, 1024, 512, 9, "dup"),      # expert 2: 18 slots
    ("phases_all_picks", 6, 6, 4096, 2880, 16, "spread"),   # 16 slots on each of 6 rows
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_host_bank_equals_device_bank_and_oracle(case):
    name, E, k, H, I, T, routing = case
    print(f"host-bank case {name}: E={E} k={k} H={H} I={I} T={T}", flush=True)
    seed = 73
    owners = np.arange(E, dtype=np.int32)
    arrays = host_bank(owners, seed, 0, H, I)
    ids, _ = synth.skewed_routing(T, k, E, seed, 0, 0)
    if routing == "dup":
        ids[:, 0] = 2
        ids[:, 1] = 2    # two picks of expert 2 per token (caller-side duplicates)
    elif routing == "spread":
        ids = (np.arange(T * k, dtype=np.int32).reshape(T, k) * 7) % E
    x = synth.activations(T, H, seed)
    Yd = _ffn(device_bank(arrays), ids, x, E, k, H, I)
    Yh = _ffn(pinned_bank(arrays), ids, x, E, k, H, I)
    assert np.array_equal(Yh, Yd), name
    ob = oracle_bank(arrays)
    for s in range(T * k):
        t, e = s // k, int(ids.reshape(-1)[s])
        ref = oracle.expert_ffn(ob.w13[e], ob.s13[e], ob.w2[e], ob.s2[e], x[t], H, I)["y_bf16"]
        err = rel_errors(Yh[s], ref)
        assert err[0] <= REL_L2 and err[1] <= MAX_REL, (name, s, err)


def _split_host_bank(arrays: dict) -> moe.Bank:
    """Weights pinned on the host, scales in device memory."""
    w = pinned_bank(arrays)
    s = device_bank(arrays)
    return moe.Bank(w.w13, s.s13, w.w2, s.s2, on_host=moe.BANK_HOST_WEIGHTS)


SPLIT_CASES = [
    # name, E, k, H, I, T: host kernels (T <= 16), token-tiled / resident, FP4 (T >= 256)
    ("h4096_i2880_t16", 10, 6, 4096, 2880, 16),
    ("h2048_i1472_t7", 8, 4, 2048, 1472, 7),
    ("h1024_i512_t40", 12, 4, 1024, 512, 40),
    ("h1024_i512_t300", 12, 4, 1024, 512, 300),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_host_weights_device_scales_bank_equals_host_bank(case):
    """A bank whose weights sit in pinned host memory and whose scales sit in
    HBM gives the same bits as the all-host and all-device banks."""
    name, E, k, H, I, T = case
    print(f"host-weights bank case {name}: E={E} k={k} H={H} I={I} T={T}", flush=True)
    seed = 91
    arrays = host_bank(np.arange(E, dtype=np.int32), seed, 0, H, I)
    ids, _ = synth.skewed_routing(T, k, E, seed, 0, 0)
    x = synth.activations(T, H, seed)
    Yd = _ffn(device_bank(arrays), ids, x, E, k, H, I)
    Yh = _ffn(pinned_bank(arrays), ids, x, E, k, H, I)
    Ys = _ffn(_split_host_bank(arrays), ids, x, E, k, H, I)
    assert np.array_equal(Ys, Yh), name
    assert np.array_equal(Ys, Yd), name
