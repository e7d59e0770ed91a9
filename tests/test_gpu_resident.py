"""GPU parity of the gate/up kernel with all activations resident in LDS.

The library runs it for device-resident banks when 1 <= T <= 16 (decode). It
must match the oracle within tolerance (relative L2 <= 1e-2, max relative <=
3e-2, every slot on its own) and give the same bits as the other kernel
families for every pick:
  - decode shapes (T = 1, 7, 16 at full H = 4096, I = 2880; a ragged I; a row
    whose scale bytes fill a quarter line (H = 1024), three quarters (3072)
    or two lines (8192));
  - an expert picked by all 16 tokens (one full 16-token pass) and an expert
    with 64 slots from duplicate ids (four passes);
  - bitwise against the decode kernel (steps with T > 16), with the bank in
    HBM and in pinned host memory; a pinned-memory bank against the oracle.
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


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield


def log(msg):
    print(msg, flush=True)


def _check(rm, hot, cold, ids, w, x, H, I, cold_pinned=False):
    T, k = ids.shape
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
    return Y


@pytest.mark.parametrize("shape", [(48, 6, 4096, 2880, 1), (48, 6, 4096, 2880, 7),
                                   (48, 6, 4096, 2880, 16), (24, 4, 1024, 320, 16),
                                   (24, 4, 3072, 512, 16), (16, 4, 8192, 512, 8)],
                         ids=["T1", "T7", "T16", "I320_T16", "H3072_T16", "H8192_T8"])
def test_resident_matches_oracle(shape):
    E, k, H, I, T = shape
    log(f"resident {shape}")
    rm, ho, co = synth.random_map(E, E // 4, 7)
    hot, cold = host_bank(ho, 7, 0, H, I), host_bank(co, 7, 0, H, I)
    ids, w = synth.skewed_routing(T, k, E, 7, 0, 0)
    x = synth.activations(T, H, 7)
    _check(rm, hot, cold, ids, w, x, H, I)


def test_resident_full_pass_and_duplicates():
    """Expert 2 in every token's picks (16 slots: one full pass); expert 5 in
    every pick of tokens 0..15 of a second call (64 slots: four passes)."""
    E, k, H, I, T = 8, 4, 512, 256, 16
    rm, ho, co = synth.map_from_cold_set(E, [7])
    hot, cold = host_bank(ho, 9, 0, H, I), host_bank(co, 9, 0, H, I)
    x = synth.activations(T, H, 9)
    ids, w = synth.gaussian_routing(T, k, E, 9)
    for t in range(T):
        if 2 not in ids[t]:
            ids[t, t % k] = 2
    log("resident: expert with 16 slots")
    _check(rm, hot, cold, ids, w, x, H, I)
    ids_dup = np.full((T, k), 5, np.int32)
    log("resident: expert with 64 slots (duplicate ids)")
    _check(rm, hot, cold, ids_dup, np.full((T, k), 0.25, np.float32), x, H, I)


@pytest.mark.parametrize("where", ["device", "pinned_host"])
def test_resident_equals_decode_kernel_bitwise(where):
    """The first 4 tokens of a 20-token step (T > 16: decode kernel) and the
    same 4 tokens alone (resident kernel) give identical Y rows, with every
    expert in HBM or every expert in pinned host memory."""
    E, k, H, I, T = 24, 2, 4096, 2880, 20  # 40 picks on 24 rows: the decode kernels
    all_map, owners, _ = synth.all_hot_map(E)
    arrays = host_bank(owners, 13, 0, H, I)
    ids, w = synth.gaussian_routing(T, k, E, 13)
    x = synth.activations(T, H, 13)
    if where == "device":
        bank, rm, other = device_bank(arrays), all_map, None
        run = lambda n: run_layer(bank, other, rm, ids[:n], w[:n], x[:n], H, I)[0]
    else:
        empty = device_bank(host_bank(np.zeros(0, np.int32), 13, 0, H, I))
        bank, rm = pinned_bank(arrays), -1 - all_map  # every expert cold, same rows
        run = lambda n: run_layer(empty, bank, rm, ids[:n], w[:n], x[:n], H, I)[0]
    Y20, Y4 = run(T), run(4)
    assert np.array_equal(Y20[: 4 * k], Y4)


@pytest.mark.parametrize("shape", [(32, 6, 4096, 2880, 16), (16, 4, 8192, 512, 8)],
                         ids=["H4096_T16", "H8192_T8"])
def test_resident_host_bank_matches_oracle(shape):
    """Resident kernel reading a bank in pinned host memory, against the oracle
    (at H = 8192, above the host-bank kernels' limit, the cold bank's gate/up
    runs the resident kernel on the host bank's few CUs)."""
    E, k, H, I, T = shape
    rm, ho, co = synth.random_map(E, 8, 17)
    hot, cold = host_bank(ho, 17, 0, H, I), host_bank(co, 17, 0, H, I)
    ids, w = synth.skewed_routing(T, k, E, 17, 0, 0)
    x = synth.activations(T, H, 17)
    _check(rm, hot, cold, ids, w, x, H, I, cold_pinned=True)
