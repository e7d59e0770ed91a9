"""GPU parity of the persistent down kernel (a workgroup's h rows staged in
LDS, weights streamed continuously, per-item scale blocks).

The library runs it for the down GEMM of steps below the token-tiled range
when the chunk count of I is a multiple of the kernel's ring length (I = 1472,
1536, 2880 here) and the down-scale tensor is 16-byte aligned. It must match
the oracle within tolerance (relative L2 <= 1e-2, max relative <= 3e-2, every
slot on its own) and give the same bits as the decode down kernel, which runs
instead when the same scale bytes sit 2 bytes off 16-byte alignment:
  - against the oracle: I = 1472 (last chunk: 3 of 4 lane quarters in range),
    I = 1536, and decode steps at H = 4096, I = 2880;
  - bitwise against the decode kernel at full shape (T = 16), with one expert
    in all 24 tokens (two 16-column passes), and with 64 slots on each of 6
    experts at I = 1472 (more h rows than one workgroup's LDS holds: two
    phases);
  - the bank in pinned host memory (8 workgroups) against the same bank in HBM
    (all CUs but 8): the work split differs, the bits must not.
For a bank in HBM with a 128-byte aligned weight tensor, shapes whose rows
allow it (I = 2880, 2048, 1856 here) take line-aligned loads, each chunk put
together on chip from two lines; with the weight tensor 16 bytes off a line
the same bank takes the unaligned loads (I = 2880) or the decode down kernel
(I = 1856, whose 8 chunks are no multiple of the unaligned ring): same bits.
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


def offset_s2_bank(arrays: dict, off: int = 2) -> moe.Bank:
    """The bank in HBM with its down-scale tensor starting `off` bytes past a
    16-byte boundary (same bytes), which sends the down GEMM to the decode kernel."""
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in arrays.items()}
    s2 = np.ascontiguousarray(arrays["s2"])
    buf = torch.zeros(s2.size + 16, dtype=torch.uint8, device="cuda")
    view = buf[off:off + s2.size].view(s2.shape)
    view.copy_(torch.from_numpy(s2))
    assert view.data_ptr() % 16 == off
    return moe.Bank(t["w13"], t["s13"], t["w2"], view, on_host=False)


def offset_w2_bank(arrays: dict, off: int = 16) -> moe.Bank:
    """The bank in HBM with its down-weight tensor starting `off` bytes past a
    128-byte boundary (same bytes): no line-aligned loads for it."""
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in arrays.items()}
    w2 = np.ascontiguousarray(arrays["w2"])
    buf = torch.zeros(w2.size + 128, dtype=torch.uint8, device="cuda")
    view = buf[off:off + w2.size].view(w2.shape)
    view.copy_(torch.from_numpy(w2))
    assert view.data_ptr() % 128 == off
    return moe.Bank(t["w13"], t["s13"], view, t["s2"], on_host=False)


def _all_hot(E, seed, H, I):
    rm, owners, _ = synth.all_hot_map(E)
    return rm, host_bank(owners, seed, 0, H, I)


def _vs_oracle(rm, arrays, ids, w, x, H, I, Y):
    T, k = ids.shape
    empty = host_bank(np.zeros(0, np.int32), 0, 0, H, I)
    Yr, outr, bad = oracle.moe_layer(oracle_bank(arrays), oracle_bank(empty), rm, ids, w, x, H, I)
    assert bad == 0
    Yr = Yr.reshape(T * k, H)
    e = rel_errors(Y, Yr)
    log(f"  Y rel-L2 {e[0]:.2e} max-rel {e[1]:.2e}")
    assert e[0] <= REL_L2 and e[1] <= MAX_REL
    for s in range(T * k):
        r = rel_errors(Y[s], Yr[s])
        assert r[0] <= REL_L2, (s, r)


# banks large enough that every step stays below 2 picks per row (the token-tiled range)
@pytest.mark.parametrize("shape", [(48, 4, 1024, 1472, 16), (24, 4, 1024, 1536, 9),
                                   (64, 6, 4096, 2880, 16), (48, 6, 4096, 2880, 3),
                                   (48, 4, 1024, 2048, 16), (48, 4, 1024, 1856, 11)],
                         ids=["I1472_T16", "I1536_T9", "I2880_T16", "I2880_T3", "I2048_T16",
                              "I1856_T11"])
def test_down_resident_matches_oracle(shape):
    E, k, H, I, T = shape
    log(f"down resident vs oracle {shape}")
    rm, arrays = _all_hot(E, 21, H, I)
    ids, w = synth.skewed_routing(T, k, E, 21, 0, 0)
    x = synth.activations(T, H, 21)
    Y, _, ninv = run_layer(device_bank(arrays), None, rm, ids, w, x, H, I)
    assert ninv == 0
    _vs_oracle(rm, arrays, ids, w, x, H, I, Y)


def _bitwise_vs_decode(E, k, H, I, ids, w, x, seed, check_oracle=False):
    rm, arrays = _all_hot(E, seed, H, I)
    Yr, outr, _ = run_layer(device_bank(arrays), None, rm, ids, w, x, H, I)
    Yd, outd, _ = run_layer(offset_s2_bank(arrays), None, rm, ids, w, x, H, I)
    assert np.array_equal(Yr, Yd), "persistent and decode down kernels differ"
    assert np.array_equal(outr, outd)
    if check_oracle:
        _vs_oracle(rm, arrays, ids, w, x, H, I, Yr)
    return rm, arrays, Yr


def test_down_resident_equals_decode_full_shape():
    E, k, H, I, T = 64, 6, 4096, 2880, 16
    log("down resident == decode kernel, full shape T=16")
    ids, w = synth.skewed_routing(T, k, E, 23, 0, 0)
    x = synth.activations(T, H, 23)
    _bitwise_vs_decode(E, k, H, I, ids, w, x, 23)


def test_down_resident_two_passes():
    """Expert 3 in every one of 24 tokens: 24 slots, two 16-column passes."""
    E, k, H, I, T = 64, 4, 1024, 1472, 24  # 96 picks on 64 rows: below the token-tiled range
    log("down resident: 24 slots on one expert")
    ids, w = synth.gaussian_routing(T, k, E, 25)
    for t in range(T):
        if 3 not in ids[t]:
            ids[t, t % k] = 3
    x = synth.activations(T, H, 25)
    _bitwise_vs_decode(E, k, H, I, ids, w, x, 25, check_oracle=True)


def test_down_resident_two_phases():
    """Every token picks experts 0..5 (in rotating order): 64 slots per
    expert, more h rows than one workgroup's LDS holds at I = 1472 (49)."""
    E, k, H, I, T = 200, 6, 1024, 1472, 64  # 384 picks on 200 rows: below the token-tiled range
    log("down resident: 64 slots on each of 6 experts (two LDS phases)")
    ids = np.array([[(t + j) % 6 for j in range(k)] for t in range(T)], np.int32)
    w = np.full((T, k), 1.0 / k, np.float32)
    x = synth.activations(T, H, 27)
    _bitwise_vs_decode(E, k, H, I, ids, w, x, 27, check_oracle=True)


def test_down_resident_host_bank_equals_device_bank():
    """Pinned host bank (8 workgroups) and the same bank in HBM give the same bits."""
    E, k, H, I, T = 64, 6, 4096, 2880, 16
    log("down resident: pinned host bank == device bank")
    rm, arrays = _all_hot(E, 29, H, I)
    ids, w = synth.skewed_routing(T, k, E, 29, 0, 0)
    x = synth.activations(T, H, 29)
    Yd, _, _ = run_layer(device_bank(arrays), None, rm, ids, w, x, H, I)
    empty = device_bank(host_bank(np.zeros(0, np.int32), 29, 0, H, I))
    Yh, _, _ = run_layer(empty, pinned_bank(arrays), -1 - rm, ids, w, x, H, I)
    assert np.array_equal(Yd, Yh)


@pytest.mark.parametrize("shape", [(64, 6, 4096, 2880, 16), (48, 4, 1024, 1856, 11),
                                   (40, 4, 1024, 2048, 7)],
                         ids=["I2880_T16", "I1856_T11", "I2048_T7"])
def test_down_aligned_loads_equal_unaligned(shape):
    """Line-aligned loads (weight tensor on a 128-byte boundary) give the bits
    of the same bank with its weight tensor 16 bytes off a line."""
    E, k, H, I, T = shape
    log(f"down aligned == unaligned weight tensor {shape}")
    rm, arrays = _all_hot(E, 31, H, I)
    ids, w = synth.skewed_routing(T, k, E, 31, 0, 0)
    x = synth.activations(T, H, 31)
    Ya, outa, _ = run_layer(device_bank(arrays), None, rm, ids, w, x, H, I)
    Yu, outu, _ = run_layer(offset_w2_bank(arrays), None, rm, ids, w, x, H, I)
    assert np.array_equal(Ya, Yu) and np.array_equal(outa, outu)
