"""GPU parity of the token-tiled expert FFN (steps with many picks per row).

Below 256 tokens per step the library runs the token-tiled kernels when a call
averages at least 2 picks per launchable bank row, and the decode kernels
otherwise; both are meant to give the same bits for every pick (steps of 256
tokens and more take the FP4 path, tested in test_gpu_fp4.py). Every step
here has fewer than 256 tokens. Checked here:
  - the tiled path against the oracle (relative L2 <= 1e-2, max relative
    <= 3e-2, every slot on its own), on shapes with reduction tails (K = 320,
    192, 64), tiles of 1..130 tokens (partial column groups, several tiles per
    expert), a pinned-host cold bank, and full H = 4096, I = 2880;
  - split == unsplit, bitwise, on the tiled path;
  - the two kernel families against each other, bitwise: a step of many
    tokens (tiled) and the step of its first few tokens (decode) give the same
    Y rows for the slots they share, since a pick's row depends only on its
    expert and its token's activations.
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

TILED_MIN_PICKS_PER_ROW = 2  # the library's switch-over (average picks per launchable row)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield


def log(msg):
    print(msg, flush=True)


def tiled(T, k, n_rows):
    return T * k >= TILED_MIN_PICKS_PER_ROW * min(n_rows, T * k)


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


def _counts_case(counts, H, I, seed):
    """k = 1; expert e gets counts[e] consecutive tokens; expert 0 is cold."""
    E = len(counts)
    rm, ho, co = synth.map_from_cold_set(E, [0])
    hot, cold = host_bank(ho, seed, 0, H, I), host_bank(co, seed, 0, H, I)
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])[:, None]
    w = np.ones_like(ids, dtype=np.float32)
    x = synth.activations(len(ids), H, seed)
    return rm, ho, co, hot, cold, ids, w, x


def _check_vs_oracle(rm, hot, cold, ids, w, x, H, I, cold_pinned):
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
    return Y, out


TILED_CASES = [
    # name, E, k, H, I, T, n_cold, routing, cold pinned
    ("small", 16, 2, 256, 128, 255, 4, "gaussian", False),
    ("ragged_K320_I192", 8, 2, 320, 192, 200, 2, "skewed", True),
    ("K64", 4, 1, 64, 64, 100, 1, "gaussian", False),
    ("mid_skewed", 64, 4, 1024, 512, 250, 16, "skewed", True),
]


@pytest.mark.parametrize("case", TILED_CASES, ids=[c[0] for c in TILED_CASES])
def test_tiled_matches_oracle(case):
    name, E, k, H, I, T, n_cold, routing, pinned = case
    log(f"tiled case {name}")
    rm, ho, co, hot, cold, ids, w, x = _case(E, k, H, I, T, n_cold, 61, routing)
    assert tiled(T, k, len(ho)) and tiled(T, k, len(co))
    _check_vs_oracle(rm, hot, cold, ids, w, x, H, I, pinned)


def test_tiled_tile_sizes():
    """Experts with 1, 5, 15, 16, 17, 63, 64 and 65 tokens: partial column
    groups, exact tiles, and an expert spanning two tiles (255 tokens)."""
    counts = [9, 1, 15, 16, 17, 63, 64, 65, 5]
    H, I = 512, 256
    rm, ho, co, hot, cold, ids, w, x = _counts_case(counts, H, I, 71)
    assert tiled(len(ids), 1, len(ho))
    log(f"tiled tile sizes {counts}")
    _check_vs_oracle(rm, hot, cold, ids, w, x, H, I, True)


def test_tiled_full_shape():
    """H = 4096, I = 2880 with 4 experts and 48 tokens of top-2 (24 picks per row)."""
    E, k, H, I, T = 4, 2, 4096, 2880, 48
    rm, ho, co, hot, cold, ids, w, x = _case(E, k, H, I, T, 1, 81, "gaussian")
    assert tiled(T, k, len(ho))
    log("tiled full shape")
    _check_vs_oracle(rm, hot, cold, ids, w, x, H, I, True)


@pytest.mark.parametrize("shape", [(16, 2, 512, 256, 240), (8, 2, 4096, 2880, 128)],
                         ids=["H512", "H4096"])
def test_tiled_equals_decode_bitwise(shape):
    """Same picks through both kernel families give identical Y rows."""
    E, k, H, I, T = shape
    rm, ho, co, hot, cold, ids, w, x = _case(E, k, H, I, T, 2, 91, "gaussian")
    small = 4
    assert tiled(T, k, len(ho)) and not tiled(small, k, len(ho))
    hb = device_bank(hot)
    Yt, _, _ = run_layer(hb, device_bank(cold), rm, ids, w, x, H, I)
    Yd, _, _ = run_layer(hb, device_bank(cold), rm, ids[:small], w[:small], x[:small], H, I)
    assert np.array_equal(Yt[: small * k], Yd)


def test_tiled_split_equals_unsplit():
    """Bitwise split (hot in HBM + cold pinned) == unsplit (all rows in one
    HBM bank) with every bank call on the tiled path."""
    E, k, H, I, T, seed = 16, 2, 512, 256, 250, 101
    rm, ho, co, hot, cold, ids, w, x = _case(E, k, H, I, T, 4, seed, "skewed")
    assert tiled(T, k, len(ho)) and tiled(T, k, len(co)) and tiled(T, k, E)
    Ys, outs, _ = run_layer(device_bank(hot), pinned_bank(cold), rm, ids, w, x, H, I)
    all_map, all_owner, _ = synth.all_hot_map(E)
    Yu, outu, _ = run_layer(device_bank(host_bank(all_owner, seed, 0, H, I)), None, all_map, ids,
                            w, x, H, I)
    assert np.array_equal(Ys, Yu) and np.array_equal(outs, outu)
