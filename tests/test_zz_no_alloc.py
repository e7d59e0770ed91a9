"""moe_expert_ffn_mxfp4_noalloc (the FFN entry point that takes no workspace
and allocates nothing: its intermediate rows live in the library's static
per-device scratch buffer) against moe_expert_ffn_mxfp4 with a caller's
workspace, bit for bit, through the C ABI: two calls in a row, the second on
a smaller step (the buffer still holds the first call's rows), for a hot bank
in HBM and a cold bank read in place from pinned memory, on the decode,
token-tiled and FP4 prefill kernel families; and a step too large for the
buffer is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import expert_weight_residency_amd as moe
import synth
from gpu_util import device_bank, host_bank, pinned_bank

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield


def _step(E, k, H, I, T, n_cold, seed):
    rm, ho, co = synth.random_map(E, n_cold, seed)
    hot, cold = device_bank(host_bank(ho, seed, 0, H, I)), pinned_bank(host_bank(co, seed, 0, H, I))
    ids, _ = synth.skewed_routing(T, k, E, seed, 0, 0)
    x = torch.from_numpy(synth.activations(T, H, seed).view(np.int16)).cuda()
    hs, cs = moe.Split.empty(len(ho), T, k), moe.Split.empty(len(co), T, k)
    ninv = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_route_split(torch.from_numpy(ids).cuda(), torch.from_numpy(rm).cuda(), len(ho),
                        len(co), hs, cs, ninv)
    return hot, cold, hs, cs, x


def _both(hot, cold, hs, cs, x, k, H, I):
    T = int(x.shape[0])
    ws = torch.empty(max(moe.moe_ffn_workspace_bytes(T, k, H, I), 16), dtype=torch.uint8,
                     device="cuda")
    Y_ref = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    Y_na = torch.full((T * k, H), 0x7FC1, dtype=torch.int16, device="cuda")  # no stale zeros
    for bank, split in ((hot, hs), (cold, cs)):
        moe.moe_expert_ffn_mxfp4(bank, split, x, k, I, ws, Y_ref)
    for bank, split in ((hot, hs), (cold, cs)):
        moe.moe_expert_ffn_mxfp4_noalloc(bank, split, x, k, I, Y_na)
    torch.cuda.synchronize()
    return Y_ref, Y_na


@pytest.mark.parametrize("family,big,small", [
    # (E, k, H, I, T, n_cold): first call, then a smaller second call
    ("decode", (64, 4, 1024, 512, 12, 16), (16, 2, 256, 128, 5, 4)),
    ("tiled", (24, 3, 512, 320, 200, 6), (24, 3, 512, 320, 40, 6)),
    ("fp4_prefill", (32, 2, 512, 320, 300, 8), (32, 2, 512, 320, 256, 8)),
    ("full_shape", (64, 6, 4096, 2880, 16, 16), (64, 6, 4096, 2880, 7, 16)),
])
def test_noalloc_equals_workspace_call(family, big, small):
    for n, (E, k, H, I, T, n_cold) in enumerate((big, small)):
        print(f"no-alloc {family} call {n}: E={E} k={k} H={H} I={I} T={T}", flush=True)
        hot, cold, hs, cs, x = _step(E, k, H, I, T, n_cold, 40 + n)
        Y_ref, Y_na = _both(hot, cold, hs, cs, x, k, H, I)
        assert torch.equal(Y_ref, Y_na), (family, n)
        assert bool((Y_ref != 0).any())


def test_noalloc_refuses_oversize_step():
    E, k, H, I = 16, 6, 4096, 2880
    T = 400  # FP4 path: 400 * 6 * 28 * 528 bytes > 32 MiB
    assert moe.moe_ffn_workspace_bytes(T, k, H, I) > moe.MOE_NOALLOC_SCRATCH_BYTES
    bank = moe.Bank(*[torch.empty(s, dtype=torch.uint8, device="cuda")
                      for s in synth.tensor_shapes(2, H, I).values()])
    split = moe.Split.empty(2, T, k)
    x = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    Y = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_expert_ffn_mxfp4_noalloc(bank, split, x, k, I, Y)
    assert e.value.code == moe.MOE_EINVAL and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not bool(Y.any())
