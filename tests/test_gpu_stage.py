"""GPU tests of moe_stage_rows: the cold bank's active rows copied into a
compact HBM bank before the cold FFN.

Bit-exact: the staged rows equal the source rows the split names, the staged
row list is 0..n_active-1, staging one part (gate/up or down tensors) leaves
the other untouched, and a layer run through the stage gives the same Y rows
and output as the in-place run (small shape on one stream and with either
bank's FFN on a side stream, and the full shape with the fitted map and 16
decode tokens), including a step with no cold picks.
"""
import numpy as np
import pytest
import torch

import expert_weight_residency_amd as moe
import synth
from expert_weight_residency_amd.layer import ColdStage, LayerBuffers, ResidencyLayer
from gpu_util import device_bank, host_bank, pinned_bank, routing_tensors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield


def log(msg):
    print(msg, flush=True)


def _run(hot, cold, rm, ids, w, x, H, I, stage, cold_stream=None, hot_stream=None):
    T, k = ids.shape
    ids_d, w_d, x_d = routing_tensors(ids, w, x)
    bufs = LayerBuffers.allocate(T, k, H, I, hot.n_rows, cold.n_rows)
    layer = ResidencyLayer(hot, cold, torch.from_numpy(rm).cuda(), H, I, stage=stage)
    layer.forward(x_d, ids_d, w_d, bufs, cold_stream=cold_stream, hot_stream=hot_stream)
    torch.cuda.synchronize()
    return (bufs.Y[: T * k].cpu().numpy().copy(), bufs.out[:T].cpu().numpy().copy(), bufs)


def test_stage_copies_named_rows():
    E, k, H, I, T = 24, 3, 512, 320, 12
    rm, ho, co = synth.random_map(E, 9, 3)
    cold_arr = host_bank(co, 3, 0, H, I)
    cold = pinned_bank(cold_arr)
    ids, _ = synth.skewed_routing(T, k, E, 3, 0, 0)
    hs, cs = moe.Split.empty(E - 9, T, k), moe.Split.empty(9, T, k)
    ninv = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_route_split(torch.from_numpy(ids).cuda(), torch.from_numpy(rm).cuda(), E - 9, 9, hs, cs,
                        ninv)
    stage = ColdStage(min(9, T * k), H, I)
    stage.rows.fill_(-5)
    staged = moe.moe_stage_rows(cold, cs, T, k, stage.bank, stage.rows, H, I)
    torch.cuda.synchronize()
    active, _, _ = cs.to_host()
    n = len(active)
    log(f"{n} active cold rows")
    assert n > 0
    assert np.array_equal(staged.active_rows[:n].cpu().numpy(), np.arange(n))
    for name in ("w13", "s13", "w2", "s2"):
        got = getattr(stage.bank, name)[:n].cpu().numpy()
        assert np.array_equal(got, cold_arr[name][active]), name


@pytest.mark.parametrize("streams", ["one", "cold_side", "hot_side"])
def test_staged_layer_equals_in_place_bitwise(streams):
    """The staged cold path (on two streams: gate/up tensors staged first, the
    gate/up GEMM on them beside the copy of the down tensors) gives the bits of
    the in-place path, whichever bank's FFN runs on the side stream."""
    E, k, H, I, T = 32, 4, 1024, 512, 24
    rm, ho, co = synth.random_map(E, 10, 5)
    hot = device_bank(host_bank(ho, 5, 0, H, I))
    cold = pinned_bank(host_bank(co, 5, 0, H, I))
    ids, w = synth.skewed_routing(T, k, E, 5, 0, 0)
    x = synth.activations(T, H, 5)
    side = {"cold_stream": torch.cuda.Stream()} if streams == "cold_side" else (
        {"hot_stream": torch.cuda.Stream()} if streams == "hot_side" else {})
    log(f"staged layer, streams={streams}")
    Y0, o0, _ = _run(hot, cold, rm, ids, w, x, H, I, None)
    Y1, o1, _ = _run(hot, cold, rm, ids, w, x, H, I, ColdStage(min(10, T * k), H, I), **side)
    assert np.array_equal(Y0, Y1) and np.array_equal(o0, o1)


def test_stage_parts():
    """Staging the gate/up tensors leaves the down tensors of the stage
    untouched; staging the down tensors then completes the rows."""
    E, k, H, I, T = 24, 3, 512, 320, 12
    rm, ho, co = synth.random_map(E, 9, 31)
    cold_arr = host_bank(co, 31, 0, H, I)
    cold = pinned_bank(cold_arr)
    ids, _ = synth.skewed_routing(T, k, E, 31, 0, 0)
    hs, cs = moe.Split.empty(E - 9, T, k), moe.Split.empty(9, T, k)
    ninv = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_route_split(torch.from_numpy(ids).cuda(), torch.from_numpy(rm).cuda(), E - 9, 9, hs, cs,
                        ninv)
    stage = ColdStage(min(9, T * k), H, I)
    for t in stage.bank.tensors().values():
        t.fill_(0xA5)
    moe.moe_stage_rows(cold, cs, T, k, stage.bank, stage.rows, H, I, parts=moe.STAGE_GATE_UP)
    torch.cuda.synchronize()
    active, _, _ = cs.to_host()
    n = len(active)
    assert n > 0
    for name in ("w13", "s13"):
        assert np.array_equal(getattr(stage.bank, name)[:n].cpu().numpy(), cold_arr[name][active])
    for name in ("w2", "s2"):
        assert (getattr(stage.bank, name).cpu().numpy() == 0xA5).all(), name
    moe.moe_stage_rows(cold, cs, T, k, stage.bank, stage.rows, H, I, parts=moe.STAGE_DOWN)
    torch.cuda.synchronize()
    for name in ("w13", "s13", "w2", "s2"):
        assert np.array_equal(getattr(stage.bank, name)[:n].cpu().numpy(), cold_arr[name][active])


def test_staged_full_shape_decode_bitwise():
    E, k, H, I, T, n_cold = 384, 6, 4096, 2880, 16, 89
    rm, ho, co = synth.fitted_map(E, n_cold, 7, 0)
    hb = moe.Bank(*[torch.empty(s, dtype=torch.uint8, device="cuda")
                    for s in synth.tensor_shapes(len(ho), H, I).values()], on_host=False)
    synth.fill_bank_device(hb.tensors(), torch.from_numpy(ho).cuda(), 7, 0, H, I)
    cb = moe.Bank(*[torch.empty(s, dtype=torch.uint8, pin_memory=True)
                    for s in synth.tensor_shapes(n_cold, H, I).values()], on_host=True)
    synth.fill_bank_host(cb.tensors(), co, 7, 0, H, I)
    stage = ColdStage(min(n_cold, T * k), H, I)
    for step in range(3):
        ids, w = synth.skewed_routing(T, k, E, 7, 0, step)
        if step == 2:  # no cold picks at all
            hot_ids = ho[:E - n_cold]
            ids = hot_ids[np.arange(T * k).reshape(T, k) % len(hot_ids)].astype(np.int32)
        x = synth.activations(T, H, 7, 0, step)
        n_cold_picks = int((rm[ids] < 0).sum())
        log(f"full shape step {step}: {n_cold_picks} cold picks")
        side = "hot_stream" if step == 1 else "cold_stream"
        Y0, o0, _ = _run(hb, cb, rm, ids, w, x, H, I, None, **{side: torch.cuda.Stream()})
        Y1, o1, _ = _run(hb, cb, rm, ids, w, x, H, I, stage, **{side: torch.cuda.Stream()})
        assert np.array_equal(Y0, Y1) and np.array_equal(o0, o1)


def test_dma_stage_equals_kernel_stage_and_in_place():
    """moe_stage_rows_dma (the DMA engines, from the active rows read back to
    the host) copies the same bytes as moe_stage_rows, and the layer run
    through it gives the bits of the in-place run; a second call with fewer
    cold picks reuses the stage."""
    E, k, H, I = 32, 4, 1024, 512
    rm, ho, co = synth.random_map(E, 10, 7)
    hot = device_bank(host_bank(ho, 7, 0, H, I))
    cold_arr = host_bank(co, 7, 0, H, I)
    cold = pinned_bank(cold_arr)
    for T, seed in ((24, 0), (5, 1)):
        ids, w = synth.skewed_routing(T, k, E, 7, 0, seed)
        x = synth.activations(T, H, 7 + seed)
        log(f"dma stage: T={T}")
        Y0, out0, _ = _run(hot, cold, rm, ids, w, x, H, I, None)
        stage = ColdStage(min(10, T * k), H, I, dma=True)
        Y1, out1, bufs = _run(hot, cold, rm, ids, w, x, H, I, stage)
        assert np.array_equal(Y1, Y0) and np.array_equal(out1, out0)
        active, _, _ = bufs.cold_split.to_host()
        n = len(active)
        assert n == int(stage.n_host[0])
        for name in ("w13", "s13", "w2", "s2"):
            got = getattr(stage.bank, name)[:n].cpu().numpy()
            assert np.array_equal(got, cold_arr[name][active]), name
        # the kernel copy of the same rows gives the same stage bytes
        kstage = ColdStage(min(10, T * k), H, I)
        moe.moe_stage_rows(cold, bufs.cold_split, T, k, kstage.bank, kstage.rows, H, I)
        torch.cuda.synchronize()
        for name in ("w13", "s13", "w2", "s2"):
            assert torch.equal(getattr(kstage.bank, name)[:n], getattr(stage.bank, name)[:n])


def test_host_weights_bank_in_place_and_staged():
    """A cold bank with its weights pinned on the host and its scales in HBM
    gives, in place, staged by the kernel and staged by the DMA engines, the
    bits of the all-host cold bank in place."""
    E, k, H, I = 32, 4, 1024, 512
    rm, ho, co = synth.random_map(E, 10, 9)
    hot = device_bank(host_bank(ho, 9, 0, H, I))
    cold_arr = host_bank(co, 9, 0, H, I)
    cold = pinned_bank(cold_arr)
    w, s = pinned_bank(cold_arr), device_bank(cold_arr)
    split_cold = moe.Bank(w.w13, s.s13, w.w2, s.s2, on_host=moe.BANK_HOST_WEIGHTS)
    for T, seed in ((16, 0), (40, 1)):
        ids, wt = synth.skewed_routing(T, k, E, 9, 0, seed)
        x = synth.activations(T, H, 9 + seed)
        log(f"host-weights cold bank: T={T}")
        Y0, out0, _ = _run(hot, cold, rm, ids, wt, x, H, I, None)
        Y1, out1, _ = _run(hot, split_cold, rm, ids, wt, x, H, I, None)
        assert np.array_equal(Y1, Y0) and np.array_equal(out1, out0)
        for dma in (False, True):
            stage = ColdStage(min(10, T * k), H, I, dma=dma)
            Y2, out2, _ = _run(hot, split_cold, rm, ids, wt, x, H, I, stage)
            assert np.array_equal(Y2, Y0) and np.array_equal(out2, out0), dma
