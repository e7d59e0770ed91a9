"""A whole residency layer captured as a HIP graph and replayed.

One layer step (split with the usage counter, the cold path staged in two
parts with its gate/up GEMM on the stage's stream, the hot FFN on a side
stream, finalize) is captured once, reading fixed input buffers. Each replay,
with new inputs copied in and eager work and synchronisations between
replays, must give exactly the bits the same layer gives when run eagerly on
those inputs, and the counter must grow by one histogram per replay.
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


def test_layer_graph_replays_match_eager():
    E, k, H, I, T, n_cold = 32, 4, 1024, 1536, 12, 10
    rm_np, ho, co = synth.random_map(E, n_cold, 41)
    hot = device_bank(host_bank(ho, 41, 0, H, I))
    cold = pinned_bank(host_bank(co, 41, 0, H, I))
    rm = torch.from_numpy(rm_np).cuda()
    stage = ColdStage(min(n_cold, T * k), H, I)
    layer = ResidencyLayer(hot, cold, rm, H, I, stage=stage)
    inputs = []
    for step in range(4):
        ids, w = synth.skewed_routing(T, k, E, 41, 0, step)
        x = synth.activations(T, H, 41, 0, step)
        inputs.append(routing_tensors(ids, w, x))
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")

    # eager reference for every input
    bufs = LayerBuffers.allocate(T, k, H, I, hot.n_rows, cold.n_rows)
    want = []
    for ids_d, w_d, x_d in inputs:
        layer.forward(x_d, ids_d, w_d, bufs, stream=main, hot_stream=side)
        main.synchronize()
        want.append(bufs.out[:T].cpu().numpy().copy())

    # capture once on fixed buffers
    ids_st, w_st, x_st = (t.clone() for t in inputs[0])
    gbufs = LayerBuffers.allocate(T, k, H, I, hot.n_rows, cold.n_rows)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=main):
        layer.forward(x_st, ids_st, w_st, gbufs, counts_layer=counts, stream=main,
                      hot_stream=side)
    torch.cuda.synchronize()
    assert int(counts.sum()) == 0, "capture must not execute"

    hist = np.zeros(E, np.int64)
    for rep, (ids_d, w_d, x_d) in enumerate(inputs[1:] + inputs[:1]):
        idx = (rep + 1) % len(inputs)
        ids_st.copy_(ids_d)
        w_st.copy_(w_d)
        x_st.copy_(x_d)
        junk = torch.randn(4096, device="cuda").sum()   # eager work between replays
        with torch.cuda.stream(main):
            g.replay()
        torch.cuda.synchronize()
        got = gbufs.out[:T].cpu().numpy()
        log(f"replay {rep} (input {idx})")
        assert np.array_equal(got, want[idx]), f"replay {rep} differs from eager"
        hist += np.bincount(ids_d.cpu().numpy().ravel(), minlength=E)
        assert np.array_equal(counts.cpu().numpy(), hist), rep
        del junk
