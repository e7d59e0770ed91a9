"""Helpers shared by the GPU tests: build banks on the device / pinned host
from the seeded generators, run one layer through the C ABI, and measure
errors against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import expert_weight_residency_amd as moe
import oracle
import synth
from expert_weight_residency_amd.layer import LayerBuffers, ResidencyLayer

# FFN tolerance against the fp32 oracle (relative L2 over the tensor and
# max-abs error relative to max-abs reference)
REL_L2 = 1e-2
MAX_REL = 3e-2


def rel_errors(got_bits: np.ndarray, ref_bits: np.ndarray):
    g = oracle.bf16_to_f32(got_bits).astype(np.float64)
    r = oracle.bf16_to_f32(ref_bits).astype(np.float64)
    d = g - r
    rl2 = float(np.linalg.norm(d) / max(np.linalg.norm(r), 1e-300))
    mr = float(np.abs(d).max() / max(np.abs(r).max(), 1e-300)) if d.size else 0.0
    return rl2, mr


def host_bank(owners, seed, layer, H, I, **kw):
    return synth.make_bank_host(owners, seed, layer, H, I, **kw)


def device_bank(arrays: dict, device="cuda") -> moe.Bank:
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in arrays.items()}
    return moe.Bank(t["w13"], t["s13"], t["w2"], t["s2"], on_host=False)


def pinned_bank(arrays: dict) -> moe.Bank:
    t = {}
    for k, v in arrays.items():
        p = torch.empty(v.shape, dtype=torch.uint8, pin_memory=True)
        p.numpy()[...] = v
        t[k] = p
    return moe.Bank(t["w13"], t["s13"], t["w2"], t["s2"], on_host=True)


def empty_bank_host(n_rows, H, I, pinned=False, device=None):
    shapes = synth.tensor_shapes(n_rows, H, I)
    if device is not None:
        t = {k: torch.empty(s, dtype=torch.uint8, device=device) for k, s in shapes.items()}
    else:
        t = {k: torch.empty(s, dtype=torch.uint8, pin_memory=pinned) for k, s in shapes.items()}
    return moe.Bank(t["w13"], t["s13"], t["w2"], t["s2"], on_host=(device is None))


def oracle_bank(arrays: dict) -> oracle.Bank:
    return oracle.Bank(arrays["w13"], arrays["s13"], arrays["w2"], arrays["s2"])


def routing_tensors(ids: np.ndarray, w: np.ndarray, x: np.ndarray, device="cuda"):
    return (torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(device),
            torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(device),
            torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device))


def run_layer(hot: moe.Bank, cold: moe.Bank, row_map: np.ndarray, ids, w, x, H, I,
              counts_layer=None, cold_stream=None):
    """One layer through the ABI; returns (Y bits [T*k,H], out bits [T,H], n_invalid)."""
    T, k = ids.shape
    rm = torch.from_numpy(np.ascontiguousarray(row_map, np.int32)).cuda()
    ids_d, w_d, x_d = routing_tensors(ids, w, x)
    bufs = LayerBuffers.allocate(T, k, H, I, hot.n_rows, cold.n_rows if cold else 0)
    if cold is None:
        cold = empty_bank_host(0, H, I, device="cuda")
        cold.on_host = False
    layer = ResidencyLayer(hot, cold, rm, H, I)
    layer.forward(x_d, ids_d, w_d, bufs, counts_layer=counts_layer, cold_stream=cold_stream)
    torch.cuda.synchronize()
    Y = bufs.Y[: T * k].cpu().numpy().view(np.uint16).copy()
    out = bufs.out[:T].cpu().numpy().view(np.uint16).copy()
    return Y, out, int(bufs.n_invalid.item())
