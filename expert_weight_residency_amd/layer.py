"""One MoE layer with hot/cold residency, as a sequence of ABI calls.

Holds the two banks, the device row map and the preallocated split, workspace
and output buffers for a given token count, and issues, per step:
moe_route_split -> moe_expert_ffn_mxfp4 (hot) -> moe_expert_ffn_mxfp4 (cold)
-> moe_finalize ("vLLM: Pin Hot Experts", section "Results, September 17":
split the ids by residency, one routed call per bank without finalization,
one ordered finalize). The cold call may run on a second stream: the two calls
write disjoint slots, so the result does not depend on the overlap. Nothing
here computes; it only sequences the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (Bank, Split, moe_expert_ffn_mxfp4, moe_ffn_workspace_bytes, moe_finalize,
               moe_route_split)


@dataclass
class LayerBuffers:
    hot_split: Split
    cold_split: Split
    n_invalid: torch.Tensor
    workspace: torch.Tensor
    Y: torch.Tensor
    out: torch.Tensor

    @classmethod
    def allocate(cls, T: int, k: int, H: int, I: int, n_hot: int, n_cold: int, device="cuda"):
        ws = max(moe_ffn_workspace_bytes(T, k, I), 16)
        return cls(Split.empty(n_hot, T, k, device), Split.empty(n_cold, T, k, device),
                   torch.zeros(1, dtype=torch.int32, device=device),
                   torch.empty(ws, dtype=torch.uint8, device=device),
                   torch.empty((max(T * k, 1), H), dtype=torch.int16, device=device),
                   torch.empty((max(T, 1), H), dtype=torch.int16, device=device))


class ResidencyLayer:
    def __init__(self, hot: Bank, cold: Bank, row_map: torch.Tensor, H: int, I: int):
        self.hot, self.cold, self.row_map, self.H, self.I = hot, cold, row_map, H, I

    def forward(self, x, topk_ids, topk_w, bufs: LayerBuffers, counts_layer=None,
                count_tmax: int = 256, stream=None, cold_stream=None):
        """x bf16 [T,H] (as int16 or bfloat16), topk_ids int32 [T,k], topk_w fp32
        [T,k] -> bufs.out [T,H] bf16 bits. All on `stream` (default: current);
        with cold_stream, the cold FFN runs there between two event waits."""
        k = int(topk_ids.shape[1])
        s = stream if stream is not None else torch.cuda.current_stream()
        moe_route_split(topk_ids, self.row_map, self.hot.n_rows, self.cold.n_rows, bufs.hot_split,
                        bufs.cold_split, bufs.n_invalid, counts_layer, count_tmax, stream=s)
        if cold_stream is None:
            moe_expert_ffn_mxfp4(self.hot, bufs.hot_split, x, k, self.I, bufs.workspace, bufs.Y,
                                 stream=s)
            moe_expert_ffn_mxfp4(self.cold, bufs.cold_split, x, k, self.I, bufs.workspace, bufs.Y,
                                 stream=s)
        else:
            cold_stream.wait_stream(s)
            moe_expert_ffn_mxfp4(self.hot, bufs.hot_split, x, k, self.I, bufs.workspace, bufs.Y,
                                 stream=s)
            moe_expert_ffn_mxfp4(self.cold, bufs.cold_split, x, k, self.I, bufs.workspace, bufs.Y,
                                 stream=cold_stream)
            s.wait_stream(cold_stream)
        moe_finalize(bufs.Y, topk_w, bufs.out, stream=s)
        return bufs.out
