"""One MoE layer with hot/cold residency, as a sequence of ABI calls.

Holds the two banks, the device row map and the preallocated split, workspace
and output buffers for a given token count, and issues, per step:
moe_route_split -> moe_expert_ffn_mxfp4 (hot) -> moe_expert_ffn_mxfp4 (cold,
optionally after moe_stage_rows into an HBM stage) -> moe_finalize ("vLLM: Pin Hot Experts", section "Results, September 17":
split the ids by residency, one routed call per bank without finalization,
one ordered finalize). The cold call may run on a second stream: the two calls
write disjoint slots, so the result does not depend on the overlap. Nothing
here computes; it only sequences the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (Bank, Split, moe_expert_ffn_mxfp4, moe_ffn_workspace_bytes, moe_finalize,
               moe_route_split, moe_stage_rows)


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


class ColdStage:
    """A device bank the step's active cold rows are copied into before the
    cold FFN (moe_stage_rows), with its row list. Rows: at least min(cold
    rows, T*k) of the largest step; one stage can serve every layer in turn."""

    def __init__(self, n_rows: int, H: int, I: int, device="cuda"):
        shapes = {"w13": (n_rows, 2 * I, H // 2), "s13": (n_rows, 2 * I, H // 32),
                  "w2": (n_rows, H, I // 2), "s2": (n_rows, H, I // 32)}
        t = {k: torch.empty(sh, dtype=torch.uint8, device=device) for k, sh in shapes.items()}
        self.bank = Bank(t["w13"], t["s13"], t["w2"], t["s2"], on_host=False)
        self.rows = torch.zeros(max(n_rows, 1), dtype=torch.int32, device=device)


class ResidencyLayer:
    def __init__(self, hot: Bank, cold: Bank, row_map: torch.Tensor, H: int, I: int,
                 stage: ColdStage | None = None):
        """With `stage`, the cold bank's active rows are copied to it in one
        contiguous stream per row and the cold FFN reads them from HBM."""
        self.hot, self.cold, self.row_map, self.H, self.I = hot, cold, row_map, H, I
        self.stage = stage

    def _cold_ffn(self, x, k, bufs, stream):
        if self.stage is None:
            moe_expert_ffn_mxfp4(self.cold, bufs.cold_split, x, k, self.I, bufs.workspace, bufs.Y,
                                 stream=stream)
            return
        T = int(x.shape[0])
        staged = moe_stage_rows(self.cold, bufs.cold_split, T, k, self.stage.bank, self.stage.rows,
                                self.H, self.I, stream=stream)
        moe_expert_ffn_mxfp4(self.stage.bank, staged, x, k, self.I, bufs.workspace, bufs.Y,
                             stream=stream)

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
            self._cold_ffn(x, k, bufs, s)
        else:
            # cold first: its few workgroups start at once beside the hot bank's
            cold_stream.wait_stream(s)
            self._cold_ffn(x, k, bufs, cold_stream)
            moe_expert_ffn_mxfp4(self.hot, bufs.hot_split, x, k, self.I, bufs.workspace, bufs.Y,
                                 stream=s)
            s.wait_stream(cold_stream)
        moe_finalize(bufs.Y, topk_w, bufs.out, stream=s)
        return bufs.out
