"""One MoE layer with hot/cold residency, as a sequence of ABI calls.

Holds the two banks, the device row map and the preallocated split, workspace
and output buffers for a given token count, and issues, per step:
moe_route_split -> moe_expert_ffn_mxfp4 (hot) -> moe_expert_ffn_mxfp4 (cold,
optionally after moe_stage_rows, or moe_stage_rows_dma, into an HBM stage) ->
moe_finalize ("vLLM: Pin
Hot Experts", section "Results, September 17": split the ids by residency, one
routed call per bank without finalization, one ordered finalize). The cold
call may run on a second stream (and, with a stage, its gate/up GEMM beside
the copy of the down tensors): the calls write disjoint slots, so the result
does not depend on the overlap. Nothing here computes; it only sequences the
library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (STAGE_ALL, STAGE_DOWN, STAGE_GATE_UP, Bank, Split, moe_expert_down_mxfp4,
               moe_expert_ffn_mxfp4, moe_expert_gate_up_mxfp4, moe_ffn_workspace_bytes,
               moe_finalize, moe_route_split, moe_stage_rows, moe_stage_rows_dma)


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
        ws = max(moe_ffn_workspace_bytes(T, k, H, I), 16)
        return cls(Split.empty(n_hot, T, k, device), Split.empty(n_cold, T, k, device),
                   torch.zeros(1, dtype=torch.int32, device=device),
                   torch.empty(ws, dtype=torch.uint8, device=device),
                   torch.empty((max(T * k, 1), H), dtype=torch.int16, device=device),
                   torch.empty((max(T, 1), H), dtype=torch.int16, device=device))


class ColdStage:
    """A device bank the step's active cold rows are copied into before the
    cold FFN (moe_stage_rows), with its row list. Rows: at least min(cold
    rows, T*k) of the largest step; one stage can serve every layer in turn.
    dma: copy with the DMA engines (moe_stage_rows_dma) from a row list read
    back to the host after the split, instead of the copy kernel."""

    def __init__(self, n_rows: int, H: int, I: int, device="cuda", dma: bool = False):
        self.dma = dma
        if dma:
            # the DMA copy needs the active rows on the host: read back after
            # the split into pinned buffers; the staged split's row list is
            # then 0 .. n-1 once and for all
            self.n_host = torch.zeros(1, dtype=torch.int32, pin_memory=True)
            self.rows_host = torch.zeros(max(n_rows, 1), dtype=torch.int32, pin_memory=True)
        shapes = {"w13": (n_rows, 2 * I, H // 2), "s13": (n_rows, 2 * I, H // 32),
                  "w2": (n_rows, H, I // 2), "s2": (n_rows, H, I // 32)}
        t = {k: torch.empty(sh, dtype=torch.uint8, device=device) for k, sh in shapes.items()}
        self.bank = Bank(t["w13"], t["s13"], t["w2"], t["s2"], on_host=False)
        self.rows = (torch.arange(max(n_rows, 1), dtype=torch.int32, device=device) if dma else
                     torch.zeros(max(n_rows, 1), dtype=torch.int32, device=device))
        # runs the FFN on the stage while the copy is still going (see
        # enqueue_cold_ffn), with the two events that order it (re-recorded
        # every call: a wait takes the record before it)
        self.ffn_stream = torch.cuda.Stream(device=device)
        self.gu_ready = torch.cuda.Event()
        self.gu_done = torch.cuda.Event()


def enqueue_cold_ffn(cold: Bank, split: Split, x, k: int, H: int, I: int, bufs: LayerBuffers,
                     stage: ColdStage | None, stream, overlap: bool = False):
    """Enqueue the cold bank's FFN for one step on `stream`. Without a stage
    the kernels read the bank in place. With a stage, the step's active rows
    are first copied into it (moe_stage_rows); with overlap the gate/up tensors
    are copied first and the gate/up GEMM on them runs on the stage's own
    stream while the down tensors are still being copied; the down GEMM then
    follows the copy on `stream` (its wait for the gate/up GEMM is normally
    long satisfied, so the copy -> down hand-over stays on one stream)."""
    if stage is None:
        moe_expert_ffn_mxfp4(cold, split, x, k, I, bufs.workspace, bufs.Y, stream=stream)
        return stream
    T = int(x.shape[0])
    if stage.dma:
        # copy-on-miss by the DMA engines: the split's active cold rows come
        # back to the host (this waits for the split), then one copy per run of
        # consecutive rows per tensor
        cap = min(cold.n_rows, T * k)
        if cap == 0:
            return stream
        with torch.cuda.stream(stream):
            stage.n_host.copy_(split.n_active[:1], non_blocking=True)
            stage.rows_host[:cap].copy_(split.active_rows[:cap], non_blocking=True)
        stream.synchronize()
        n = int(stage.n_host[0])
        moe_stage_rows_dma(cold, stage.rows_host[:n], stage.bank, H, I, parts=STAGE_ALL,
                           stream=stream)
        staged = Split(split.n_active, stage.rows, split.row_off, split.slots)
        moe_expert_ffn_mxfp4(stage.bank, staged, x, k, I, bufs.workspace, bufs.Y, stream=stream)
        return stream
    if not overlap:
        staged = moe_stage_rows(cold, split, T, k, stage.bank, stage.rows, H, I,
                                parts=STAGE_ALL, stream=stream)
        moe_expert_ffn_mxfp4(stage.bank, staged, x, k, I, bufs.workspace, bufs.Y, stream=stream)
        return stream
    staged = moe_stage_rows(cold, split, T, k, stage.bank, stage.rows, H, I,
                            parts=STAGE_GATE_UP, stream=stream)
    stage.gu_ready.record(stream)
    moe_stage_rows(cold, split, T, k, stage.bank, stage.rows, H, I, parts=STAGE_DOWN,
                   stream=stream)
    f = stage.ffn_stream
    f.wait_event(stage.gu_ready)
    moe_expert_gate_up_mxfp4(stage.bank, staged, x, k, I, bufs.workspace, stream=f)
    stage.gu_done.record(f)
    stream.wait_event(stage.gu_done)
    moe_expert_down_mxfp4(stage.bank, staged, T, k, H, I, bufs.workspace, bufs.Y, stream=stream)
    return stream


class ResidencyLayer:
    def __init__(self, hot: Bank, cold: Bank, row_map: torch.Tensor, H: int, I: int,
                 stage: ColdStage | None = None):
        """With `stage`, the cold bank's active rows are copied to it in one
        contiguous stream per row and the cold FFN reads them from HBM."""
        self.hot, self.cold, self.row_map, self.H, self.I = hot, cold, row_map, H, I
        self.stage = stage

    def _cold_ffn(self, x, k, bufs, stream, overlap=False):
        return enqueue_cold_ffn(self.cold, bufs.cold_split, x, k, self.H, self.I, bufs,
                                self.stage, stream, overlap)

    def forward(self, x, topk_ids, topk_w, bufs: LayerBuffers, counts_layer=None,
                count_tmax: int = 256, stream=None, cold_stream=None, hot_stream=None):
        """x bf16 [T,H] (as int16 or bfloat16), topk_ids int32 [T,k], topk_w fp32
        [T,k] -> bufs.out [T,H] bf16 bits. All on `stream` (default: current);
        with cold_stream, the cold FFN runs there between two event waits; with
        hot_stream, the hot FFN runs there instead and the cold path stays on
        `stream` with the split and the finalize (for steps where the cold
        path is the longer one, so that it never waits on another stream)."""
        k = int(topk_ids.shape[1])
        s = stream if stream is not None else torch.cuda.current_stream()
        moe_route_split(topk_ids, self.row_map, self.hot.n_rows, self.cold.n_rows, bufs.hot_split,
                        bufs.cold_split, bufs.n_invalid, counts_layer, count_tmax, stream=s)
        if hot_stream is not None:
            hot_stream.wait_stream(s)
            moe_expert_ffn_mxfp4(self.hot, bufs.hot_split, x, k, self.I, bufs.workspace, bufs.Y,
                                 stream=hot_stream)
            self._cold_ffn(x, k, bufs, s, overlap=True)
            s.wait_stream(hot_stream)
        elif cold_stream is None:
            moe_expert_ffn_mxfp4(self.hot, bufs.hot_split, x, k, self.I, bufs.workspace, bufs.Y,
                                 stream=s)
            self._cold_ffn(x, k, bufs, s)
        else:
            # cold first: its few workgroups start at once beside the hot bank's
            cold_stream.wait_stream(s)
            last = self._cold_ffn(x, k, bufs, cold_stream, overlap=True)
            moe_expert_ffn_mxfp4(self.hot, bufs.hot_split, x, k, self.I, bufs.workspace, bufs.Y,
                                 stream=s)
            s.wait_stream(last)
        moe_finalize(bufs.Y, topk_w, bufs.out, stream=s)
        return bufs.out
