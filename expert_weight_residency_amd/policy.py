"""Host-side swap policy over the usage counter ("We Built the Counter",
section 2 and the policy defaults of section 9).

Every `read_every` steps the caller snapshots the counter table with
moe_usage_counts and passes it to observe(). The per-(layer, expert) counts
since the last read are folded into an exponentially weighted average with a
half-life of `half_life` steps. decide() then proposes, per layer, promoting
the busiest cold experts in exchange for the idlest hot ones, at most
`swaps_per_layer` per layer, only when the cold expert's average is at least
`min_avg` and exceeds the hot one's by the hysteresis factor, and at most
`swaps_per_barrier` in total (largest gain first). Each proposal names the
rows and the experts it was decided against, so moe_swap_rows can refuse it if
the owners changed in between.

Readings of the pages: the average is kept in counts per read window; "minimum
average 8" applies to the promoted expert's average.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class PolicyConfig:
    read_every: int = 64
    half_life: float = 500.0
    swaps_per_layer: int = 2
    hysteresis: float = 1.5
    min_avg: float = 8.0
    swaps_per_barrier: int = 8


@dataclass
class Swap:
    layer: int
    hot_row: int
    cold_row: int
    expect_hot_expert: int
    expect_cold_expert: int
    gain: float


class AdaptivePolicy:
    def __init__(self, layers: int, experts: int, cfg: PolicyConfig | None = None):
        self.cfg = cfg or PolicyConfig()
        self.avg = np.zeros((layers, experts), np.float64)
        self.prev = None
        self.decay = 0.5 ** (self.cfg.read_every / self.cfg.half_life)

    def observe(self, snapshot: np.ndarray) -> None:
        """snapshot: int32 [L, E] counter table (never reset; wraps mod 2^32)."""
        cur = np.asarray(snapshot).astype(np.int64) & 0xFFFFFFFF
        if self.prev is None:
            self.prev = cur
            return
        delta = (cur - self.prev) & 0xFFFFFFFF
        self.prev = cur
        self.avg = self.avg * self.decay + delta * (1.0 - self.decay)

    def decide(self, hot_owner: list, cold_owner: list) -> list:
        """hot_owner[l] / cold_owner[l]: int arrays, expert held by each row."""
        c = self.cfg
        props = []
        for layer, (ho, co) in enumerate(zip(hot_owner, cold_owner)):
            if len(ho) == 0 or len(co) == 0:
                continue
            a = self.avg[layer]
            cold_rank = np.argsort(-a[co], kind="stable")
            hot_rank = np.argsort(a[ho], kind="stable")
            for n in range(min(c.swaps_per_layer, len(co), len(ho))):
                b, r = int(cold_rank[n]), int(hot_rank[n])
                ec, eh = int(co[b]), int(ho[r])
                if a[ec] >= c.min_avg and a[ec] > c.hysteresis * a[eh]:
                    props.append(Swap(layer, r, b, eh, ec, float(a[ec] - a[eh])))
        props.sort(key=lambda s: -s.gain)
        return props[: c.swaps_per_barrier]
