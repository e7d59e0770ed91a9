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

Runtime control (same section: a small JSON file that freezes adaptation,
turns counting on or off, changes budgets, dumps counts or queues a restore to
the boot-time map): RuntimeControl reads such a file when it changes and
applies it to the policy; restore_swaps() lists the swaps that bring every
layer back to its boot-time hot set; Telemetry appends JSON lines per barrier
and per swap.

Readings of the pages: the average is kept in counts per read window; "minimum
average 8" applies to the promoted expert's average; a restore brings back the
boot-time hot/cold membership of every expert (a hot-cold swap moves one
expert each way, so the rows an expert ends up in may differ from its boot
rows; the row map always says where its weights are).
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, fields

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
        self.frozen = False  # observe() keeps averaging; decide() proposes nothing
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
        if self.frozen:
            return []
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


def swaps_to(hot_owner: list, cold_owner: list, target_hot: list,
             limit: int | None = None) -> list:
    """Swaps that turn each layer's live hot set into target_hot[l] (owners as
    the banks hold them now): each exchanges a hot expert that the target
    places cold with a cold expert that it places hot, both in ascending
    expert order. At most `limit` in total (None: all); after applying them,
    call again until none are left. Raises ValueError if a target is not a
    hot set of that layer's experts of the bank's size."""
    props = []
    for layer, (ho, co, th) in enumerate(zip(hot_owner, cold_owner, target_hot)):
        want = set(int(e) for e in th)
        out = sorted((int(e), r) for r, e in enumerate(ho) if int(e) not in want)
        back = sorted((int(e), r) for r, e in enumerate(co) if int(e) in want)
        if len(want) != len(ho) or len(out) != len(back):
            raise ValueError(f"layer {layer}: target is not a hot set of {len(ho)} of this "
                             f"layer's experts")
        for (eh, r), (ec, b) in zip(out, back):
            props.append(Swap(layer, r, b, eh, ec, 0.0))
    return props if limit is None else props[:limit]


def restore_swaps(hot_owner: list, cold_owner: list, boot_hot_owner: list,
                  limit: int | None = None) -> list:
    """Swaps that return every layer to its boot-time hot set (swaps_to the
    boot hot sets)."""
    return swaps_to(hot_owner, cold_owner, boot_hot_owner, limit)


class RuntimeControl:
    """Applies a JSON control file to a policy when the file changes.

    Keys (all optional): "freeze" (bool), "counting" (bool: whether the caller
    passes the counter table to moe_route_split), any PolicyConfig budget
    ("swaps_per_barrier", "swaps_per_layer", "min_avg", "hysteresis"),
    "dump_counts" (a path: the next counter snapshot is written there as JSON)
    and "restore_map" (true: queue a restore to the boot-time hot sets).
    Unknown keys are reported, not applied."""

    BUDGETS = ("swaps_per_barrier", "swaps_per_layer", "min_avg", "hysteresis")

    def __init__(self, policy: AdaptivePolicy, path: str | None = None):
        self.policy, self.path = policy, path
        self.counting = True
        self.restore_pending = False
        self.dump_path = None
        self._mtime = None

    def apply(self, ctrl: dict) -> list:
        """Apply one control record; returns the keys it did not know."""
        unknown = []
        names = {f.name for f in fields(PolicyConfig)}
        for key, val in ctrl.items():
            if key == "freeze":
                self.policy.frozen = bool(val)
            elif key == "counting":
                self.counting = bool(val)
            elif key == "restore_map":
                self.restore_pending = bool(val)
            elif key == "dump_counts":
                self.dump_path = str(val) if val else None
            elif key in self.BUDGETS and key in names:
                cast = int if key.startswith("swaps") else float
                setattr(self.policy.cfg, key, cast(val))
            else:
                unknown.append(key)
        return unknown

    def poll(self) -> list | None:
        """Re-read the control file if it changed; returns the unknown keys of
        the record applied, or None if nothing was read."""
        if not self.path or not os.path.exists(self.path):
            return None
        mtime = os.stat(self.path).st_mtime_ns
        if mtime == self._mtime:
            return None
        self._mtime = mtime
        with open(self.path) as f:
            return self.apply(json.load(f))

    def maybe_dump(self, snapshot: np.ndarray) -> bool:
        if not self.dump_path:
            return False
        with open(self.dump_path, "w") as f:
            json.dump(np.asarray(snapshot).astype(np.int64).tolist(), f)
        self.dump_path = None
        return True


class Telemetry:
    """Appends one JSON object per line to a file (or keeps them in memory)."""

    def __init__(self, path: str | None = None):
        self.path = path
        self.records = []

    def log(self, **record) -> None:
        self.records.append(record)
        if self.path:
            with open(self.path, "a") as f:
                f.write(json.dumps(record) + "\n")
