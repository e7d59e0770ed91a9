"""Off-line residency maps fitted to counted traffic.

"vLLM: Pin Hot Experts" builds its row map from a count-only boot: expert
selections counted over the lane's decode traffic, the busiest experts of
each layer placed in HBM and the rest in host memory (section "Results",
with the map's cold share checked by leave-one-out), and re-profiling on
other traffic gives another map, applied at the next boot (section "Closed,
September 17 evening": a separate map for each kind of traffic served works
better there than one fitted to a mix).
"MiMo-V2.6-Pro testing" ranks on decode counts, can mix a second histogram
in at a weight (its 5:05 PM entry) and merges live counts into a candidate
list only above a floor of decode tokens per layer (its 5:50 PM entry).

Here a count profile is an integer [layers, experts] table of selections,
e.g. the difference of two moe_usage_counts snapshots. fit_maps() scores
each expert by the weighted sum of its counts over the profiles given and
keeps, per layer, the experts - n_cold highest scores hot; equal scores go to
the lower expert id, so the map depends on the counts alone. Rows ascend with
expert id within each bank (hot expert e at row r >= 0: row_map[e] = r; cold
at row b: row_map[e] = -1 - b). Applying a fitted map to live banks is a set
of hot-cold swaps (policy.swaps_to, re-exported here), each moving one
expert each way; a boot loads the banks in the fitted order directly.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .policy import swaps_to  # noqa: F401 (applies a fitted map to live banks)

# Decode tokens per layer below which a profile is refused (the merge floor
# of "MiMo-V2.6-Pro testing", 5:50 PM entry).
MIN_TOKENS_PER_LAYER = 50_000


class ProfileTooSmall(ValueError):
    """A layer's profile holds fewer tokens than the floor asked for."""


@dataclass
class FittedMap:
    row_map: np.ndarray    # int32 [E]
    hot_owner: np.ndarray  # int32 [E - n_cold], ascending
    cold_owner: np.ndarray  # int32 [n_cold], ascending


def counts_between(before: np.ndarray, after: np.ndarray) -> np.ndarray:
    """Selections counted between two snapshots of the (never reset, 32-bit
    wrapping) counter table: int64 [L, E]."""
    a = np.asarray(after).astype(np.int64) & 0xFFFFFFFF
    b = np.asarray(before).astype(np.int64) & 0xFFFFFFFF
    return (a - b) & 0xFFFFFFFF


def score(profiles, weights=None) -> np.ndarray:
    """Weighted sum of count tables (float64 [L, E]); weights default to 1."""
    profiles = [np.asarray(p, np.float64) for p in profiles]
    if not profiles:
        raise ValueError("no count profile given")
    if weights is None:
        weights = [1.0] * len(profiles)
    if len(weights) != len(profiles):
        raise ValueError("one weight per profile")
    shape = profiles[0].shape
    if len(shape) != 2 or any(p.shape != shape for p in profiles):
        raise ValueError("profiles must share one [layers, experts] shape")
    out = np.zeros(shape, np.float64)
    for p, w in zip(profiles, weights):
        if w < 0 or not np.isfinite(w):
            raise ValueError("weights must be finite and non-negative")
        out += w * p
    return out


def _map_for(cold: np.ndarray, E: int) -> FittedMap:
    is_cold = np.zeros(E, bool)
    is_cold[cold] = True
    hot_owner = np.nonzero(~is_cold)[0].astype(np.int32)
    cold_owner = np.nonzero(is_cold)[0].astype(np.int32)
    row_map = np.empty(E, np.int32)
    row_map[hot_owner] = np.arange(hot_owner.size, dtype=np.int32)
    row_map[cold_owner] = -1 - np.arange(cold_owner.size, dtype=np.int32)
    return FittedMap(row_map, hot_owner, cold_owner)


def fit_maps(scores: np.ndarray, n_cold: int, top_k: int | None = None,
             min_tokens: int | None = None) -> list:
    """One FittedMap per layer: cold = the n_cold lowest-scoring experts
    (ties: the higher expert id goes cold). With top_k and min_tokens, a
    layer whose profile holds fewer than min_tokens tokens (selections /
    top_k) raises ProfileTooSmall."""
    s = np.asarray(scores, np.float64)
    if s.ndim != 2:
        raise ValueError("scores must be [layers, experts]")
    L, E = s.shape
    if not 0 <= n_cold <= E:
        raise ValueError(f"n_cold {n_cold} outside [0, {E}]")
    if min_tokens is not None:
        if not top_k or top_k <= 0:
            raise ValueError("min_tokens needs top_k")
        for layer in range(L):
            tokens = s[layer].sum() / top_k
            if tokens < min_tokens:
                raise ProfileTooSmall(f"layer {layer}: {tokens:.0f} tokens < {min_tokens}")
    maps = []
    ids = np.arange(E)
    for layer in range(L):
        # rank: score descending, then expert id ascending; the tail goes cold
        order = np.lexsort((ids, -s[layer]))
        maps.append(_map_for(order[E - n_cold:], E))
    return maps


def cold_share(counts: np.ndarray, maps) -> np.ndarray:
    """Fraction of each layer's selections that land on its cold set
    (float64 [L]; 0 for a layer with no selections)."""
    c = np.asarray(counts, np.float64)
    out = np.zeros(c.shape[0])
    for layer, m in enumerate(maps):
        tot = c[layer].sum()
        out[layer] = c[layer, m.cold_owner].sum() / tot if tot else 0.0
    return out


def overall_cold_share(counts: np.ndarray, maps) -> float:
    c = np.asarray(counts, np.float64)
    tot = c.sum()
    return float(sum(c[l, m.cold_owner].sum() for l, m in enumerate(maps)) / tot) if tot else 0.0


def leave_one_out(slices, n_cold: int) -> list:
    """Cold share of each profile slice under the map fitted to all the
    other slices (the held-out check of "vLLM: Pin Hot Experts", Results)."""
    slices = [np.asarray(p, np.float64) for p in slices]
    if len(slices) < 2:
        raise ValueError("leave-one-out needs at least two slices")
    out = []
    for i, held in enumerate(slices):
        maps = fit_maps(score([p for j, p in enumerate(slices) if j != i]), n_cold)
        out.append(overall_cold_share(held, maps))
    return out


def changed_cold(cold_owner_a, cold_owner_b) -> int:
    """Experts cold in b that were not cold in a."""
    return len(set(int(e) for e in cold_owner_b) - set(int(e) for e in cold_owner_a))
