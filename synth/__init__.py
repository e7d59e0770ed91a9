"""Seeded synthetic inputs for the hot/cold-residency MoE layer.

Input generators only: nothing here computes any part of the MoE layer. The
same inputs feed the CPU oracle (tests) and the GPU path (tests, benchmark).

- Weights: counter-based SplitMix64 byte streams keyed by (seed, layer, expert,
  tensor), filled on the host by ``libsynth.so`` and on the device by
  ``libsynth_dev.so`` (same definition, see synth.c). Weight bytes are uniform
  (two uniform E2M1 codes, -0 included); E8M0 scale bytes are spread over a
  small window (default 124..128, i.e. 2^-3 .. 2^1).
- Activations: N(0, 1) drawn by torch's CPU generator, rounded to bf16 by torch.
- Routing: a skewed per-layer expert distribution shaped after the decode
  histogram on "Offload by Expert on GB300", section "The skew is real" (top
  25/50/73% of experts carry 71.4/91.8/98.7% of decode picks, mean Gini 0.632):
  rank pmf p_r proportional to r^-0.30 * exp(-r/100), a seeded permutation from
  rank to expert id per layer, logits = ln p + Gumbel(0, 1) per token, the top-k
  logits in descending order (ties to the lower id) and fp32 softmax weights
  over the k picked logits. That is Plackett-Luce sampling of k distinct
  experts from p.
- Residency maps: "fitted" keeps the top-R_hot experts of the layer's pmf hot
  (the usage map of "vLLM: Pin Hot Experts", section "Results, September 17"),
  "positional" puts the last R_cold ids cold (the positional offload it is
  compared against). Rows are assigned in ascending expert id within a bank.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None
_dev = None

TENSORS = ("w13", "s13", "w2", "s2")


def lib():
    global _lib
    if _lib is None:
        p = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(p):
            raise RuntimeError(f"synth library not built: {p} (run `make synth`)")
        L = ctypes.CDLL(p)
        L.synth_key.restype = ctypes.c_uint64
        L.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        L.synth_fill_bank.restype = None
        L.synth_fill_bank.argtypes = ([ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_uint64, ctypes.c_int64] + [ctypes.c_int] * 5)
        _lib = L
    return _lib


def dev_lib():
    global _dev
    if _dev is None:
        p = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(p):
            raise RuntimeError(f"device synth library not built: {p} (run `make synth`)")
        L = ctypes.CDLL(p)
        L.synth_dev_fill_bank.restype = ctypes.c_int
        L.synth_dev_fill_bank.argtypes = ([ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_uint64, ctypes.c_int64] + [ctypes.c_int] * 4
                                          + [ctypes.c_void_p])
        _dev = L
    return _dev


# ------------------------------------------------------------------ sizes --

def expert_sizes(H: int, I: int) -> dict:
    """Bytes of one expert's four tensors (w13 packed, s13, w2 packed, s2)."""
    return {"w13": 2 * I * (H // 2), "s13": 2 * I * (H // 32), "w2": H * (I // 2), "s2": H * (I // 32)}


def expert_bytes(H: int, I: int) -> int:
    return sum(expert_sizes(H, I).values())


def tensor_shapes(n_rows: int, H: int, I: int) -> dict:
    return {"w13": (n_rows, 2 * I, H // 2), "s13": (n_rows, 2 * I, H // 32),
            "w2": (n_rows, H, I // 2), "s2": (n_rows, H, I // 32)}


# ---------------------------------------------------------------- weights --

def fill_bank_host(arrays: dict, owners, seed: int, layer: int, H: int, I: int,
                   scale_lo: int = 124, scale_cnt: int = 5, nthreads: int = 0) -> None:
    """Fill host arrays (numpy uint8 or pinned torch uint8 via .data_ptr) in place.

    ``arrays`` maps w13/s13/w2/s2 to objects exposing either ``ctypes.data``
    (numpy) or ``data_ptr()`` (torch, CPU)."""
    owners = np.ascontiguousarray(owners, np.int32)
    ptrs = []
    for name in TENSORS:
        a = arrays[name]
        ptrs.append(a.ctypes.data if isinstance(a, np.ndarray) else a.data_ptr())
    lib().synth_fill_bank(*ptrs, int(owners.shape[0]), owners.ctypes.data, int(seed) & (2**64 - 1),
                          int(layer), H, I, scale_lo, scale_cnt, nthreads)


def make_bank_host(owners, seed: int, layer: int, H: int, I: int, scale_lo: int = 124,
                   scale_cnt: int = 5) -> dict:
    """New numpy bank whose row r holds expert owners[r]."""
    owners = np.asarray(owners, np.int32)
    arrays = {k: np.empty(s, np.uint8) for k, s in tensor_shapes(len(owners), H, I).items()}
    if len(owners):
        fill_bank_host(arrays, owners, seed, layer, H, I, scale_lo, scale_cnt)
    return arrays


def fill_bank_device(tensors: dict, owners_dev, seed: int, layer: int, H: int, I: int,
                     scale_lo: int = 124, scale_cnt: int = 5, stream: int = 0) -> None:
    """Fill device tensors (torch, cuda) in place with the device twin.
    ``owners_dev`` is an int32 cuda tensor [n_rows]."""
    rc = dev_lib().synth_dev_fill_bank(*[tensors[k].data_ptr() for k in TENSORS],
                                       int(owners_dev.shape[0]), owners_dev.data_ptr(),
                                       int(seed) & (2**64 - 1), int(layer), H, I, scale_lo,
                                       scale_cnt, ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill_bank failed: {rc}")


# ------------------------------------------------------------ activations --

def activations(T: int, H: int, seed: int, layer: int = 0, step: int = 0) -> np.ndarray:
    """x ~ N(0,1) as bf16 bits [T, H] (torch CPU generator, torch's bf16 rounding)."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed((int(seed) * 1_000_003 + int(layer) * 7_919 + int(step) * 104_729) % (2**63))
    x = torch.randn(T, H, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16).copy()


# ---------------------------------------------------------------- routing --

def rank_pmf(E: int = 384, alpha: float = 0.30, tau: float = 100.0) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-alpha) * np.exp(-r / tau)
    return p / p.sum()


def layer_permutation(E: int, seed: int, layer: int) -> np.ndarray:
    """perm[rank] = expert id for this layer."""
    rng = np.random.default_rng([int(seed), 0x5EED, int(layer)])
    return rng.permutation(E).astype(np.int32)


def topk_desc(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, descending, ties to the lower id."""
    order = np.argsort(-logits, axis=-1, kind="stable")
    return order[..., :k].astype(np.int32)


def softmax_selected(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=-1).astype(np.float32)
    z = sel - sel.max(axis=-1, keepdims=True)
    e = np.exp(z, dtype=np.float32)
    return (e / e.sum(axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)


def skewed_routing(T: int, k: int, E: int, seed: int, layer: int, step: int,
                   pmf: np.ndarray | None = None, perm: np.ndarray | None = None):
    """Plackett-Luce top-k from the layer's skewed pmf. Returns (ids int32 [T,k],
    weights fp32 [T,k])."""
    if pmf is None:
        pmf = rank_pmf(E)
    if perm is None:
        perm = layer_permutation(E, seed, layer)
    logp = np.empty(E)
    logp[perm] = np.log(pmf)
    rng = np.random.default_rng([int(seed), 0x70C5, int(layer), int(step)])
    logits = logp[None, :] + rng.gumbel(size=(T, E))
    ids = topk_desc(logits, k)
    return ids, softmax_selected(logits.astype(np.float32), ids)


# Verify-window routing: the tokens of one speculative verify window share
# experts. The pages measure the touched set of a window ("vLLM: Pin Hot
# Experts", the paragraph after the off-domain table): 6.0, 10.1, 16.8, 22.5
# and 27.4 unique experts per layer for windows of 1, 2, 4, 6 and 8 tokens at
# top-6, the same across traffic categories. Independent tokens touch 11.7,
# 22.3, 31.9 and 40.7 (for 2..8 tokens). Model: logits of token t in window w
# = WINDOW_SHARP * ln p + WINDOW_SHARED * S[w, e] + Gumbel[t, e], with S ~
# N(0, 1) drawn once per window and expert. Fitted on the CPU (grid over the
# two constants, 1,500 windows): 6.0 / 10.4 / 17.2 / 22.8 / 27.5 unique
# experts, Gini 0.62 of the pick counts, 1.7-1.8% of picks on the fitted cold
# set (the pages: Gini 0.63, 1.55%).
WINDOW_SHARED = 2.0
WINDOW_SHARP = 1.1


def window_routing(T: int, k: int, E: int, seed: int, layer: int, step: int, window: int = 7,
                   pmf: np.ndarray | None = None, perm: np.ndarray | None = None):
    """Top-k routing of T tokens in consecutive verify windows of `window`
    tokens (the last may be shorter), tokens of a window correlated through a
    shared per-window term (see above). Returns (ids int32 [T,k], weights fp32
    [T,k]: softmax over the k selected logits)."""
    if pmf is None:
        pmf = rank_pmf(E)
    if perm is None:
        perm = layer_permutation(E, seed, layer)
    logp = np.empty(E)
    logp[perm] = np.log(pmf)
    rng = np.random.default_rng([int(seed), 0x3E7A, int(layer), int(step)])
    nwin = (T + window - 1) // window
    shared = rng.standard_normal((nwin, E))
    gum = rng.gumbel(size=(T, E))
    win_of = np.arange(T) // window
    logits = WINDOW_SHARP * logp[None, :] + WINDOW_SHARED * shared[win_of] + gum
    ids = topk_desc(logits, k)
    return ids, softmax_selected(logits.astype(np.float32), ids)


def gaussian_routing(T: int, k: int, E: int, seed: int, layer: int = 0, step: int = 0):
    """Router logits N(0,1) [T,E], top-k, softmax over the k (the tiny config)."""
    rng = np.random.default_rng([int(seed), 0x7147, int(layer), int(step)])
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids = topk_desc(logits, k)
    return ids, softmax_selected(logits, ids)


# ------------------------------------------------------------------- maps --

def map_from_cold_set(E: int, cold_ids) -> tuple:
    """Row map + owner lists from a cold set. Rows ascend with expert id within
    each bank. Returns (row_map int32 [E], hot_owner int32 [R_h], cold_owner
    int32 [R_c])."""
    cold = np.zeros(E, bool)
    cold[np.asarray(cold_ids, np.int64)] = True
    hot_owner = np.nonzero(~cold)[0].astype(np.int32)
    cold_owner = np.nonzero(cold)[0].astype(np.int32)
    row_map = np.empty(E, np.int32)
    row_map[hot_owner] = np.arange(len(hot_owner), dtype=np.int32)
    row_map[cold_owner] = -1 - np.arange(len(cold_owner), dtype=np.int32)
    return row_map, hot_owner, cold_owner


def fitted_map(E: int, n_cold: int, seed: int, layer: int, pmf=None):
    """Cold = the n_cold least probable experts of the layer's pmf."""
    perm = layer_permutation(E, seed, layer)
    return map_from_cold_set(E, perm[E - n_cold:])


def positional_map(E: int, n_cold: int):
    """Cold = the last n_cold expert ids."""
    return map_from_cold_set(E, np.arange(E - n_cold, E))


def random_map(E: int, n_cold: int, seed: int):
    rng = np.random.default_rng([int(seed), 0xC01D])
    return map_from_cold_set(E, rng.choice(E, n_cold, replace=False))


def all_hot_map(E: int):
    return map_from_cold_set(E, [])


# ------------------------------------------------------------ statistics --

def gini(counts) -> float:
    c = np.sort(np.asarray(counts, np.float64))
    n = c.size
    if c.sum() == 0:
        return 0.0
    i = np.arange(1, n + 1)
    return float((2 * (i * c).sum() / (n * c.sum())) - (n + 1) / n)


def top_share(counts, frac: float) -> float:
    c = np.sort(np.asarray(counts, np.float64))[::-1]
    m = int(round(frac * c.size))
    return float(c[:m].sum() / c.sum())


# ---------------------------------------------------------------- configs --

@dataclass
class Config:
    """One workload: shapes, residency split and routing kind."""
    name: str
    E: int
    k: int
    H: int
    I: int
    T: int
    n_hot: int
    n_cold: int
    layers: int = 1
    routing: str = "skewed"       # "skewed" | "gaussian"
    cold_map: str = "fitted"      # "fitted" | "positional" | "random"
    count_tmax: int = 256
    seed: int = 20260917
    extra: dict = field(default_factory=dict)

    @property
    def picks(self) -> int:
        return self.T * self.k

    def routing_for(self, layer: int, step: int):
        if self.routing == "gaussian":
            return gaussian_routing(self.T, self.k, self.E, self.seed, layer, step)
        return skewed_routing(self.T, self.k, self.E, self.seed, layer, step)

    def map_for(self, layer: int):
        if self.cold_map == "positional":
            return positional_map(self.E, self.n_cold)
        if self.cold_map == "random":
            return random_map(self.E, self.n_cold, self.seed + layer)
        return fitted_map(self.E, self.n_cold, self.seed, layer)


TINY = Config("tiny", E=16, k=2, H=256, I=128, T=8, n_hot=12, n_cold=4, routing="gaussian",
              cold_map="random")
FULL_LAYER = Config("full_layer_decode_t16", E=384, k=6, H=4096, I=2880, T=16, n_hot=295, n_cold=89)
FULL_STEP = Config("full_step_decode_t7", E=384, k=6, H=4096, I=2880, T=7, n_hot=295, n_cold=89,
                   layers=40)
HIGH_CONC = Config("high_concurrency_t112", E=384, k=6, H=4096, I=2880, T=112, n_hot=295,
                   n_cold=89, layers=40)
HIGH_CONC_POS = Config("high_concurrency_t112_positional", E=384, k=6, H=4096, I=2880, T=112,
                       n_hot=295, n_cold=89, layers=40, cold_map="positional")
PREFILL = Config("prefill_t4096", E=384, k=6, H=4096, I=2880, T=4096, n_hot=295, n_cold=89,
                 layers=40)
CONFIGS = {c.name: c for c in (TINY, FULL_LAYER, FULL_STEP, HIGH_CONC, HIGH_CONC_POS, PREFILL)}
