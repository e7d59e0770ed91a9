"""CPU oracle for the hot/cold-residency MXFP4 MoE layer.

TEST INFRASTRUCTURE ONLY: the plain definition the GPU path is checked
against. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import it. The product package never imports it and it
imports nothing from the product package.

Numerics (dequant, expert FFN, finalize) live in ``moe_oracle.c`` and are
reached through ctypes. The bookkeeping steps (residency split, usage counter,
row swap) are written here in numpy as the plain definitions:

- split: "vLLM: Pin Hot Experts", section "The one open door" (an int32 row map
  per layer resolves a global expert id to which tensor and which row) and
  section "Results, September 17" (each token's ids are split by residency and
  each bank is called once);
- counter: "We Built the Counter", section 2 (one masked atomic add per routed
  pick into a fixed layers x experts int table; only steps of at most 256
  tokens are counted);
- swap: "vLLM: Pin Hot Experts", section "Closed, September 17 evening", E4/E4b
  (hot row to staging, cold row into the hot slot, staging into the cold slot,
  then a two-element row-map write), with the stale check of "We Built the
  Counter", section 2.

Every function here is pinned by a CPU test against something other than
itself (the OCP MX value table, closed forms, a float64 library matmul on an
independent dequantization, brute force on tiny inputs, crafted finalize
inputs, page-printed sizes); the pin of each function is listed next to it:

- e2m1, e8m0, dequant: the OCP MX value table and exponent bit patterns,
  every (code, scale byte) pair;
- silu: the logistic function of scipy; f32_to_bf16: torch's rounding
  (ties, both parities, specials);
- expert_ffn: all-ones weights (sum of x), one-hot rows (gate/up order,
  nibble order, scale index), a float64 numpy matmul on an independent
  dequantization;
- finalize: k = 1 identity, an fma-sensitive input, an order-sensitive input;
- moe_layer: split result == unsplit result, the same picks through
  expert_ffn one by one;
- resolve, route_split: brute force over random tiny cases;
- usage_count: the T*k total, the 256-token gate, the int32 wrap;
- swap_rows: five ordered swaps at 384/295/89 geometry, a mis-ordered map
  write that diverges, stale refusal, a round trip.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")


def lib():
    """Load liboracle.so (built by ``make oracle``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"oracle library not built: {_LIB_PATH} (run `make oracle`)")
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_e2m1.restype = ctypes.c_double
        L.oracle_e2m1.argtypes = [ctypes.c_int]
        L.oracle_e8m0.restype = ctypes.c_double
        L.oracle_e8m0.argtypes = [ctypes.c_int]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_dequant.restype = None
        L.oracle_dequant.argtypes = [_u8p, _u8p, ctypes.c_int64, ctypes.c_int, _f32p]
        L.oracle_expert_ffn.restype = None
        L.oracle_expert_ffn.argtypes = [_u8p, _u8p, _u8p, _u8p, ctypes.c_int, ctypes.c_int,
                                        _u16p] + [ctypes.c_void_p] * 4 + [_u16p]
        L.oracle_finalize.restype = None
        L.oracle_finalize.argtypes = [_u16p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _u16p]
        L.oracle_moe_layer.restype = ctypes.c_int
        L.oracle_moe_layer.argtypes = ([_u8p] * 4 + [ctypes.c_int] + [_u8p] * 4 + [ctypes.c_int]
                                       + [_i32p, ctypes.c_int, _i32p, _f32p] + [ctypes.c_int] * 4
                                       + [_u16p, _u16p, _u16p, ctypes.c_int])
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        _lib = L
    return _lib


# ---------------------------------------------------------------- numerics --

def e2m1(code: int) -> float:
    return lib().oracle_e2m1(int(code))


def e8m0(byte: int) -> float:
    return lib().oracle_e8m0(int(byte))


def silu(z: float) -> float:
    return lib().oracle_silu(float(z))


def f32_to_bf16(a) -> np.ndarray:
    """Elementwise fp32 -> bf16 bits (round to nearest even), via the C oracle."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    f = lib().oracle_f32_to_bf16
    return np.array([f(float(v)) for v in a.reshape(-1)], dtype=np.uint16).reshape(a.shape)


def bf16_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def dequant(w: np.ndarray, s: np.ndarray, K: int) -> np.ndarray:
    """w: uint8 [rows, K/2], s: uint8 [rows, K/32] -> fp32 [rows, K]."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    rows = w.size // (K // 2)
    out = np.empty((rows, K), dtype=np.float32)
    lib().oracle_dequant(w.reshape(-1), s.reshape(-1), rows, K, out.reshape(-1))
    return out


def expert_ffn(w13, s13, w2, s2, x_bf16, H: int, I: int):
    """One expert on one token. Returns dict of g, u, h (fp32 [I]), y (fp32 [H]),
    y_bf16 (uint16 [H])."""
    g = np.empty(I, np.float32)
    u = np.empty(I, np.float32)
    h = np.empty(I, np.float32)
    y = np.empty(H, np.float32)
    yb = np.empty(H, np.uint16)
    lib().oracle_expert_ffn(
        np.ascontiguousarray(w13, np.uint8).reshape(-1), np.ascontiguousarray(s13, np.uint8).reshape(-1),
        np.ascontiguousarray(w2, np.uint8).reshape(-1), np.ascontiguousarray(s2, np.uint8).reshape(-1),
        H, I, np.ascontiguousarray(x_bf16, np.uint16).reshape(-1),
        g.ctypes.data, u.ctypes.data, h.ctypes.data, y.ctypes.data, yb)
    return {"g": g, "u": u, "h": h, "y": y, "y_bf16": yb}


def finalize(Y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Y: bf16 bits [T, k, H]; w: fp32 [T, k] -> bf16 bits [T, H]."""
    Y = np.ascontiguousarray(Y, np.uint16)
    w = np.ascontiguousarray(w, np.float32)
    T, k, H = Y.shape
    out = np.empty((T, H), np.uint16)
    lib().oracle_finalize(Y.reshape(-1), w.reshape(-1), T, k, H, out.reshape(-1))
    return out


@dataclass
class Bank:
    """Host copy of one residency bank: w13 [R, 2I, H/2], s13 [R, 2I, H/32],
    w2 [R, H, I/2], s2 [R, H, I/32], all uint8."""
    w13: np.ndarray
    s13: np.ndarray
    w2: np.ndarray
    s2: np.ndarray

    @property
    def n_rows(self) -> int:
        return int(self.w13.shape[0])


def _flat(a):
    return np.ascontiguousarray(a, np.uint8).reshape(-1)


def moe_layer(hot: Bank, cold: Bank, row_map, topk_ids, topk_w, x_bf16, H: int, I: int,
              nthreads: int = 0):
    """The whole layer. Returns (Y bf16 [T,k,H], out bf16 [T,H], n_bad)."""
    topk_ids = np.ascontiguousarray(topk_ids, np.int32)
    T, k = topk_ids.shape
    Y = np.empty((T, k, H), np.uint16)
    out = np.empty((T, H), np.uint16)
    empty = np.zeros(1, np.uint8)

    def parts(b: Bank):
        if b is None or b.n_rows == 0:
            return [empty] * 4, 0
        return [_flat(b.w13), _flat(b.s13), _flat(b.w2), _flat(b.s2)], b.n_rows

    hp, nh = parts(hot)
    cp, nc = parts(cold)
    bad = lib().oracle_moe_layer(*hp, nh, *cp, nc, np.ascontiguousarray(row_map, np.int32),
                                 int(row_map.shape[0]), topk_ids.reshape(-1),
                                 np.ascontiguousarray(topk_w, np.float32).reshape(-1), T, k, H, I,
                                 np.ascontiguousarray(x_bf16, np.uint16).reshape(-1),
                                 Y.reshape(-1), out.reshape(-1), int(nthreads))
    return Y, out, bad


def max_threads() -> int:
    return int(lib().oracle_max_threads())


# ------------------------------------------------------------ bookkeeping --

def resolve(row_map, ids, n_hot: int, n_cold: int):
    """Per pick: (bank, row) with bank 0 = hot, 1 = cold, -1 = invalid.

    Row-map encoding: m >= 0 is hot row m, m < 0 is cold row -1-m. An id outside
    [0, E) or a row outside its bank is invalid."""
    row_map = np.asarray(row_map, np.int64)
    ids = np.asarray(ids, np.int64).reshape(-1)
    E = row_map.shape[0]
    bank = np.full(ids.shape, -1, np.int64)
    row = np.full(ids.shape, -1, np.int64)
    ok = (ids >= 0) & (ids < E)
    m = np.where(ok, row_map[np.clip(ids, 0, max(E - 1, 0))] if E else 0, 0)
    hot = ok & (m >= 0) & (m < n_hot)
    cold = ok & (m < 0) & ((-1 - m) < n_cold)
    bank[hot] = 0
    row[hot] = m[hot]
    bank[cold] = 1
    row[cold] = (-1 - m)[cold]
    return bank, row


def route_split(topk_ids, row_map, n_hot: int, n_cold: int):
    """Residency split with deterministic compaction.

    For each bank: the active rows in ascending row order, CSR offsets into a
    slot list, and the slot list, where slot s = t*k + j and the slots of one row
    appear in ascending s. Returns {"hot": (active_rows, row_off, slots),
    "cold": (...), "n_invalid": int}."""
    ids = np.asarray(topk_ids).reshape(-1)
    bank, row = resolve(row_map, ids, n_hot, n_cold)
    res = {"n_invalid": int(np.count_nonzero(bank < 0))}
    for b, name in ((0, "hot"), (1, "cold")):
        s = np.nonzero(bank == b)[0]
        order = np.argsort(row[s], kind="stable")
        slots = s[order].astype(np.int32)
        active, cnt = np.unique(row[s], return_counts=True)
        row_off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
        res[name] = (active.astype(np.int32), row_off, slots)
    return res


def usage_count(counts_layer: np.ndarray, topk_ids, E: int, count_tmax: int = 256) -> np.ndarray:
    """Counter update for one layer: +1 per pick whose id is in [0, E), only when
    the step has at most count_tmax tokens. Returns the new counts (int32, wraps)."""
    ids = np.asarray(topk_ids)
    T = ids.shape[0]
    out = np.array(counts_layer, dtype=np.int64, copy=True)
    if T <= count_tmax:
        v = ids.reshape(-1)
        v = v[(v >= 0) & (v < E)]
        out += np.bincount(v, minlength=E)[:E]
    return (out & 0xFFFFFFFF).astype(np.uint32).view(np.int32)


class SwapStale(Exception):
    """The swap was decided against an owner list that has changed since."""


def swap_rows(hot: Bank, cold: Bank, hot_row: int, cold_row: int, expect_hot: int, expect_cold: int,
              row_map: np.ndarray, hot_owner: np.ndarray, cold_owner: np.ndarray) -> None:
    """True row swap on host byte arrays (in place).

    Stale check first: the hot row must still hold expect_hot and the cold row
    expect_cold, else SwapStale and nothing changes. Then, for each of the four
    tensors: staging <- hot[a]; hot[a] <- cold[b]; cold[b] <- staging. Then the
    two-element map write and the owner-mirror update."""
    if hot_owner[hot_row] != expect_hot or cold_owner[cold_row] != expect_cold:
        raise SwapStale(f"hot row {hot_row} holds {hot_owner[hot_row]} (expected {expect_hot}), "
                        f"cold row {cold_row} holds {cold_owner[cold_row]} (expected {expect_cold})")
    for name in ("w13", "s13", "w2", "s2"):
        h = getattr(hot, name)
        c = getattr(cold, name)
        staging = h[hot_row].copy()
        h[hot_row] = c[cold_row]
        c[cold_row] = staging
    row_map[expect_hot] = -1 - cold_row
    row_map[expect_cold] = hot_row
    hot_owner[hot_row] = expect_cold
    cold_owner[cold_row] = expect_hot
