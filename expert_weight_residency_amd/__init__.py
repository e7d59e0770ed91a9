"""Hot/cold expert-residency MXFP4 MoE layer for MI355X (gfx950).

A thin ctypes binding over ``libmoe_residency.so``: every function here has the
name of a C entry point in ``include/moe_residency.h`` and only marshals
arguments (torch tensors -> device pointers, the current HIP stream). Every
step of the layer runs in the library's HIP kernels; there is no fallback, and
importing a function whose library is missing raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_residency.so")

MOE_OK, MOE_EINVAL, MOE_EHIP, MOE_ESTALE, MOE_ENOTSUP = 0, -1, -2, -3, -4
MOE_MAX_EXPERTS = MOE_MAX_ROWS = 4096
MOE_MAX_TOPK = 32

# entry points declared in include/moe_residency.h
ENTRY_POINTS = ("moe_expert_bytes", "moe_ffn_workspace_bytes", "moe_route_split",
                "moe_expert_ffn_mxfp4", "moe_expert_gate_up_mxfp4", "moe_expert_down_mxfp4",
                "moe_stage_rows", "moe_finalize", "moe_usage_counts", "moe_swap_rows",
                "moe_last_error", "moe_expert_ffn_mxfp4_noalloc", "moe_stage_rows_dma")
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class MoeStale(MoeError):
    """moe_swap_rows refused a swap decided against outdated owner lists."""


class MoeBankC(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("s13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("s2", ctypes.c_void_p), ("n_rows", ctypes.c_int32), ("on_host", ctypes.c_int32)]


class MoeSplitC(ctypes.Structure):
    _fields_ = [("n_active", ctypes.c_void_p), ("active_rows", ctypes.c_void_p),
                ("row_off", ctypes.c_void_p), ("slots", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} (run `make lib` or "
                               "__graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_expert_bytes.restype = sz
        L.moe_expert_bytes.argtypes = [i32, i32]
        L.moe_ffn_workspace_bytes.restype = sz
        L.moe_ffn_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_route_split.restype = i32
        L.moe_route_split.argtypes = [vp, i32, i32, vp, i32, i32, i32, vp, i32, MoeSplitC,
                                      MoeSplitC, vp, vp]
        L.moe_expert_ffn_mxfp4.restype = i32
        L.moe_expert_ffn_mxfp4.argtypes = [ctypes.POINTER(MoeBankC), MoeSplitC, vp, i32, i32, i32,
                                           i32, vp, vp, vp]
        L.moe_expert_ffn_mxfp4_noalloc.restype = i32
        L.moe_expert_ffn_mxfp4_noalloc.argtypes = [ctypes.POINTER(MoeBankC), MoeSplitC, vp, i32,
                                                   i32, i32, i32, vp, vp]
        L.moe_expert_gate_up_mxfp4.restype = i32
        L.moe_expert_gate_up_mxfp4.argtypes = [ctypes.POINTER(MoeBankC), MoeSplitC, vp, i32, i32,
                                               i32, i32, vp, vp]
        L.moe_expert_down_mxfp4.restype = i32
        L.moe_expert_down_mxfp4.argtypes = [ctypes.POINTER(MoeBankC), MoeSplitC, i32, i32, i32, i32,
                                            vp, vp, vp]
        L.moe_stage_rows.restype = i32
        L.moe_stage_rows.argtypes = [ctypes.POINTER(MoeBankC), MoeSplitC, i32, i32,
                                     ctypes.POINTER(MoeBankC), vp, i32, i32, i32, vp]
        L.moe_stage_rows_dma.restype = i32
        L.moe_stage_rows_dma.argtypes = [ctypes.POINTER(MoeBankC), vp, i32,
                                         ctypes.POINTER(MoeBankC), i32, i32, i32, vp]
        L.moe_finalize.restype = i32
        L.moe_finalize.argtypes = [vp, vp, i32, i32, i32, vp, vp]
        L.moe_usage_counts.restype = i32
        L.moe_usage_counts.argtypes = [vp, i32, i32, vp, vp]
        L.moe_swap_rows.restype = i32
        L.moe_swap_rows.argtypes = [ctypes.POINTER(MoeBankC), ctypes.POINTER(MoeBankC), i32, i32,
                                    i32, i32, vp, i32, vp, vp, vp, sz, i32, i32, vp]
        _lib = L
    return _lib


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def _check(rc: int) -> None:
    if rc != MOE_OK:
        msg = moe_last_error()
        raise (MoeStale if rc == MOE_ESTALE else MoeError)(rc, msg)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# Host-side argument checks (a wrong dtype, a CPU tensor or a strided view
# would otherwise reach the kernels as a raw pointer). They raise MoeError
# with MOE_EINVAL before anything is enqueued.
_BF16_BITS = ("torch.int16", "torch.bfloat16", "torch.uint16")


def _bad(name: str, want: str, t) -> MoeError:
    got = f"{getattr(t, 'dtype', type(t).__name__)} on {getattr(t, 'device', '?')}"
    return MoeError(MOE_EINVAL, f"{name}: need {want}, got {got}")


def _gpu(t, name: str, dtypes=None):
    """Data pointer of a contiguous GPU tensor of one of `dtypes` (str names)."""
    dev = getattr(t, "device", None)
    if dev is None or dev.type != "cuda" or not t.is_contiguous() or \
            (dtypes is not None and str(t.dtype) not in dtypes):
        raise _bad(name, f"a contiguous GPU tensor ({', '.join(dtypes or ('any dtype',))})", t)
    return t.data_ptr()


def _gpu_opt(t, name: str, dtypes=None):
    return None if t is None else _gpu(t, name, dtypes)


def _nbytes(t) -> int:
    return int(t.numel()) * int(t.element_size())


def _need(t, name: str, nbytes: int) -> None:
    """Raise MOE_EINVAL unless tensor t holds at least nbytes bytes (a
    too-small buffer would otherwise be written past its end on the GPU)."""
    if _nbytes(t) < nbytes:
        raise MoeError(MOE_EINVAL, f"{name}: holds {_nbytes(t)} bytes, the call needs {nbytes}")


def _check_bank(bank: "Bank", H: int, I: int, name: str = "bank") -> None:
    """Every tensor of the bank holds n_rows rows of the layout for (H, I)
    (remembered per bank for the tensors and sizes last checked)."""
    key = (bank.w13.data_ptr(), bank.s13.data_ptr(), bank.w2.data_ptr(), bank.s2.data_ptr(),
           int(bank.w13.numel()), int(bank.s13.numel()), int(bank.w2.numel()),
           int(bank.s2.numel()), H, I)
    if bank.__dict__.get("_sized") == key:
        return
    R = bank.n_rows
    want = {"w13": R * 2 * I * (H // 2), "s13": R * 2 * I * (H // 32),
            "w2": R * H * (I // 2), "s2": R * H * (I // 32)}
    for t, n in want.items():
        got = int(getattr(bank, t).numel())
        if got != n:
            raise MoeError(MOE_EINVAL, f"{name} {t}: {got} bytes, {R} rows at H={H}, I={I} "
                                       f"need {n}")
    bank.__dict__["_sized"] = key


def _check_split(split: "Split", n_rows: int, T: int, k: int, name: str = "split") -> None:
    """The split's buffers hold the capacity moe_route_split writes for a bank
    of n_rows rows at T tokens, k picks each."""
    cap = min(n_rows, T * k)
    for f, n in (("n_active", 1), ("active_rows", cap), ("row_off", cap + 1),
                 ("slots", T * k)):
        if int(getattr(split, f).numel()) < n:
            raise MoeError(MOE_EINVAL, f"{name} {f}: {int(getattr(split, f).numel())} entries, "
                                       f"need {n} (bank rows {n_rows}, T*k {T * k})")


def moe_expert_bytes(H: int, I: int) -> int:
    return int(lib().moe_expert_bytes(H, I))


def moe_ffn_workspace_bytes(T: int, k: int, H: int, I: int) -> int:
    return int(lib().moe_ffn_workspace_bytes(T, k, H, I))


# ------------------------------------------------------------ containers --

# where a bank's tensors sit (moe_bank.on_host)
BANK_DEVICE, BANK_HOST, BANK_HOST_WEIGHTS = 0, 1, 2


@dataclass
class Bank:
    """One residency bank: uint8 tensors w13 [R,2I,H/2], s13 [R,2I,H/32],
    w2 [R,H,I/2], s2 [R,H,I/32] on the device (on_host=False / BANK_DEVICE),
    all four pinned on the host (on_host=True / BANK_HOST, read in place by
    the kernels), or w13, w2 pinned on the host and the scales s13, s2 on the
    device (BANK_HOST_WEIGHTS)."""
    w13: object
    s13: object
    w2: object
    s2: object
    on_host: int = BANK_DEVICE

    @property
    def n_rows(self) -> int:
        return int(self.w13.shape[0])

    def abi(self) -> MoeBankC:
        # built once per set of tensors (the call path stays cheap on the host)
        key = (self.w13.data_ptr(), self.s13.data_ptr(), self.w2.data_ptr(),
               self.s2.data_ptr(), self.n_rows, self.on_host)
        c = self.__dict__.get("_abi")
        if c is None or c[0] != key:
            where = int(self.on_host)
            if where not in (BANK_DEVICE, BANK_HOST, BANK_HOST_WEIGHTS):
                raise MoeError(MOE_EINVAL, f"bank on_host={self.on_host!r}: expected "
                               "BANK_DEVICE, BANK_HOST or BANK_HOST_WEIGHTS")
            for name, t in self.tensors().items():
                if str(t.dtype) != "torch.uint8" or not t.is_contiguous():
                    raise _bad(f"bank {name}", "a contiguous uint8 tensor", t)
                host = where == BANK_HOST or (where == BANK_HOST_WEIGHTS and name[0] == "w")
                if host and (t.device.type != "cpu" or not t.is_pinned()):
                    raise _bad(f"bank {name}", f"pinned host memory (on_host={where})", t)
                if not host and t.device.type != "cuda":
                    raise _bad(f"bank {name}", f"GPU memory (on_host={where})", t)
            c = (key, MoeBankC(self.w13.data_ptr(), self.s13.data_ptr(), self.w2.data_ptr(),
                               self.s2.data_ptr(), self.n_rows, where))
            self.__dict__["_abi"] = c
        return c[1]

    def tensors(self) -> dict:
        return {"w13": self.w13, "s13": self.s13, "w2": self.w2, "s2": self.s2}


@dataclass
class Split:
    """Device int32 buffers of one bank's split (see moe_split)."""
    n_active: object
    active_rows: object
    row_off: object
    slots: object

    @classmethod
    def empty(cls, n_rows: int, T: int, k: int, device="cuda") -> "Split":
        import torch
        cap = min(n_rows, T * k)
        return cls(torch.zeros(1, dtype=torch.int32, device=device),
                   torch.zeros(max(cap, 1), dtype=torch.int32, device=device),
                   torch.zeros(cap + 1, dtype=torch.int32, device=device),
                   torch.zeros(max(T * k, 1), dtype=torch.int32, device=device))

    def abi(self) -> MoeSplitC:
        key = (self.n_active.data_ptr(), self.active_rows.data_ptr(), self.row_off.data_ptr(),
               self.slots.data_ptr())
        c = self.__dict__.get("_abi")
        if c is None or c[0] != key:
            ptrs = [_gpu(getattr(self, f), f"split {f}", ("torch.int32",))
                    for f in ("n_active", "active_rows", "row_off", "slots")]
            c = (key, MoeSplitC(*ptrs))
            self.__dict__["_abi"] = c
        return c[1]

    def to_host(self):
        """(active_rows, row_off, slots) as numpy, trimmed to n_active."""
        n = int(self.n_active.item())
        off = self.row_off[: n + 1].cpu().numpy()
        return (self.active_rows[:n].cpu().numpy(), off, self.slots[: int(off[-1])].cpu().numpy())


# ---------------------------------------------------------- entry points --

def moe_route_split(topk_ids, row_map, n_hot_rows: int, n_cold_rows: int, hot: Split, cold: Split,
                    n_invalid, counts_layer=None, count_tmax: int = 256, stream=None) -> None:
    T, k = int(topk_ids.shape[0]), int(topk_ids.shape[1])
    i32 = ("torch.int32",)
    E = int(row_map.shape[0])
    _check_split(hot, n_hot_rows, T, k, "hot split")
    _check_split(cold, n_cold_rows, T, k, "cold split")
    _need(n_invalid, "n_invalid", 4)
    if counts_layer is not None:
        _need(counts_layer, "counts_layer", 4 * E)
    _check(lib().moe_route_split(_gpu(topk_ids, "topk_ids", i32), T, k,
                                 _gpu(row_map, "row_map", i32), int(row_map.shape[0]),
                                 n_hot_rows, n_cold_rows, _gpu_opt(counts_layer, "counts", i32),
                                 count_tmax, hot.abi(), cold.abi(),
                                 _gpu(n_invalid, "n_invalid", i32), _stream(stream)))


def _ffn_sizes(bank: Bank, split: Split, T: int, k: int, H: int, I: int, workspace, Y) -> None:
    if T <= 0 or bank.n_rows == 0:
        return
    _check_bank(bank, H, I)
    # The split is read here, written by moe_route_split (whose wrapper checks
    # its capacities): a staged split pairs one bank's row lists with another
    # bank, so only the slot list's length is fixed by this call.
    if int(split.slots.numel()) < T * k:
        raise MoeError(MOE_EINVAL, f"split slots: {int(split.slots.numel())} entries, "
                                   f"need T*k = {T * k}")
    ws = moe_ffn_workspace_bytes(T, k, H, I)
    if ws == 0:
        raise MoeError(MOE_ENOTSUP, f"no workspace size for T={T}, k={k}, H={H}, I={I}")
    _need(workspace, "workspace", ws)
    if Y is not None:
        _need(Y, "Y", 2 * T * k * H)


def moe_expert_ffn_mxfp4(bank: Bank, split: Split, x, k: int, I: int, workspace, Y,
                         stream=None) -> None:
    T, H = int(x.shape[0]), int(x.shape[1])
    _ffn_sizes(bank, split, T, k, H, I, workspace, Y)
    b = bank.abi()
    _check(lib().moe_expert_ffn_mxfp4(ctypes.byref(b), split.abi(), _gpu(x, "x", _BF16_BITS), T, k,
                                      H, I, _gpu(workspace, "workspace"),
                                      _gpu(Y, "Y", _BF16_BITS), _stream(stream)))


def moe_expert_ffn_mxfp4_noalloc(bank: Bank, split: Split, x, k: int, I: int, Y,
                                 stream=None) -> None:
    """moe_expert_ffn_mxfp4 with the library's static scratch buffer instead of
    a workspace (allocates nothing; see the header for the size limit and the
    sharing rule)."""
    T, H = int(x.shape[0]), int(x.shape[1])
    if T > 0 and bank.n_rows > 0:
        _check_bank(bank, H, I)
        if int(split.slots.numel()) < T * k:
            raise MoeError(MOE_EINVAL, f"split slots: {int(split.slots.numel())} entries, "
                                       f"need T*k = {T * k}")
        _need(Y, "Y", 2 * T * k * H)
    b = bank.abi()
    _check(lib().moe_expert_ffn_mxfp4_noalloc(ctypes.byref(b), split.abi(),
                                              _gpu(x, "x", _BF16_BITS), T, k, H, I,
                                              _gpu(Y, "Y", _BF16_BITS), _stream(stream)))


def moe_expert_gate_up_mxfp4(bank: Bank, split: Split, x, k: int, I: int, workspace,
                             stream=None) -> None:
    T, H = int(x.shape[0]), int(x.shape[1])
    _ffn_sizes(bank, split, T, k, H, I, workspace, None)
    b = bank.abi()
    _check(lib().moe_expert_gate_up_mxfp4(ctypes.byref(b), split.abi(), _gpu(x, "x", _BF16_BITS),
                                          T, k, H, I, _gpu(workspace, "workspace"),
                                          _stream(stream)))


def moe_expert_down_mxfp4(bank: Bank, split: Split, T: int, k: int, H: int, I: int, workspace, Y,
                          stream=None) -> None:
    _ffn_sizes(bank, split, T, k, H, I, workspace, Y)
    b = bank.abi()
    _check(lib().moe_expert_down_mxfp4(ctypes.byref(b), split.abi(), T, k, H, I,
                                       _gpu(workspace, "workspace"), _gpu(Y, "Y", _BF16_BITS),
                                       _stream(stream)))


STAGE_GATE_UP, STAGE_DOWN, STAGE_ALL = 1, 2, 3


def moe_stage_rows(src: Bank, split: Split, T: int, k: int, dst: Bank, dst_rows, H: int, I: int,
                   parts: int = STAGE_ALL, stream=None) -> Split:
    """Copy src's active rows (per split) of the tensors `parts` names
    (STAGE_GATE_UP, STAGE_DOWN, STAGE_ALL) to rows 0.. of the device bank dst;
    returns the split that drives the expert FFN on dst."""
    if T > 0 and src.n_rows > 0:
        cap = min(src.n_rows, T * k)
        _check_bank(src, H, I, "src")
        _check_bank(dst, H, I, "dst")
        _check_split(split, src.n_rows, T, k)
        _need(dst_rows, "dst_rows", 4 * cap)
    s, d = src.abi(), dst.abi()
    _check(lib().moe_stage_rows(ctypes.byref(s), split.abi(), T, k, ctypes.byref(d),
                                _gpu(dst_rows, "dst_rows", ("torch.int32",)), H, I, int(parts),
                                _stream(stream)))
    return Split(split.n_active, dst_rows, split.row_off, split.slots)


def moe_stage_rows_dma(src: Bank, rows, dst: Bank, H: int, I: int, parts: int = STAGE_ALL,
                       stream=None) -> None:
    """Copy rows[a] of src's tensors that `parts` names to row a of the device
    bank dst with the DMA engines; rows: host int32 (a CPU tensor or array)."""
    import numpy as np
    r = np.ascontiguousarray(rows.cpu().numpy() if hasattr(rows, "cpu") else rows, dtype=np.int32)
    n = int(r.shape[0])
    if n > 0:
        _check_bank(src, H, I, "src")
        _check_bank(dst, H, I, "dst")
    s, d = src.abi(), dst.abi()
    _check(lib().moe_stage_rows_dma(ctypes.byref(s), r.ctypes.data if n else None, n,
                                    ctypes.byref(d), H, I, int(parts), _stream(stream)))


def moe_finalize(Y, topk_w, out, stream=None) -> None:
    T, k = int(topk_w.shape[0]), int(topk_w.shape[1])
    H = int(out.shape[1])
    _need(Y, "Y", 2 * T * k * H)
    _need(out, "out", 2 * T * H)
    _need(topk_w, "topk_w", 4 * T * k)
    _check(lib().moe_finalize(_gpu(Y, "Y", _BF16_BITS), _gpu(topk_w, "topk_w", ("torch.float32",)),
                              T, k, H, _gpu(out, "out", _BF16_BITS), _stream(stream)))


def moe_usage_counts(counts, host_dst, stream=None) -> None:
    L, E = int(counts.shape[0]), int(counts.shape[1])
    if str(getattr(host_dst, "dtype", "")) != "torch.int32" or host_dst.device.type != "cpu" or \
            not host_dst.is_pinned() or not host_dst.is_contiguous():
        raise _bad("host_dst", "a contiguous pinned host int32 tensor", host_dst)
    _need(host_dst, "host_dst", 4 * L * E)
    _check(lib().moe_usage_counts(_gpu(counts, "counts", ("torch.int32",)), L, E,
                                  host_dst.data_ptr(), _stream(stream)))


def moe_swap_rows(hot: Bank, cold: Bank, hot_row: int, cold_row: int, expect_hot_expert: int,
                  expect_cold_expert: int, row_map, hot_owner, cold_owner, staging, H: int, I: int,
                  stream=None) -> None:
    """hot_owner / cold_owner: host int32 arrays (numpy or CPU torch), updated in place."""

    def hptr(a):
        return a.ctypes.data if hasattr(a, "ctypes") else a.data_ptr()

    for name, a in (("hot_owner", hot_owner), ("cold_owner", cold_owner)):
        if str(a.dtype) not in ("int32", "torch.int32") or \
                not (a.flags["C_CONTIGUOUS"] if hasattr(a, "flags") else a.is_contiguous()) or \
                getattr(getattr(a, "device", None), "type", "cpu") != "cpu":
            raise _bad(name, "a contiguous host int32 array", a)
    _check_bank(hot, H, I, "hot bank")
    _check_bank(cold, H, I, "cold bank")
    for name, a, b in (("hot_owner", hot_owner, hot), ("cold_owner", cold_owner, cold)):
        n = a.size if hasattr(a, "size") and not callable(a.size) else a.numel()
        if int(n) != b.n_rows:
            raise MoeError(MOE_EINVAL, f"{name}: {int(n)} entries for a bank of {b.n_rows} rows")
    hb, cb = hot.abi(), cold.abi()
    nbytes = staging.numel() * staging.element_size()
    _check(lib().moe_swap_rows(ctypes.byref(hb), ctypes.byref(cb), hot_row, cold_row,
                               expect_hot_expert, expect_cold_expert,
                               _gpu(row_map, "row_map", ("torch.int32",)),
                               int(row_map.shape[0]), hptr(hot_owner), hptr(cold_owner),
                               _gpu(staging, "staging"), nbytes, H, I, _stream(stream)))
