"""The C ABI library without a GPU: it loads, exports every function the
header declares, and its host-side checks reject bad arguments before any
GPU call."""
import ctypes
import os
import re

import numpy as np
import pytest

import expert_weight_residency_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_residency.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail(f"library not built: {moe.LIB_PATH}")
    return moe.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(moe.ENTRY_POINTS), names
    raw = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_sizes(L):
    assert moe.moe_expert_bytes(4096, 2880) == 18_800_640
    assert moe.moe_expert_bytes(256, 128) == 52_224
    assert moe.moe_ffn_workspace_bytes(16, 6, 4096, 2880) == 16 * 6 * 2880 * 2
    assert moe.moe_ffn_workspace_bytes(255, 6, 4096, 2880) == 255 * 6 * 2880 * 2
    # prefill-sized steps: x and h per slot as two E4M3 terms (512 data + 16 scale
    # bytes per 256-element chunk; H = 4096 -> 16 chunks, I = 2880 -> 12)
    assert moe.moe_ffn_workspace_bytes(256, 6, 4096, 2880) == 256 * 6 * (16 + 12) * 528
    assert moe.moe_ffn_workspace_bytes(0, 6, 4096, 2880) == 0


def _split(p=0x1000):
    return moe.MoeSplitC(p, p, p, p)


def test_route_split_rejects_bad_shapes(L):
    p = 0x1000
    assert L.moe_route_split(p, -1, 6, p, 384, 295, 89, None, 256, _split(), _split(), p, None) == moe.MOE_EINVAL
    assert L.moe_route_split(p, 4, 0, p, 384, 295, 89, None, 256, _split(), _split(), p, None) == moe.MOE_EINVAL
    assert L.moe_route_split(p, 4, 6, p, 0, 0, 0, None, 256, _split(), _split(), p, None) == moe.MOE_EINVAL
    assert L.moe_route_split(p, 4, 6, p, 384, 5000, 89, None, 256, _split(), _split(), p, None) == moe.MOE_EINVAL
    assert L.moe_route_split(p, 4, 6, None, 384, 295, 89, None, 256, _split(), _split(), p, None) == moe.MOE_EINVAL
    assert L.moe_route_split(p, 4, 6, p, 384, 295, 89, None, 256, _split(0), _split(), p, None) == moe.MOE_EINVAL
    assert "split" in moe.moe_last_error()


def test_ffn_rejects_bad_shapes(L):
    p = 0x1000
    bank = moe.MoeBankC(p, p, p, p, 4, 0)
    for (H, I) in ((4000, 2880), (4096, 2850), (0, 64)):
        assert L.moe_expert_ffn_mxfp4(ctypes.byref(bank), _split(), p, 4, 2, H, I, p, p, None) == moe.MOE_EINVAL
    assert L.moe_expert_ffn_mxfp4(None, _split(), p, 4, 2, 256, 128, p, p, None) == moe.MOE_EINVAL
    # misaligned activations
    assert L.moe_expert_ffn_mxfp4(ctypes.byref(bank), _split(), p + 2, 4, 2, 256, 128, p, p, None) == moe.MOE_EINVAL
    # nothing to do is success without touching the GPU
    empty = moe.MoeBankC(p, p, p, p, 0, 0)
    assert L.moe_expert_ffn_mxfp4(ctypes.byref(empty), _split(), p, 4, 2, 256, 128, p, p, None) == moe.MOE_OK
    assert L.moe_expert_ffn_mxfp4(ctypes.byref(bank), _split(), p, 0, 2, 256, 128, p, p, None) == moe.MOE_OK


def test_stage_rows_rejects_bad_args(L):
    """Argument errors of moe_stage_rows come back before any GPU call (device
    banks: no pointer translation either)."""
    p = 0x1000
    src = moe.MoeBankC(p, p, p, p, 10, 0)
    dst = moe.MoeBankC(p, p, p, p, 10, 0)
    rows = p

    def call(src_=src, dst_=dst, T=4, k=2, H=256, I=128, parts=moe.STAGE_ALL, split=None):
        return L.moe_stage_rows(ctypes.byref(src_) if src_ is not None else None,
                                split or _split(), T, k,
                                ctypes.byref(dst_) if dst_ is not None else None, rows, H, I,
                                parts, None)

    for parts in (0, 4, -1):
        assert call(parts=parts) == moe.MOE_EINVAL
        assert "parts" in moe.moe_last_error()
    assert call(k=0) == moe.MOE_EINVAL
    assert call(H=100) == moe.MOE_EINVAL
    assert call(src_=None) == moe.MOE_EINVAL
    assert call(dst_=None) == moe.MOE_EINVAL
    assert call(dst_=moe.MoeBankC(p, p, p, p, 10, 1)) == moe.MOE_EINVAL  # dst in host memory
    assert "device bank" in moe.moe_last_error()
    # the split can name min(10, 4*2) = 8 rows; a 7-row stage is too small
    assert call(dst_=moe.MoeBankC(p, p, p, p, 7, 0)) == moe.MOE_EINVAL
    assert call(split=_split(0)) == moe.MOE_EINVAL
    # a scale tensor off 16-byte alignment is refused only when its part is staged
    odd = moe.MoeBankC(p, p + 2, p, p, 10, 0)
    assert call(src_=odd, parts=moe.STAGE_GATE_UP) == moe.MOE_EINVAL
    assert "aligned" in moe.moe_last_error()
    assert call(src_=odd, T=0) == moe.MOE_OK  # nothing to do: no launch, no error
    assert call(src_=moe.MoeBankC(p, p, p, p, 0, 0)) == moe.MOE_OK


def test_stage_rows_dma_rejects_bad_args(L):
    """Argument errors of moe_stage_rows_dma come back before any copy is
    enqueued (device banks: no pointer translation either)."""
    p = 0x1000
    src = moe.MoeBankC(p, p, p, p, 10, 0)
    dst = moe.MoeBankC(p, p, p, p, 4, 0)

    def call(rows, n=None, src_=src, dst_=dst, H=256, I=128, parts=moe.STAGE_ALL):
        r = np.ascontiguousarray(rows, dtype=np.int32)
        return L.moe_stage_rows_dma(ctypes.byref(src_) if src_ is not None else None,
                                    r.ctypes.data if r.size else None,
                                    len(r) if n is None else n,
                                    ctypes.byref(dst_) if dst_ is not None else None, H, I,
                                    parts, None)

    for parts in (0, 4, -1):
        assert call([1, 2], parts=parts) == moe.MOE_EINVAL
        assert "parts" in moe.moe_last_error()
    assert call([1, 2], n=-1) == moe.MOE_EINVAL
    assert call([1, 2], H=100) == moe.MOE_EINVAL
    assert call([1, 2], src_=None) == moe.MOE_EINVAL
    assert call([1, 10]) == moe.MOE_EINVAL  # row outside the source bank
    assert "rows[1]" in moe.moe_last_error()
    assert call([-1]) == moe.MOE_EINVAL
    assert call([0, 1, 2, 3, 4]) == moe.MOE_EINVAL  # 5 rows into a 4-row stage
    assert "dst holds" in moe.moe_last_error()
    assert call([1], dst_=moe.MoeBankC(p, p, p, p, 4, 1)) == moe.MOE_EINVAL  # dst on the host
    assert call([1], dst_=moe.MoeBankC(p, p, p, p, 4, moe.BANK_HOST_WEIGHTS)) == moe.MOE_EINVAL
    assert call([1], src_=moe.MoeBankC(p, p, p, p, 10, 3)) == moe.MOE_EINVAL  # no such placement
    assert "on_host=3" in moe.moe_last_error()
    assert L.moe_stage_rows_dma(ctypes.byref(src), None, 1, ctypes.byref(dst), 256, 128, 3,
                                None) == moe.MOE_EINVAL  # rows NULL
    assert call([]) == moe.MOE_OK  # nothing to copy


def test_finalize_and_counts_reject_bad_args(L):
    p = 0x1000
    assert L.moe_finalize(p, p, 4, 2, 12, p, None) == moe.MOE_EINVAL
    assert L.moe_finalize(p, p, 4, 99, 16, p, None) == moe.MOE_EINVAL
    assert L.moe_finalize(p, p, 0, 2, 16, p, None) == moe.MOE_OK
    assert L.moe_usage_counts(p, 40, 0, p, None) == moe.MOE_EINVAL
    assert L.moe_usage_counts(None, 40, 384, p, None) == moe.MOE_EINVAL


def test_swap_stale_check_runs_on_host(L):
    """A swap decided against outdated owner lists is refused before anything
    is enqueued, and the mirrors are untouched."""
    p = 0x1000
    hot = moe.MoeBankC(p, p, p, p, 3, 0)
    cold = moe.MoeBankC(p, p, p, p, 2, 0)
    hot_owner = np.array([4, 5, 6], np.int32)
    cold_owner = np.array([1, 2], np.int32)
    need = moe.moe_expert_bytes(256, 128)
    rc = L.moe_swap_rows(ctypes.byref(hot), ctypes.byref(cold), 1, 0, 6, 1, p, 8,
                         hot_owner.ctypes.data, cold_owner.ctypes.data, p, need, 256, 128, None)
    assert rc == moe.MOE_ESTALE
    assert "stale" in moe.moe_last_error()
    assert hot_owner.tolist() == [4, 5, 6] and cold_owner.tolist() == [1, 2]
    # staging too small / bad rows are argument errors
    assert L.moe_swap_rows(ctypes.byref(hot), ctypes.byref(cold), 1, 0, 5, 1, p, 8,
                           hot_owner.ctypes.data, cold_owner.ctypes.data, p, need - 1, 256, 128,
                           None) == moe.MOE_EINVAL
    assert L.moe_swap_rows(ctypes.byref(hot), ctypes.byref(cold), 3, 0, 5, 1, p, 8,
                           hot_owner.ctypes.data, cold_owner.ctypes.data, p, need, 256, 128,
                           None) == moe.MOE_EINVAL
    nowhere = moe.MoeBankC(p, p, p, p, 2, 3)  # no such placement
    assert L.moe_swap_rows(ctypes.byref(hot), ctypes.byref(nowhere), 1, 0, 5, 1, p, 8,
                           hot_owner.ctypes.data, cold_owner.ctypes.data, p, need, 256, 128,
                           None) == moe.MOE_EINVAL
    assert "on_host=3" in moe.moe_last_error()


def test_python_errors_raise(L):
    with pytest.raises(moe.MoeError):
        moe._check(moe.MOE_EINVAL)
    with pytest.raises(moe.MoeStale):
        moe._check(moe.MOE_ESTALE)


def test_binding_rejects_bad_tensors(L):
    """CPU tensors, wrong dtypes and strided views are refused on the host
    (MoeError, MOE_EINVAL) before any pointer reaches the library."""
    import torch
    cpu_i32 = torch.zeros((4, 2), dtype=torch.int32)
    split = moe.Split(*(torch.zeros(8, dtype=torch.int32) for _ in range(4)))
    with pytest.raises(moe.MoeError) as e:
        moe.moe_route_split(cpu_i32, torch.zeros(8, dtype=torch.int32), 6, 2, split, split,
                            torch.zeros(1, dtype=torch.int32))
    assert e.value.code == moe.MOE_EINVAL and "topk_ids" in str(e.value)
    with pytest.raises(moe.MoeError) as e:
        split.abi()
    assert "split n_active" in str(e.value)
    bank = moe.Bank(*(torch.zeros((2, 4), dtype=torch.uint8) for _ in range(4)), on_host=False)
    with pytest.raises(moe.MoeError) as e:
        bank.abi()
    assert "GPU memory" in str(e.value)
    host = moe.Bank(*(torch.zeros((2, 4), dtype=torch.uint8) for _ in range(4)), on_host=True)
    with pytest.raises(moe.MoeError) as e:  # not pinned
        host.abi()
    assert "pinned" in str(e.value)
    split_host = moe.Bank(*(torch.zeros((2, 4), dtype=torch.uint8) for _ in range(4)),
                          on_host=moe.BANK_HOST_WEIGHTS)
    with pytest.raises(moe.MoeError) as e:  # weights must be pinned host memory
        split_host.abi()
    assert "bank w13" in str(e.value) and "pinned" in str(e.value)
    nowhere = moe.Bank(*(torch.zeros((2, 4), dtype=torch.uint8) for _ in range(4)), on_host=3)
    with pytest.raises(moe.MoeError) as e:
        nowhere.abi()
    assert e.value.code == moe.MOE_EINVAL and "on_host=3" in str(e.value)
    wrong = moe.Bank(*(torch.zeros((2, 4), dtype=torch.int16) for _ in range(4)))
    with pytest.raises(moe.MoeError) as e:
        wrong.abi()
    assert "uint8" in str(e.value)
    strided = torch.zeros((4, 4), dtype=torch.int32)[:, ::2]
    with pytest.raises(moe.MoeError):
        moe._gpu(strided, "x", ("torch.int32",))
    with pytest.raises(moe.MoeError) as e:
        moe.moe_usage_counts(torch.zeros((2, 8), dtype=torch.int32),
                             torch.zeros((2, 8), dtype=torch.int32))
    assert "host_dst" in str(e.value)
    ho = np.zeros(3, np.int64)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_swap_rows(bank, bank, 0, 0, 0, 0, None, ho, ho, None, 256, 128)
    assert "hot_owner" in str(e.value)


def test_fp4_step_past_32bit_offsets_is_refused(L):
    """The FP4 path addresses each quantized activation region with 32-bit
    byte offsets: a step whose region would reach 4 GB is refused before any
    work (MOE_ENOTSUP), and its workspace size reads 0."""
    p = 0x1000
    bank = moe.MoeBankC(p, p, p, p, 295, 0)
    # H = 4096: 16 chunks of 512 bytes per slot row -> 2^32 bytes at 524,288 slots
    T_ok, T_bad = 524_287 // 6, 524_288 // 6 + 1
    assert moe.moe_ffn_workspace_bytes(T_ok, 6, 4096, 2880) > 0
    assert moe.moe_ffn_workspace_bytes(T_bad, 6, 4096, 2880) == 0
    for fn in ("moe_expert_ffn_mxfp4",):
        rc = getattr(L, fn)(ctypes.byref(bank), _split(), p, T_bad, 6, 4096, 2880, p, p, None)
        assert rc == moe.MOE_ENOTSUP, rc
        assert "32-bit" in moe.moe_last_error()
    assert L.moe_expert_gate_up_mxfp4(ctypes.byref(bank), _split(), p, T_bad, 6, 4096, 2880, p,
                                      None) == moe.MOE_ENOTSUP
    assert L.moe_expert_down_mxfp4(ctypes.byref(bank), _split(), T_bad, 6, 4096, 2880, p, p,
                                   None) == moe.MOE_ENOTSUP
    # the largest hidden size: 128 chunks per row -> the limit is 65,536 slots
    assert moe.moe_ffn_workspace_bytes(65_535 // 2, 2, 32768, 2880) > 0
    assert moe.moe_ffn_workspace_bytes(65_536 // 2, 2, 32768, 2880) == 0


def test_binding_rejects_undersized_buffers(L):
    """Buffers too small for the call's sizes are refused on the host
    (MOE_EINVAL) before anything reaches the library: workspace, Y, split
    capacities, bank tensors that do not hold n_rows rows at (H, I), the
    finalize's and the counter snapshot's buffers, owner mirrors."""
    import torch
    T, k, H, I, R = 16, 6, 256, 128, 10
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    bank = moe.Bank(u8(R, 2 * I, H // 2), u8(R, 2 * I, H // 32), u8(R, H, I // 2),
                    u8(R, H, I // 32))
    split = moe.Split.empty(R, T, k, device="cpu")
    x = torch.zeros((T, H), dtype=torch.int16)
    Y = torch.zeros((T * k, H), dtype=torch.int16)
    ws = u8(moe.moe_ffn_workspace_bytes(T, k, H, I))

    def raises(fn, *a, match):
        with pytest.raises(moe.MoeError) as e:
            fn(*a)
        assert e.value.code == moe.MOE_EINVAL and match in str(e.value), str(e.value)

    raises(moe.moe_expert_ffn_mxfp4, bank, split, x, k, I, ws[:-16], Y, match="workspace")
    raises(moe.moe_expert_ffn_mxfp4, bank, split, x, k, I, ws, Y[:-1], match="Y")
    raises(moe.moe_expert_down_mxfp4, bank, split, T, k, H, I, ws, Y[:-1], match="Y")
    raises(moe.moe_expert_gate_up_mxfp4, bank, split, x, k, I, ws[:-16], match="workspace")
    short = moe.Split(split.n_active, split.active_rows, split.row_off, split.slots[:-1])
    raises(moe.moe_expert_ffn_mxfp4, bank, short, x, k, I, ws, Y, match="slots")
    thin = moe.Bank(bank.w13, bank.s13, bank.w2[:, :, :-16].contiguous(), bank.s2)
    raises(moe.moe_expert_ffn_mxfp4, thin, split, x, k, I, ws, Y, match="w2")
    # a prefill-sized step needs the FP4 workspace, ~10x the decode one per slot
    Tp = 256
    raises(moe.moe_expert_ffn_mxfp4, bank, moe.Split.empty(R, Tp, k, device="cpu"),
           torch.zeros((Tp, H), dtype=torch.int16), k, I,
           u8(moe.moe_ffn_workspace_bytes(Tp - 1, k, H, I)),
           torch.zeros((Tp * k, H), dtype=torch.int16), match="workspace")
    # route split: capacities for min(rows, T*k) active rows and T*k slots
    ids, rm, ninv = i32(T, k), i32(384), i32(1)
    small = moe.Split(i32(1), i32(R - 1), i32(R + 1), i32(T * k))
    raises(moe.moe_route_split, ids, rm, R, 0, small, split, ninv, match="active_rows")
    small = moe.Split(i32(1), i32(R), i32(R), i32(T * k))
    raises(moe.moe_route_split, ids, rm, R, 0, small, split, ninv, match="row_off")
    small = moe.Split(i32(1), i32(R), i32(R + 1), i32(T * k - 1))
    raises(moe.moe_route_split, ids, rm, R, 0, small, split, ninv, match="slots")
    raises(moe.moe_route_split, ids, rm, R, 0, split, split, ninv, i32(383), match="counts")
    # finalize and the snapshot
    w = torch.zeros((T, k), dtype=torch.float32)
    raises(moe.moe_finalize, Y[:-1], w, torch.zeros((T, H), dtype=torch.int16), match="Y")
    raises(moe.moe_finalize, Y, w, torch.zeros((T - 1, H), dtype=torch.int16), match="out")
    # owners must have one entry per bank row
    raises(moe.moe_swap_rows, bank, bank, 0, 0, 1, 2, i32(384), np.zeros(R - 1, np.int32),
           np.zeros(R, np.int32), u8(16), H, I, match="hot_owner")


def test_abi_cache_follows_tensor_storage(L):
    """The cached C struct of a bank or split is rebuilt when a field is
    replaced by another tensor (the cache is keyed on data pointers)."""
    import torch
    b = moe.Bank(*(torch.zeros((2, 4), dtype=torch.uint8) for _ in range(4)))
    key = lambda: (b.w13.data_ptr(), b.s13.data_ptr(), b.w2.data_ptr(), b.s2.data_ptr())
    b.__dict__["_abi"] = ((key() + (b.n_rows, b.on_host)), "cached")
    assert b.abi() == "cached"
    b.w2 = torch.ones((2, 4), dtype=torch.uint8)   # new storage: the cache must not be used
    with pytest.raises(moe.MoeError):               # rebuilt: CPU tensors are refused
        b.abi()
