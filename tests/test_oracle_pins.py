"""Pins for the CPU oracle: each test checks it against something other than
itself (a published value table, a closed form, a textbook routine, brute force
or a crafted input whose exact answer is known), so that a dropped term, a
wrong sign or index, or a transposed operand fails at least one of them."""
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def pow2_from_exponent_field(b: int) -> float:
    """2^(b-127) built as an fp32 bit pattern (exponent field b, zero mantissa);
    b = 0 is the subnormal 2^-127 (mantissa bit 22)."""
    bits = (b << 23) if b > 0 else (1 << 22)
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def e2m1_table(golden_dir):
    vals = {}
    with open(os.path.join(golden_dir, "e2m1_ocp_mx.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                vals[int(c)] = float(v)
    return vals


# ------------------------------------------------------------ formats --

def test_e2m1_matches_published_table(golden_dir):
    table = e2m1_table(golden_dir)
    assert sorted(table) == list(range(16))
    for c, v in table.items():
        got = oracle.e2m1(c)
        assert got == v, (c, got, v)
        assert math.copysign(1.0, got) == math.copysign(1.0, v), c  # -0 for code 8


def test_e8m0_all_bytes():
    for b in range(255):
        assert oracle.e8m0(b) == pow2_from_exponent_field(b), b
    assert math.isnan(oracle.e8m0(255))


def test_dequant_every_code_scale_pair(golden_dir):
    """All 16 x 255 (code, scale) pairs, with both nibble positions and several
    scale blocks in one row."""
    table = e2m1_table(golden_dir)
    K = 64  # two scale blocks
    for b in range(255):
        for c in range(16):
            # even elements carry code c (low nibble), odd elements carry 15-c (high nibble)
            w = np.full((1, K // 2), c | ((15 - c) << 4), np.uint8)
            s = np.array([[b, (b + 1) % 255]], np.uint8)
            got = oracle.dequant(w, s, K)[0]
            s0, s1 = pow2_from_exponent_field(b), pow2_from_exponent_field((b + 1) % 255)
            exact = np.array([(table[c] if e % 2 == 0 else table[15 - c]) * (s0 if e < 32 else s1)
                              for e in range(K)], np.float64)
            with np.errstate(over="ignore"):
                exp = exact.astype(np.float32)   # exact, or +-inf past the fp32 range
            assert np.array_equal(got, exp), (b, c)
            assert np.array_equal(np.signbit(got), np.signbit(exp)), (b, c)


# -------------------------------------------------------------- silu --

def test_silu_closed_form():
    from scipy.special import expit  # library logistic sigmoid
    zs = np.concatenate([np.linspace(-100, 100, 20001), [-700.0, -50.5, 0.0, 1e-300, 50.5, 745.0]])
    for z in zs:
        ref = z * float(expit(z))
        got = oracle.silu(float(z))
        assert abs(got - ref) <= 4e-15 * abs(ref) + 1e-320, (z, got, ref)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(-800.0) == 0.0 or oracle.silu(-800.0) < 0  # underflows towards -0


# ---------------------------------------------------------- bf16 RNE --

def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(2000).astype(np.float32) * np.float32(3.0))
    # exact ties at the 16th bit, both parities, and specials
    for base in (0x3F800000, 0x3F810000, 0xC0490000, 0x00010000, 0x7F7F0000):
        vals.append(struct.unpack("<f", struct.pack("<I", base | 0x8000))[0])
        vals.append(struct.unpack("<f", struct.pack("<I", base | 0x7FFF))[0])
        vals.append(struct.unpack("<f", struct.pack("<I", base | 0x8001))[0])
    vals += [0.0, -0.0, float("inf"), float("-inf"), 3.4028234e38, 1e-45]
    a = np.array(vals, np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(a)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------- FFN pins --

def _pack(codes: np.ndarray) -> np.ndarray:
    """[rows, K] codes -> [rows, K/2] bytes, low nibble = even element."""
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_ffn_all_ones_closed_form():
    H, I = 256, 128
    x = synth.activations(1, H, seed=3)[0]
    w13 = np.full((2 * I, H // 2), 0x22, np.uint8)   # code 2 = 1.0 in both nibbles
    s13 = np.full((2 * I, H // 32), 127, np.uint8)   # scale 2^0
    w2 = np.full((H, I // 2), 0x22, np.uint8)
    s2 = np.full((H, I // 32), 127, np.uint8)
    r = oracle.expert_ffn(w13, s13, w2, s2, x, H, I)
    xs = oracle.bf16_to_f32(x).astype(np.float64)
    sx = np.float32(math.fsum(xs))               # exact sum, one rounding
    assert np.all(r["g"] == sx) and np.all(r["u"] == sx)
    sig = 0.5 * (1.0 + math.tanh(float(sx) / 2.0))
    h_ref = np.float32(float(sx) * sig * float(sx))
    assert np.allclose(r["h"], h_ref, rtol=2e-7, atol=0)
    y_ref = math.fsum([float(v) for v in r["h"]])
    assert np.allclose(r["y"], np.float32(y_ref), rtol=2e-7, atol=0)


def test_ffn_one_hot_rows_pin_layout():
    """Each gate row i picks x[pg(i)], each up row i picks 2*x[pu(i)] (code 6 =
    4.0 with scale 2^-1), each down row o picks h[pd(o)] times 1.5 (code 3).
    Pins gate/up order, rows vs columns, nibble order, scale-block index and
    silu(g)*u (not silu(u)*g)."""
    H, I = 256, 64
    rng = np.random.default_rng(11)
    pg, pu = rng.integers(0, H, I), rng.integers(0, H, I)
    pd = rng.integers(0, I, H)
    c13 = np.zeros((2 * I, H), np.int64)
    s13 = np.full((2 * I, H // 32), 127, np.uint8)
    for i in range(I):
        c13[i, pg[i]] = 2
        c13[I + i, pu[i]] = 6
        s13[I + i, pu[i] // 32] = 126
    c2 = np.zeros((H, I), np.int64)
    for o in range(H):
        c2[o, pd[o]] = 3
    w13, w2 = _pack(c13), _pack(c2)
    s2 = np.full((H, I // 32), 127, np.uint8)
    x = synth.activations(1, H, seed=5)[0]
    xf = oracle.bf16_to_f32(x)
    r = oracle.expert_ffn(w13, s13, w2, s2, x, H, I)
    assert np.array_equal(r["g"], xf[pg])
    assert np.array_equal(r["u"], np.float32(2.0) * xf[pu])
    g = r["g"].astype(np.float64)
    silu = g * 0.5 * (1.0 + np.tanh(g / 2.0))
    h_ref = (silu * r["u"].astype(np.float64)).astype(np.float32)
    assert np.allclose(r["h"], h_ref, rtol=1e-6, atol=1e-30)
    # the swapped form silu(u)*g must not match (unless the draw were degenerate)
    u = r["u"].astype(np.float64)
    wrong = (u * 0.5 * (1.0 + np.tanh(u / 2.0)) * g).astype(np.float32)
    assert not np.allclose(r["h"], wrong, rtol=1e-3)
    assert np.array_equal(r["y"], (np.float64(1.5) * r["h"].astype(np.float64)[pd]).astype(np.float32))


def _np_dequant(w, s, K, table):
    """Independent dequant: nibble unpack + table + 2^(b-127) from bits."""
    lo, hi = w & 15, w >> 4
    codes = np.empty((w.shape[0], K), np.int64)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    vals = np.array([table[c] for c in range(16)])[codes]
    sc = np.array([pow2_from_exponent_field(b) if b < 255 else np.nan for b in range(256)])
    return vals * np.repeat(sc[s], 32, axis=1)


@pytest.mark.parametrize("H,I", [(256, 128), (512, 320), (1024, 512)])
def test_ffn_matches_numpy_float64_matmul(H, I, golden_dir):
    table = e2m1_table(golden_dir)
    bank = synth.make_bank_host([3], seed=9, layer=1, H=H, I=I)
    x = synth.activations(2, H, seed=9)
    W13 = _np_dequant(bank["w13"][0], bank["s13"][0], H, table)
    W2 = _np_dequant(bank["w2"][0], bank["s2"][0], I, table)
    for t in range(2):
        r = oracle.expert_ffn(bank["w13"][0], bank["s13"][0], bank["w2"][0], bank["s2"][0], x[t], H, I)
        xf = oracle.bf16_to_f32(x[t]).astype(np.float64)
        g = (W13[:I] @ xf).astype(np.float32)
        u = (W13[I:] @ xf).astype(np.float32)
        assert np.allclose(r["g"], g, rtol=1e-6, atol=1e-6 * np.abs(g).max())
        assert np.allclose(r["u"], u, rtol=1e-6, atol=1e-6 * np.abs(u).max())
        gd = r["g"].astype(np.float64)
        h = (gd / (1.0 + np.exp(-gd)) * r["u"].astype(np.float64)).astype(np.float32)
        assert np.allclose(r["h"], h, rtol=1e-6, atol=1e-6 * np.abs(h).max())
        y = W2 @ r["h"].astype(np.float64)
        rel = np.linalg.norm(r["y"] - y) / np.linalg.norm(y)
        assert rel < 1e-6, rel
        yb = oracle.bf16_to_f32(r["y_bf16"]).astype(np.float64)
        assert np.all(np.abs(yb - r["y"]) <= np.abs(r["y"]) * 2.0 ** -8 + 1e-38)


# ------------------------------------------------------------ finalize --

def test_finalize_k1_unit_weight_is_identity():
    rng = np.random.default_rng(1)
    Y = rng.integers(0, 65536, (5, 1, 64)).astype(np.uint16)
    Y[(Y & 0x7F80) == 0x7F80] = 0x3F80  # no Inf/NaN
    out = oracle.finalize(Y, np.ones((5, 1), np.float32))
    # +0.0 + 1*y is y (and -0 + +0 -> +0 for y = -0)
    Yf = oracle.bf16_to_f32(Y[:, 0, :])
    exp = np.where(Yf == 0, np.uint16(0), Y[:, 0, :])
    assert np.array_equal(out, exp)


def _bits16(x: float) -> int:
    return f32_bits(x) >> 16


def test_finalize_uses_fused_multiply_add():
    # term0 = w0*y0 = -(1 + 2^-7 + 2^-20); term1 = (1 + 2^-20)(1 + 2^-7) needs 28 bits.
    # fma keeps the 2^-27 remainder; round-then-add would give 0.
    w = np.array([[-(1 + 2.0 ** -7 + 2.0 ** -20), 1 + 2.0 ** -20]], np.float32)
    Y = np.array([[[_bits16(1.0)], [_bits16(1 + 2.0 ** -7)]]], np.uint16)
    out = oracle.finalize(Y, w)
    assert oracle.bf16_to_f32(out)[0, 0] == 2.0 ** -27


def test_finalize_order_and_ties_to_even():
    # order 0,1,2 gives exactly 1 + 2^-8 (a bf16 tie -> 1.0); order 2,1,0 gives
    # 1 + 2^-8 + 2^-23 (rounds up to 1 + 2^-7).
    w = np.array([[1 + 2.0 ** -8, 2.0 ** -24, 2.0 ** -24]], np.float32)
    Y = np.full((1, 3, 1), _bits16(1.0), np.uint16)
    fwd = oracle.finalize(Y, w)
    rev = oracle.finalize(Y[:, ::-1].copy(), w[:, ::-1].copy())
    assert fwd[0, 0] == 0x3F80
    assert rev[0, 0] == 0x3F81


def test_combine_weights_sum_to_one():
    for T, k, E in ((8, 2, 16), (16, 6, 384), (112, 6, 384)):
        ids, w = synth.skewed_routing(T, k, E, seed=4, layer=2, step=3) if E > 16 else \
            synth.gaussian_routing(T, k, E, seed=4)
        s = w.astype(np.float64).sum(axis=1)
        assert np.all(np.abs(s - 1.0) <= 4 * k * 2.0 ** -24)
        assert np.all(w > 0)
        for row in ids:
            assert len(set(row.tolist())) == k


# --------------------------------------------------------- split/count --

def _brute_split(ids, row_map, n_hot, n_cold):
    T, k = ids.shape
    E = len(row_map)
    hot, cold, bad = {}, {}, 0
    for s in range(T * k):
        e = int(ids.reshape(-1)[s])
        if not 0 <= e < E:
            bad += 1
            continue
        m = int(row_map[e])
        if 0 <= m < n_hot:
            hot.setdefault(m, []).append(s)
        elif m < 0 and -1 - m < n_cold:
            cold.setdefault(-1 - m, []).append(s)
        else:
            bad += 1
    return hot, cold, bad


def _check_split(res, hot, cold, bad):
    assert res["n_invalid"] == bad
    for name, ref in (("hot", hot), ("cold", cold)):
        active, off, slots = res[name]
        assert active.tolist() == sorted(ref)
        assert off[0] == 0 and len(off) == len(active) + 1
        for a, r in enumerate(active):
            assert slots[off[a]:off[a + 1]].tolist() == ref[int(r)]


def test_route_split_brute_force():
    rng = np.random.default_rng(21)
    for trial in range(200):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 6) + 1))
        T = int(rng.integers(0, 20))
        n_cold = int(rng.integers(0, E + 1))
        row_map, ho, co = synth.random_map(E, n_cold, seed=trial)
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
        if trial % 7 == 0 and T:
            ids[0, 0] = E + 3            # out-of-range id
        if trial % 11 == 0 and T:
            ids[-1, -1] = -2
        res = oracle.route_split(ids, row_map, len(ho), len(co))
        _check_split(res, *_brute_split(ids, row_map, len(ho), len(co)))
        # hot + cold + invalid partition all picks
        n = sum(len(res[b][2]) for b in ("hot", "cold")) + res["n_invalid"]
        assert n == T * k


def test_route_split_bad_map_rows_are_invalid():
    row_map = np.array([0, 5, -1, -9], np.int32)  # hot row 5 and cold row 8 do not exist
    ids = np.array([[0, 1], [2, 3]], np.int32)
    res = oracle.route_split(ids, row_map, n_hot=2, n_cold=2)
    _check_split(res, *_brute_split(ids, row_map, 2, 2))
    assert res["n_invalid"] == 2


def test_usage_counter():
    E, k = 384, 6
    base = np.arange(E, dtype=np.int32)
    for T in (1, 7, 16, 256):
        ids, _ = synth.skewed_routing(T, k, E, seed=1, layer=0, step=T)
        c = oracle.usage_count(base, ids, E)
        assert int((c - base).sum()) == T * k
        assert np.array_equal(c - base, np.bincount(ids.ravel(), minlength=E))
    ids, _ = synth.skewed_routing(257, k, E, seed=1, layer=0, step=0)
    assert np.array_equal(oracle.usage_count(base, ids, E), base)   # prefill-sized: not counted
    wrap = np.full(E, 2**31 - 1, np.int32)
    c = oracle.usage_count(wrap, np.array([[0]], np.int32), E)
    assert c[0] == -2**31                                              # int32 wraps, readers diff mod 2^32


# ---------------------------------------------------------------- swaps --

def _banks_for_map(E, row_map, hot_owner, cold_owner, H, I, seed, layer):
    return (oracle.Bank(**synth.make_bank_host(hot_owner, seed, layer, H, I)),
            oracle.Bank(**synth.make_bank_host(cold_owner, seed, layer, H, I)))


def _expert_bytes_where_map_says(e, row_map, hot, cold):
    m = int(row_map[e])
    b, r = (hot, m) if m >= 0 else (cold, -1 - m)
    return [getattr(b, t)[r].tobytes() for t in ("w13", "s13", "w2", "s2")]


def _expected_expert_bytes(e, H, I, seed, layer):
    one = synth.make_bank_host([e], seed, layer, H, I)
    return [one[t][0].tobytes() for t in ("w13", "s13", "w2", "s2")]


def test_five_ordered_swaps_at_page_geometry():
    """384 experts, 295 hot / 89 cold (the pages' dry-run geometry), small
    expert shapes. After each swap every expert's bytes are where the map says,
    and the layer output is bit-identical to before."""
    E, n_cold, H, I, seed, layer = 384, 89, 64, 32, 5, 0
    row_map, ho, co = synth.fitted_map(E, n_cold, seed, layer)
    hot, cold = _banks_for_map(E, row_map, ho, co, H, I, seed, layer)
    ids, w = synth.skewed_routing(16, 6, E, seed, layer, step=0)
    ids[0, :] = [int(co[0]), int(co[1]), int(ho[0]), int(ho[1]), int(co[2]), int(ho[2])]
    x = synth.activations(16, H, seed)
    _, out0, bad = oracle.moe_layer(hot, cold, row_map, ids, w, x, H, I)
    assert bad == 0
    expected = {e: _expected_expert_bytes(e, H, I, seed, layer) for e in range(E)}
    rng = np.random.default_rng(3)
    for n in range(5):
        a, b = int(rng.integers(len(ho))), int(rng.integers(len(co)))
        oracle.swap_rows(hot, cold, a, b, int(ho[a]), int(co[b]), row_map, ho, co)
        for e in range(E):
            assert _expert_bytes_where_map_says(e, row_map, hot, cold) == expected[e], (n, e)
        _, out, _ = oracle.moe_layer(hot, cold, row_map, ids, w, x, H, I)
        assert np.array_equal(out, out0), n


def test_misordered_flip_diverges():
    """Negative control: flipping the map without the copies must be caught."""
    E, n_cold, H, I, seed = 16, 4, 64, 32, 8
    row_map, ho, co = synth.random_map(E, n_cold, seed)
    hot, cold = _banks_for_map(E, row_map, ho, co, H, I, seed, 0)
    ids = np.array([[int(ho[0]), int(co[0])], [int(co[0]), int(ho[1])]], np.int32)
    w = np.array([[0.6, 0.4], [0.7, 0.3]], np.float32)
    x = synth.activations(2, H, seed)
    _, out0, _ = oracle.moe_layer(hot, cold, row_map, ids, w, x, H, I)
    e_h, e_c = int(ho[0]), int(co[0])
    row_map[e_h], row_map[e_c] = -1, 0        # map flip only
    _, out1, _ = oracle.moe_layer(hot, cold, row_map, ids, w, x, H, I)
    assert not np.array_equal(out0, out1)
    assert _expert_bytes_where_map_says(e_h, row_map, hot, cold) != _expected_expert_bytes(e_h, H, I, seed, 0)


def test_stale_swap_refused_and_nothing_changes():
    E, n_cold, H, I, seed = 16, 4, 64, 32, 2
    row_map, ho, co = synth.random_map(E, n_cold, seed)
    hot, cold = _banks_for_map(E, row_map, ho, co, H, I, seed, 0)
    before = [a.copy() for a in (hot.w13, hot.s13, cold.w13, cold.s2, row_map, ho, co)]
    with pytest.raises(oracle.SwapStale):
        oracle.swap_rows(hot, cold, 0, 0, int(ho[1]), int(co[0]), row_map, ho, co)
    after = [hot.w13, hot.s13, cold.w13, cold.s2, row_map, ho, co]
    assert all(np.array_equal(p, q) for p, q in zip(before, after))


def test_swap_round_trip_restores_banks():
    """Hundreds of random swaps, then each one undone in reverse order: both
    banks, the map and the owner mirrors come back byte-identical."""
    E, n_cold, H, I, seed = 32, 9, 64, 32, 4
    row_map, ho, co = synth.random_map(E, n_cold, seed)
    hot, cold = _banks_for_map(E, row_map, ho, co, H, I, seed, 0)
    snap = [a.copy() for a in (hot.w13, hot.s13, hot.w2, hot.s2, cold.w13, cold.s13, cold.w2,
                               cold.s2, row_map, ho, co)]
    rng = np.random.default_rng(9)
    log = []
    for _ in range(300):
        a, b = int(rng.integers(len(ho))), int(rng.integers(len(co)))
        log.append((a, b, int(ho[a]), int(co[b])))
        oracle.swap_rows(hot, cold, a, b, int(ho[a]), int(co[b]), row_map, ho, co)
        for e in (log[-1][2], log[-1][3]):
            assert _expert_bytes_where_map_says(e, row_map, hot, cold) == \
                _expected_expert_bytes(e, H, I, seed, 0)
    for a, b, was_hot, was_cold in reversed(log):
        oracle.swap_rows(hot, cold, a, b, was_cold, was_hot, row_map, ho, co)
    now = (hot.w13, hot.s13, hot.w2, hot.s2, cold.w13, cold.s13, cold.w2, cold.s2, row_map, ho, co)
    assert all(np.array_equal(p, q) for p, q in zip(snap, now))


# -------------------------------------------------------- split = unsplit --

@pytest.mark.parametrize("trial", range(4))
def test_oracle_split_equals_unsplit(trial):
    """The same experts, once split 12/4 over two banks and once all in one
    bank with the identity map, give bit-identical rows and outputs."""
    E, k, H, I, T = 16, 2, 256, 128, 8
    seed = 100 + trial
    row_map, ho, co = synth.random_map(E, 4, seed)
    hot, cold = _banks_for_map(E, row_map, ho, co, H, I, seed, 0)
    ids, w = synth.gaussian_routing(T, k, E, seed)
    x = synth.activations(T, H, seed)
    Ys, outs, _ = oracle.moe_layer(hot, cold, row_map, ids, w, x, H, I)
    all_map, all_owner, _ = synth.all_hot_map(E)
    allbank = oracle.Bank(**synth.make_bank_host(all_owner, seed, 0, H, I))
    Yu, outu, _ = oracle.moe_layer(allbank, None, all_map, ids, w, x, H, I)
    assert np.array_equal(Ys, Yu) and np.array_equal(outs, outu)


# ---------------------------------------------------------------- sizes --

def test_page_sizes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_sizes.json")))
    H, I, E, L, R_h, R_c = 4096, 2880, 384, 40, 295, 89
    b = synth.expert_bytes(H, I)
    assert b == 18_800_640
    assert round(b / 2**20, 2) == g["expert_mib"]["value"]
    assert abs(b / 2**20 - g["expert_mib_alt"]["value"]) <= g["expert_mib_alt"]["tolerance"]
    assert round(E * b / 2**30, 2) == g["layer_gib"]["value"]
    assert round(L * R_h * b / 2**30, 2) == g["hot_gib_40_layers"]["value"]
    assert round(L * R_c * b / 2**30, 2) == g["cold_gib_40_layers"]["value"]
    assert round(L * E * 4 / 1000) == g["counter_table_kb"]["value"]
    assert round(120 * b / 2**30, 1) == g["prefetch_bank_gib"]["value"]
    # weights alone would be 16.875 MiB: the printed 17.93 includes the scales
    assert synth.expert_sizes(H, I)["w13"] + synth.expert_sizes(H, I)["w2"] == int(16.875 * 2**20)


# ------------------------------------------------------ layer bookkeeping --

def test_layer_rows_are_per_pick_ffn_and_finalize():
    """The layer's indexing against the per-pick definition: Y[t, j] is the
    expert FFN of the bank row the map gives for topk_ids[t, j] on token t's
    activations, an invalid pick gives a zero row and is counted, and out is
    the finalize of those rows (pins the slot -> token, id -> bank row and
    bank -> tensor offsets of the layer loop)."""
    E, k, H, I, T, seed = 12, 3, 64, 32, 5, 21
    row_map, ho, co = synth.random_map(E, 5, seed)
    hot, cold = _banks_for_map(E, row_map, ho, co, H, I, seed, 0)
    ids, w = synth.gaussian_routing(T, k, E, seed)
    ids[2, 1] = E + 3                       # out of range: invalid
    x = synth.activations(T, H, seed)
    Y, out, bad = oracle.moe_layer(hot, cold, row_map, ids, w, x, H, I)
    assert bad == 1
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if not 0 <= e < E:
                assert not Y[t, j].any()
                continue
            m = int(row_map[e])
            b, r = (hot, m) if m >= 0 else (cold, -1 - m)
            ref = oracle.expert_ffn(b.w13[r], b.s13[r], b.w2[r], b.s2[r], x[t], H, I)["y_bf16"]
            assert np.array_equal(Y[t, j], ref), (t, j)
    assert np.array_equal(out, oracle.finalize(Y, w))
