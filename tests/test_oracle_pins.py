"""Pins of the CPU oracle against facts the pages fix, closed forms and brute force.

None of these tests re-types the oracle's formula: each compares it with a value
the pages print, a hand-derived closed form, an invariant of the method, or a
brute-force search over a tiny input.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def bf16(x):
    return oracle.f32_to_bf16(np.asarray(x, np.float32))


def f32(b):
    return oracle.bf16_to_f32(b)


# ------------------------------------------------------------ worked example --

def test_worked_example_4bit():
    g = _gold("worked_example_4bit.json")
    x = np.array(g["printed"]["x"], np.float32).reshape(4, 1)
    q, s, z = oracle.quant_sym(x, bits=4)
    assert q.ravel().tolist() == g["hand_computed"]["q"]
    # s = 1/7 rounded once to fp32
    assert s[0, 0] == np.float32(1.0) / np.float32(7.0)
    assert s.view(np.uint32)[0, 0] == 0x3E124925
    assert z.ravel().tolist() == [0]
    xh = oracle.dequant_pc(q, s, None).ravel()
    # x_hat = q / 7: the ends are recovered exactly, the middle within s/2
    assert xh[0] == -1.0 and xh[3] == 1.0
    assert np.all(np.abs(xh.astype(np.float64) - x.ravel()) <= float(s[0, 0]) / 2)
    assert abs(float(xh[1]) - (-1 / 7)) < 1e-7 and abs(float(xh[2]) - 2 / 7) < 1e-7


# --------------------------------------------------------- byte accounting ----

def test_group_size_table():
    for row in _gold("group_size_table.json")["rows"]:
        g = row["g"]
        N = g * 4096
        b = oracle.int4_bytes(N, g)
        assert Fraction(b, N) == Fraction(row["bytes_per_number"]).limit_denominator(1 << 20)
        ratio = 2 * N / b
        digits = len(row["ratio_printed"].split(".")[1])
        assert f"{ratio:.{digits}f}" == row["ratio_printed"]
    # the formula's ceilings on a ragged N
    assert oracle.int4_bytes(65, 64) == 33 + 2 * 4
    assert oracle.int4_bytes(1, 32) == 1 + 4


def test_exercise_1_and_lab_line():
    e = _gold("byte_budgets.json")["exercise_1"]
    tot = oracle.int4_bytes(e["N"], e["g"])
    assert tot == e["total_bytes"] == 576 * 1024
    ratio = 2 * e["N"] / tot
    assert f"metadata: {tot // 1024} KiB; ratio = {ratio:.3f}" == e["lab_printed"]
    assert Fraction(2 * e["N"], tot) == Fraction(32, 9)


def test_residual_example_299_5_MiB():
    r = _gold("byte_budgets.json")["residual_example"]
    L = r["layer"]
    sect, tot = oracle.int4_cache_sizes(1, L["T"], L["Hkv"], L["d"], L["g"], L["R"])
    assert f"{tot * r['layers'] / 2**20:.3f}" == r["lab_printed_MiB"]
    # item by item: codes 8064*8*64, K metadata ceil(8064/64)*8*128*4, V metadata 8064*8*2*4, residual
    assert sect[0] == sect[3] == 8064 * 8 * 64
    assert sect[1] + sect[2] == 126 * 8 * 128 * 4
    assert sect[4] + sect[5] == 8064 * 8 * 2 * 4
    assert sect[6] + sect[7] == 2 * 8 * 128 * 128 * 2
    assert tot == 9_814_016


def test_bytes_accounting():
    a = _gold("byte_budgets.json")["accounting"]
    GiB = 2**30
    assert oracle.kv_bytes(a["L"], a["T"], 2 * a["H"] * a["d"], 2) == a["bf16_GiB"] * GiB
    assert oracle.kv_bytes(a["L"], a["T"], 2 * a["H_gqa"] * a["d"], 2) == a["gqa_GiB"] * GiB
    # 4-bit payload of the GQA cache: the code sections of the per-layer INT4 cache, 32 layers
    sect, _ = oracle.int4_cache_sizes(1, a["T"], a["H_gqa"], a["d"], 64, 0)
    assert a["L"] * (sect[0] + sect[3]) == a["int4_payload_GiB"] * GiB


# ------------------------------------------------------- per-channel quant ----

def test_per_channel_round_half_even():
    # absmax 7 at bits=4 gives s = 1 exactly, so x/s are exact halves
    x = np.array([7, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5], np.float32).reshape(-1, 1)
    q, s, _ = oracle.quant_sym(x, bits=4)
    assert s[0, 0] == 1.0
    assert q.ravel().tolist() == [7, 0, 2, 2, 0, -2, -2, 4]


def test_asym_zero_point_added_after_rounding():
    # mn=-127, mx=128 -> range 255 -> s = 1; zp = round(-128 + 127) = -1 (odd), so
    # round(x/s) + zp and round(x/s + zp) differ at halves.
    x = np.array([-127, 128, 0.5, 2.5, -3.5], np.float32).reshape(-1, 1)
    q, s, z = oracle.quant_asym(x, -128, 127)
    assert s[0, 0] == 1.0 and z[0, 0] == -1
    assert q.ravel().tolist() == [-128, 127, 0 - 1, 2 - 1, -4 - 1]


def test_per_channel_closed_forms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 16)).astype(np.float32)
    x[:, 5] = 0.0                     # all-zero channel
    x[:, 6] = 0.75                    # constant positive channel
    x[:, 7] = np.abs(x[:, 7]) + 1.0   # all-positive channel
    q, s, z = oracle.quant_sym(x, bits=8)
    for c in range(16):
        col = x[:, c]
        if c == 5:
            assert s[0, c] == np.float32(1e-8) / np.float32(127)
            assert np.all(q[0, :, c] == 0)
            continue
        i = int(np.argmax(np.abs(col)))
        assert q[0, i, c] == (127 if col[i] > 0 else -127)
        assert np.all(np.abs(q[0, :, c]) <= 127)
    qa, sa, za = oracle.quant_asym(x, -128, 127)
    for c in range(16):
        col = x[:, c]
        if c in (5, 6, 7):
            continue
        assert qa[0, int(np.argmin(col)), c] == -128
        assert qa[0, int(np.argmax(col)), c] == 127
    # constant channel: range floored at 1e-8
    assert sa[0, 6] == np.float32(1e-8) / np.float32(255)
    # all-positive channel: round(qmin - min/s) is far below -128 and saturates, then
    # q = clip(round(x/s) - 128, -128, 127)
    assert za[0, 7] == -128
    for r in range(64):
        t = Fraction(float(x[r, 7])) / Fraction(float(sa[0, 7]))
        n = math.floor(t + Fraction(1, 2))
        assert qa[0, r, 7] == min(127, max(-128, n - 128))


def test_per_channel_nearest_integer():
    """Each code is the integer nearest to x/s (exact rational arithmetic), clipped."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 6)).astype(np.float32)
    for bits in (2, 4, 8):
        q, s, _ = oracle.quant_sym(x, bits)
        qmax = (1 << (bits - 1)) - 1
        for r in range(40):
            for c in range(6):
                t = Fraction(float(x[r, c])) / Fraction(float(s[0, c]))
                n = int(q[0, r, c])
                if abs(n) < qmax:
                    assert abs(t - n) <= Fraction(1, 2) + Fraction(1, 1 << 20)


def test_per_channel_axes_and_batches():
    """Channels are columns; slices are independent: a column scaled by 2 gets a doubled scale."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 32, 8)).astype(np.float32)
    x2 = x.copy()
    x2[1, :, 3] *= 2
    q, s, _ = oracle.quant_sym(x, 8)
    q2, s2, _ = oracle.quant_sym(x2, 8)
    assert s2[1, 3] == np.float32(2) * s[1, 3]
    assert np.array_equal(q2, q)
    mask = np.ones_like(s, bool)
    mask[1, 3] = False
    assert np.array_equal(s2[mask], s[mask])


def test_dequant_closed_form():
    q = np.array([-7, -1, 2, 7], np.int8).reshape(1, 4, 1)
    s = np.array([[0.5]], np.float32)
    z = np.array([[3]], np.int8)
    assert oracle.dequant_pc(q, s, z).ravel().tolist() == [-5.0, -2.0, -0.5, 2.0]
    assert oracle.dequant_pc(q, s, None).ravel().tolist() == [-3.5, -0.5, 1.0, 3.5]


def test_per_channel_round_trip_bound():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((256, 128)).astype(np.float32)
    for fn in ("sym", "asym"):
        if fn == "sym":
            q, s, z = oracle.quant_sym(x, 8)
        else:
            q, s, z = oracle.quant_asym(x, -128, 127)
        xh = oracle.dequant_pc(q, s, z)[0]
        err = np.abs(x.astype(np.float64) - xh)
        # half a step, plus the fp32 rounding of x/s and of the product
        assert np.all(err <= s.astype(np.float64) * (0.5 + 1e-5))


def test_err_stats_closed_form():
    x = np.array([3, 0, 1], np.float32)
    xh = np.array([0, 4, 1], np.float32)
    raw = oracle.err_stats(x, xh)
    assert raw == (25.0, 7.0, 4.0)
    rmse, mx, mean = oracle.stats_finalize(raw, 3)
    assert rmse == math.sqrt(25 / 3) and mx == 4.0 and mean == 7 / 3
    # bf16 operands are widened exactly
    raw_b = oracle.err_stats(bf16(x), bf16(xh))
    assert raw_b == raw


def test_compression_ratio_config_1():
    # fp32 [256][128]: data 32768 B int8, scale 128 fp32, zero point 128 int8
    r = oracle.compression_ratio(256 * 128 * 4, 256 * 128, 128 * 4, 128)
    assert r == 131072 / 33408
    assert f"{r:.6f}" == "3.923372"


# ------------------------------------------------------------- INT4 groups ----

def _level_cache(B, T, H, d, g, R, seed):
    """K, V whose every group is made of exactly the 16 levels (k - z0) * s0, with s0 a
    power of two and z0 an integer in [0, 15], so scale, zero, codes and x_hat are known
    in closed form.  K groups run over tokens per channel, V groups over channels per token."""
    rng = np.random.default_rng(seed)
    Tq = T - R
    K = np.zeros((B, T, H, d), np.float32)
    V = np.zeros((B, T, H, d), np.float32)
    kcode = np.zeros((B, T, H, d), np.int64)
    vcode = np.zeros((B, T, H, d), np.int64)
    ks = np.zeros((B, H, -(-Tq // g), d))
    kz = np.zeros_like(ks)
    vs = np.zeros((B, H, Tq, d // g))
    vz = np.zeros_like(vs)
    for b in range(B):
        for h in range(H):
            for j in range(-(-Tq // g)):
                t0, n = j * g, min(g, Tq - j * g)
                for c in range(d):
                    s0 = 2.0 ** int(rng.integers(-6, 3))
                    z0 = int(rng.integers(0, 16))
                    codes = rng.integers(0, 16, n)
                    if n >= 2:
                        codes[rng.choice(n, 2, replace=False)] = [0, 15]
                    else:  # a one-token group: value 0 gives code 0 and zero 0
                        codes[0], z0 = 0, 0
                    kcode[b, t0:t0 + n, h, c] = codes
                    K[b, t0:t0 + n, h, c] = (codes - z0) * s0
                    ks[b, h, j, c] = s0 if n >= 2 else np.nan
                    kz[b, h, j, c] = z0
            for t in range(Tq):
                for k in range(d // g):
                    s0 = 2.0 ** int(rng.integers(-6, 3))
                    z0 = int(rng.integers(0, 16))
                    codes = rng.integers(0, 16, g)
                    codes[rng.choice(g, 2, replace=False)] = [0, 15]
                    vcode[b, t, h, k * g:(k + 1) * g] = codes
                    V[b, t, h, k * g:(k + 1) * g] = (codes - z0) * s0
                    vs[b, h, t, k] = s0
                    vz[b, h, t, k] = z0
    K[:, Tq:] = rng.standard_normal((B, R, H, d))
    V[:, Tq:] = rng.standard_normal((B, R, H, d))
    return bf16(K), bf16(V), kcode, vcode, ks, kz, vs, vz


@pytest.mark.parametrize("T,R,g", [(64 * 3 + 17, 16, 64), (96, 0, 32), (128 + 5, 5, 128)])
def test_int4_exact_levels(T, R, g):
    B, H, d = 2, 3, 128 if g == 128 else 64
    Kb, Vb, kcode, vcode, ks, kz, vs, vz = _level_cache(B, T, H, d, g, R, seed=T + g)
    c = oracle.int4_quant(Kb, Vb, g, R)
    Tq = T - R
    full = ~np.isnan(ks)
    assert np.array_equal(f32(c["k_scale"])[full], ks[full].astype(np.float32))
    assert np.array_equal(f32(c["k_zero"])[full], kz[full].astype(np.float32))
    assert np.array_equal(f32(c["v_scale"]), vs.astype(np.float32))
    assert np.array_equal(f32(c["v_zero"]), vz.astype(np.float32))
    # packed bytes: low nibble = even channel, high nibble = odd channel; [B][H][Tq][d/2]
    kc = kcode[:, :Tq].transpose(0, 2, 1, 3)
    vc = vcode[:, :Tq].transpose(0, 2, 1, 3)
    assert np.array_equal(c["k_codes"], (kc[..., 0::2] | (kc[..., 1::2] << 4)).astype(np.uint8))
    assert np.array_equal(c["v_codes"], (vc[..., 0::2] | (vc[..., 1::2] << 4)).astype(np.uint8))
    # dequantization reproduces the levels exactly, and the residual verbatim
    assert np.array_equal(oracle.int4_dequant(c, "k"), f32(Kb))
    assert np.array_equal(oracle.int4_dequant(c, "v"), f32(Vb))
    assert np.array_equal(c["k_res"], Kb[:, Tq:].transpose(0, 2, 1, 3))
    assert np.array_equal(c["v_res"], Vb[:, Tq:].transpose(0, 2, 1, 3))


def _c2_like(B, T, H, d, seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, T, H, d)).astype(np.float32)
    K[..., rng.choice(d, 4, replace=False)] *= 10
    V = rng.standard_normal((B, T, H, d)).astype(np.float32)
    return bf16(K), bf16(V)


def _levels_and_ids(c, side):
    """Per element of the quantized region: (code, scale, zero) as fp64, [B][Tq][H][d]."""
    B, T, H, d, g, R = (c[k] for k in ("B", "T", "H", "d", "g", "R"))
    Tq = T - R
    codes = c[side + "_codes"]
    q = np.stack([codes & 15, codes >> 4], -1).reshape(B, H, Tq, d).transpose(0, 2, 1, 3)
    s = f32(c[side + "_scale"]).astype(np.float64)
    z = f32(c[side + "_zero"]).astype(np.float64)
    if side == "k":
        s = np.repeat(s, g, axis=2)[:, :, :Tq].transpose(0, 2, 1, 3)
        z = np.repeat(z, g, axis=2)[:, :, :Tq].transpose(0, 2, 1, 3)
    else:
        s = np.repeat(s, g, axis=3).transpose(0, 2, 1, 3)
        z = np.repeat(z, g, axis=3).transpose(0, 2, 1, 3)
    return q.astype(np.int64), s, z


@pytest.mark.parametrize("g", [32, 64, 128])
def test_int4_round_trip_bound_and_nearest_level(g):
    B, T, H, d, R = 1, 300, 2, 128, 44
    Kb, Vb = _c2_like(B, T, H, d, seed=g)
    c = oracle.int4_quant(Kb, Vb, g, R)
    Tq = T - R
    for side, X in (("k", Kb), ("v", Vb)):
        x = f32(X)[:, :Tq].astype(np.float64)
        xh = oracle.int4_dequant(c, side)[:, :Tq].astype(np.float64)
        q, s, z = _levels_and_ids(c, side)
        # round trip: every element within half a (stored, bf16) step
        assert np.all(np.abs(x - xh) <= s / 2)
        # brute force: the code is the nearest of the 16 levels (k - z) * s; exact ties go
        # to the even (k - z); the levels are exact in fp64
        levels = (np.arange(16)[None, None, None, None, :] - z[..., None]) * s[..., None]
        dist = np.abs(x[..., None] - levels)
        best = dist.min(-1, keepdims=True)
        cand = dist == best
        even = ((np.arange(16)[None, None, None, None, :] - z[..., None]) % 2) == 0
        pick = np.where(cand.sum(-1) > 1, np.argmax(cand & even, -1), np.argmax(cand, -1))
        assert np.array_equal(pick, q)
        # the K outlier channels get their own (larger) per-channel scales
        if side == "k":
            ksc = f32(c["k_scale"])
            big = np.argsort(ksc.mean(axis=(0, 1, 2)))[-4:]
            assert ksc[..., big].min() > 3 * np.median(ksc)


def test_int4_special_groups():
    B, T, H, d, g = 1, 64, 1, 64, 64
    K = np.zeros((B, T, H, d), np.float32)
    V = np.zeros((B, T, H, d), np.float32)
    K[..., 1] = 3.0                       # constant channel
    K[0, :, 0, 2] = np.linspace(1, 2, T)  # all-positive channel
    c = oracle.int4_quant(bf16(K), bf16(V), g, 0)
    s0 = f32(c["k_scale"])[0, 0, 0]
    z0 = f32(c["k_zero"])[0, 0, 0]
    # all-zero channel: range floored at 1e-8, scale = smallest bf16 >= 1e-8/15, code 0, x_hat 0
    want = np.float32(np.float32(1e-8) / np.float32(15))
    assert s0[0] >= want and s0[0] < want * (1 + 2.0**-7)
    assert z0[0] == 0 and np.all((c["k_codes"][0, 0, :, 0] & 15) == 0)
    assert np.all(oracle.int4_dequant(c, "k")[..., 0] == 0)
    # all-positive group: z negative, every value still within half a step
    xh = oracle.int4_dequant(c, "k")[0, :, 0, 2].astype(np.float64)
    x = f32(bf16(K))[0, :, 0, 2].astype(np.float64)
    assert z0[2] < 0
    assert np.all(np.abs(x - xh) <= float(s0[2]) / 2)
    # V rows of zeros
    assert np.all(oracle.int4_dequant(c, "v") == 0)


# ---------------------------------------------------------- decode attention --

def _all_residual_cache(K, V, g=64):
    """A cache holding every token in the bf16 residual (Tq = 0): x_hat is the input."""
    return oracle.int4_quant(K, V, g, K.shape[1])


def test_attn_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    K = bf16(rng.standard_normal((2, 1, 2, 64)))
    V = bf16(rng.standard_normal((2, 1, 2, 64)))
    q = bf16(rng.standard_normal((2, 4, 64)))
    c = _all_residual_cache(K, V)
    o = oracle.decode_attn(c, q, 0.125)
    for b in range(2):
        for hq in range(4):
            assert np.array_equal(o[b, hq], f32(V)[b, 0, hq // 2].astype(np.float64))


def test_attn_zero_query_is_mean_of_values():
    Kb, Vb = _c2_like(1, 192, 2, 64, seed=4)
    c = oracle.int4_quant(Kb, Vb, 64, 64)
    q = np.zeros((1, 2, 64), np.uint16)
    o = oracle.decode_attn(c, q)
    vh = oracle.int4_dequant(c, "v").astype(np.float64)
    for hq in range(2):
        assert np.allclose(o[0, hq], vh[0, :, hq].mean(0), rtol=0, atol=1e-12)


def test_attn_two_tokens_closed_form():
    # q = e_0, k_0 = 0, k_1[0] = ln 3 (as bf16): weights 1/(1+e^a), e^a/(1+e^a)
    d = 64
    K = np.zeros((1, 2, 1, d), np.float32)
    K[0, 1, 0, 0] = math.log(3.0)
    V = np.zeros((1, 2, 1, d), np.float32)
    V[0, 0, 0, :] = 1.0
    V[0, 1, 0, :] = -2.0
    Kb, Vb = bf16(K), bf16(V)
    a = float(f32(Kb)[0, 1, 0, 0])
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    o = oracle.decode_attn(_all_residual_cache(Kb, Vb), bf16(q))
    w1 = math.exp(a) / (1 + math.exp(a))
    assert np.allclose(o[0, 0], (1 - w1) * 1.0 + w1 * -2.0, rtol=0, atol=1e-14)
    # the softmax scale multiplies the logits: weights exp(0.5 a) / (1 + exp(0.5 a))
    o = oracle.decode_attn(_all_residual_cache(Kb, Vb), bf16(q), 0.5)
    w1 = math.exp(0.5 * a) / (1 + math.exp(0.5 * a))
    assert np.allclose(o[0, 0], (1 - w1) * 1.0 + w1 * -2.0, rtol=0, atol=1e-14)


def test_attn_gqa_head_map():
    # V of KV head h is the constant h + 1; query head hq must read KV head hq // (Hq/Hkv)
    rng = np.random.default_rng(2)
    B, T, Hkv, Hq, d = 2, 80, 3, 12, 64
    K = bf16(rng.standard_normal((B, T, Hkv, d)))
    V = np.zeros((B, T, Hkv, d), np.float32)
    for h in range(Hkv):
        V[:, :, h, :] = h + 1
    # all tokens in the bf16 residual
    c = oracle.int4_quant(K, bf16(V), 64, T)
    q = bf16(rng.standard_normal((B, Hq, d)))
    o = oracle.decode_attn(c, q)
    for hq in range(Hq):
        assert np.allclose(o[:, hq], hq // (Hq // Hkv) + 1, rtol=0, atol=1e-12)
    # the same map with INT4 tokens in front of the residual: a constant V group is held
    # exactly (test_int4_constant_group_is_exact), so every row is still its head's constant
    c2 = oracle.int4_quant(K, bf16(V), 64, 16)
    vh = oracle.int4_dequant(c2, "v")
    o2 = oracle.decode_attn(c2, q)
    for hq in range(Hq):
        h = hq // (Hq // Hkv)
        assert np.all(vh[:, :, h] == h + 1)
        assert np.allclose(o2[:, hq], h + 1, rtol=0, atol=1e-12)


def test_int4_constant_group_is_exact():
    # A constant nonzero group has range 0 (floored at 1e-8), so the scale comes from the
    # zero-point floor |min| / 256: s = 2^-8 for x = 1, z = round(-1 / 2^-8) = -256, held
    # exactly by bf16, and x_hat = (0 + 256) * 2^-8 = 1 exactly.
    K = np.full((1, 64, 1, 64), 1.0, np.float32)
    c = oracle.int4_quant(bf16(K), bf16(K), 64, 0)
    assert np.all(f32(c["k_scale"]) == 2.0**-8) and np.all(f32(c["k_zero"]) == -256)
    assert np.all(f32(c["v_scale"]) == 2.0**-8) and np.all(f32(c["v_zero"]) == -256)
    assert np.all(oracle.int4_dequant(c, "k") == 1.0)
    assert np.all(oracle.int4_dequant(c, "v") == 1.0)


@pytest.mark.parametrize("offset", [100.0, -100.0, 3.0e4, -7.5, 0.37])
def test_int4_offset_groups_keep_the_round_trip_bound(offset):
    # Groups far from zero relative to their range (offset +- 0.25 N(0,1)): the stored zero
    # point is an integer of magnitude <= 256 (exact in bf16), every element stays within
    # half a stored step of its value, and its code is the nearest of the 16 levels.
    B, T, H, d, g, R = 1, 256, 2, 128, 64, 0
    rng = np.random.default_rng(int(abs(offset) * 10))
    K = (offset + 0.25 * rng.standard_normal((B, T, H, d))).astype(np.float32)
    V = (offset + 0.25 * rng.standard_normal((B, T, H, d))).astype(np.float32)
    Kb, Vb = bf16(K), bf16(V)
    c = oracle.int4_quant(Kb, Vb, g, R)
    for side, X in (("k", Kb), ("v", Vb)):
        z = f32(c[side + "_zero"]).astype(np.float64)
        assert np.all(np.abs(z) <= 256) and np.all(z == np.round(z))
        x = f32(X).astype(np.float64)
        xh = oracle.int4_dequant(c, side).astype(np.float64)
        q, s, zz = _levels_and_ids(c, side)
        assert np.all(np.abs(x - xh) <= s / 2)
        levels = (np.arange(16)[None, None, None, None, :] - zz[..., None]) * s[..., None]
        dist = np.abs(x[..., None] - levels)
        assert np.all(np.take_along_axis(dist, q[..., None], -1)[..., 0] == dist.min(-1))
    # a group that straddles zero keeps the plain scale rule: s = smallest bf16 >= range / 15
    Kz = np.zeros((1, 64, 1, 64), np.float32)
    Kz[0, :, 0, 0] = np.linspace(-1.0, 2.0, 64)
    cz = oracle.int4_quant(bf16(Kz), bf16(Kz), 64, 0)
    r15 = np.float32(np.float32(3.0) / np.float32(15.0))
    s0 = f32(cz["k_scale"])[0, 0, 0, 0]
    assert s0 >= r15 and s0 == f32(bf16([s0]))[0] and np.float32(s0 - r15) < r15 * 2.0**-7


def _bf16_sign_bit(b):
    return (np.asarray(b, np.uint16) >> 15) & 1


def test_int4_zero_point_sign_bits():
    # The stored zero point is the IEEE result of round(0 - min / s) (Walkthrough §1.2 with
    # qmin = 0), evaluated here by numpy in float32: min = +0 or -0 gives 0 - (+-0) = +0
    # (bits 0x0000); a minimum in (0, s/2] gives a negative quotient that rounds to -0
    # (bits 0x8000).
    d, g = 64, 64
    K = np.zeros((1, 64, 1, d), np.float32)
    V = np.zeros((1, 64, 1, d), np.float32)
    K[0, :, 0, 1] = -0.0                               # channel of -0 values
    K[0, :, 0, 2] = np.linspace(0.01, 1.0, 64)         # min in (0, s/2]
    K[0, :, 0, 3] = np.linspace(0.0, 1.0, 64)          # min = +0
    K[0, :, 0, 4] = np.linspace(-1.0, 0.0, 64)         # max = 0, min < 0
    V[0, 0, 0, :] = -0.0
    V[0, 1, 0, :] = np.linspace(0.01, 1.0, d)
    V[0, 2, 0, :] = np.linspace(0.0, 1.0, d)
    Kb, Vb = bf16(K), bf16(V)
    c = oracle.int4_quant(Kb, Vb, g, 0)
    for side, X, zb, sb in (("k", Kb, c["k_zero"][0, 0, 0, :5], c["k_scale"][0, 0, 0, :5]),
                            ("v", Vb, c["v_zero"][0, 0, :3, 0], c["v_scale"][0, 0, :3, 0])):
        x = f32(X)[0, :, 0, :]
        mins = x.min(axis=0)[:5] if side == "k" else x.min(axis=1)[:3]
        s = f32(sb)
        with np.errstate(all="ignore"):
            want = np.round(np.float32(0.0) - mins.astype(np.float32) / s)
        assert np.array_equal(f32(zb), want)
        assert np.array_equal(_bf16_sign_bit(zb), np.signbit(want).astype(np.uint16))
    assert c["k_zero"][0, 0, 0, 0] == 0x0000 and c["k_zero"][0, 0, 0, 1] == 0x0000
    assert c["k_zero"][0, 0, 0, 2] == 0x8000 and c["k_zero"][0, 0, 0, 3] == 0x0000
    assert c["v_zero"][0, 0, 0, 0] == 0x0000 and c["v_zero"][0, 0, 1, 0] == 0x8000
    assert c["v_zero"][0, 0, 2, 0] == 0x0000
    # per-channel asymmetric INT8: a channel whose minimum is +-0 has zero point qmin exactly
    xa = np.stack([np.linspace(0.0, 1.0, 16), -np.abs(np.linspace(-0.0, 0.0, 16)),
                   np.linspace(-0.0, 2.0, 16)], 1).astype(np.float32)
    qa, sa, za = oracle.quant_asym(xa, -128, 127)
    assert za.reshape(-1).tolist() == [-128, -128, -128]


def test_attn_dominant_logit_picks_its_value():
    rng = np.random.default_rng(6)
    d, T = 64, 40
    K = rng.standard_normal((1, T, 1, d)).astype(np.float32) * 0.01
    K[0, 17, 0, :] = 1.0
    V = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    q = np.full((1, 1, d), 1.0, np.float32)
    Kb, Vb = bf16(K), bf16(V)
    o = oracle.decode_attn(_all_residual_cache(Kb, Vb), bf16(q))
    assert np.allclose(o[0, 0], f32(Vb)[0, 17, 0], rtol=0, atol=1e-12)


def test_attn_rows_match_full():
    Kb, Vb = _c2_like(2, 130, 2, 64, seed=8)
    c = oracle.int4_quant(Kb, Vb, 64, 2)
    q = bf16(np.random.default_rng(8).standard_normal((2, 4, 64)))
    full = oracle.decode_attn(c, q, 0.5)
    rows = [(1, 3), (0, 0), (1, 1)]
    part = oracle.decode_attn(c, q, 0.5, rows=rows)
    for i, (b, hq) in enumerate(rows):
        assert np.array_equal(part[i], full[b, hq])


def test_attn_error_propagation_bounds():
    """Explainer, 'K error changes the weights, V error changes the content': with the
    weights fixed (K exact) the output moves by at most max_i ||dv_i||; a K error moves
    logit i by at most ||q|| ||dk_i|| (scale folded into q)."""
    rng = np.random.default_rng(12)
    B, T, H, d, g = 1, 256, 1, 64, 32
    Kl, _, _, _, _, _, _, _ = _level_cache(B, T, H, d, g, 0, seed=99)   # K exact under INT4
    _, Vb = _c2_like(B, T, H, d, seed=12)
    q = bf16(rng.standard_normal((B, 1, d)) / 8)
    exact = oracle.int4_quant(Kl, Vb, g, T)              # every token bf16
    quant = oracle.int4_quant(Kl, Vb, g, 0)              # every token INT4
    assert np.array_equal(oracle.int4_dequant(quant, "k"), f32(Kl))
    vx = f32(Vb).astype(np.float64)[0, :, 0]
    vh = oracle.int4_dequant(quant, "v").astype(np.float64)[0, :, 0]
    o_ref = oracle.decode_attn(exact, q)[0, 0]
    o_v = oracle.decode_attn(quant, q)[0, 0]
    dv = np.linalg.norm(vh - vx, axis=1).max()
    assert 0 < np.linalg.norm(o_v - o_ref) <= dv
    # K error on random K: Cauchy-Schwarz bound on each logit
    Kb, _ = _c2_like(B, T, H, d, seed=13)
    qk = oracle.int4_quant(Kb, Vb, g, 0)
    kx = f32(Kb).astype(np.float64)[0, :, 0]
    kh = oracle.int4_dequant(qk, "k").astype(np.float64)[0, :, 0]
    qv = f32(q)[0, 0].astype(np.float64)
    dlog = np.abs((kh - kx) @ qv)
    assert np.all(dlog <= np.linalg.norm(qv) * np.linalg.norm(kh - kx, axis=1) + 1e-12)


# ------------------------------------------------------------ selection -------

def test_colsum_is_sequential_fp32():
    # sequential fp32: (0 + 1e8) + 1 rounds back to 1e8, then - 1e8 gives 0
    hist = np.array([[[1e8], [1.0], [-1e8]]], np.float32)
    assert oracle.colsum(hist)[0, 0] == 0.0
    # in step order 1 + 1e8 rounds to 1e8, then - 1e8 gives 0 (the reverse order gives 1)
    hist = np.array([[[1.0], [1e8], [-1e8]]], np.float32)
    assert oracle.colsum(hist)[0, 0] == 0.0
    # exactly representable terms: exact sum
    h = (np.arange(5 * 7, dtype=np.float32).reshape(1, 5, 7) / 8.0)
    assert np.array_equal(oracle.colsum(h)[0], h[0].astype(np.float64).sum(0).astype(np.float32))


def test_keep_count_closed_form():
    for T in (1, 5, 100, 300):
        for B in (0, 3, 64, 200, 400):
            for W in (0, 1, 10, 256, 1000):
                sc = np.random.default_rng(T + B + W).random((1, T)).astype(np.float32)
                keep = oracle.select(sc, B, W)
                assert keep.shape[1] == min(T, max(B, min(W, T)))


def _rank_count_heavy(masked, k):
    n = len(masked)
    out = set()
    for i in range(n):
        better = sum(1 for j in range(n) if masked[j] > masked[i] or (masked[j] == masked[i] and j < i))
        if better < k:
            out.add(i)
    return out


def test_select_bruteforce_small():
    rng = np.random.default_rng(21)
    for trial in range(400):
        T = int(rng.integers(1, 13))
        B = int(rng.integers(0, 15))
        W = int(rng.integers(0, 6))
        sc = (rng.integers(0, 4, T) / 4.0).astype(np.float32)   # many ties
        keep = oracle.select(sc[None], B, W)[0].tolist()
        rs = max(0, T - W)
        masked = [float(sc[j]) if j < rs else -math.inf for j in range(T)]
        heavy = _rank_count_heavy(masked, min(max(0, B - (T - rs)), T))
        want = sorted(set(range(rs, T)) | heavy)
        assert keep == want, (T, B, W, sc.tolist())


def _special_better(a, b):
    """True when score a ranks strictly above score b: IEEE order for numbers (-0 == +0),
    every number above NaN, NaNs equal to one another."""
    na, nb = math.isnan(a), math.isnan(b)
    if na or nb:
        return nb and not na
    return a > b


def _special_equal(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b


def test_select_bruteforce_special_values():
    # Scores that include NaN, +0, -0, +inf and -inf: a token is heavy when fewer than k
    # tokens rank above it (larger score, or an equal score at a lower index), with the
    # recent window's scores replaced by -inf before the TopK (Walkthrough §3.2) and the
    # window ranked below every earlier token, so that the union always holds
    # min(T, max(budget, |recent|)) tokens.
    vals = [math.nan, 0.0, -0.0, math.inf, -math.inf, 0.5, -0.5]
    rng = np.random.default_rng(33)
    seen_nan_kept = seen_zero_tie = False
    for trial in range(600):
        T = int(rng.integers(1, 13))
        B = int(rng.integers(0, 15))
        W = int(rng.integers(0, 6))
        sc = np.array([vals[i] for i in rng.integers(0, len(vals), T)], np.float32)
        keep = oracle.select(sc[None], B, W)[0].tolist()
        rs = max(0, T - W)
        masked = [float(sc[j]) if j < rs else -math.inf for j in range(T)]
        k = min(max(0, B - (T - rs)), T)
        heavy = set()
        def above_of(j, i):
            if (j >= rs) != (i >= rs):
                return i >= rs
            return _special_better(masked[j], masked[i]) or (_special_equal(masked[j], masked[i]) and j < i)

        for i in range(T):
            above = sum(1 for j in range(T) if above_of(j, i))
            if above < k:
                heavy.add(i)
        want = sorted(set(range(rs, T)) | heavy)
        assert keep == want, (T, B, W, sc.tolist())
        assert len(keep) == min(T, max(B, min(W, T)))
        seen_nan_kept |= any(math.isnan(masked[i]) for i in heavy)
        seen_zero_tie |= any(masked[i] == 0.0 and math.copysign(1, masked[i]) < 0 for i in heavy)
    assert seen_nan_kept and seen_zero_tie
    # -0 and +0 tie, so the lower index wins whatever the sign; NaN ranks below -inf
    sc = np.array([[0.0, -0.0, -0.0, 0.0, np.nan, -np.inf]], np.float32)
    assert oracle.select(sc, 2, 0)[0].tolist() == [0, 1]
    sc = np.array([[-0.0, 0.0, np.nan, -np.inf]], np.float32)
    assert oracle.select(sc, 3, 0)[0].tolist() == [0, 1, 3]
    # a NaN before the window still outranks the window's masked tokens
    sc = np.array([[np.nan, np.nan, 1.0, 2.0]], np.float32)
    assert oracle.select(sc, 3, 2)[0].tolist() == [0, 2, 3]


def test_select_ties_take_lower_index():
    sc = np.full((1, 20), 0.5, np.float32)
    assert oracle.select(sc, 8, 3)[0].tolist() == [0, 1, 2, 3, 4, 17, 18, 19]


def test_select_invariants_and_snapkv_equals_h2o():
    rng = np.random.default_rng(4)
    hist = rng.random((3, 8, 500)).astype(np.float32)
    keep, scores = oracle.h2o_select(hist, 96, 32)
    assert np.array_equal(oracle.select(oracle.colsum(hist), 96, 32), keep)
    for r in range(3):
        k = keep[r]
        assert np.all(np.diff(k) > 0)
        assert set(range(500 - 32, 500)) <= set(k.tolist())
        kept = [j for j in k if j < 468]
        dropped = sorted(set(range(468)) - set(kept))
        assert min(scores[r, kept]) >= max(scores[r, dropped])


def test_token_ratio_and_total_gain():
    assert oracle.token_ratio(32768, 2048) == 16.0
    for T, K in ((0, 1), (10, 0), (10, 11), (-1, -1)):
        with pytest.raises(ValueError):
            oracle.token_ratio(T, K)
    assert oracle.total_gain(2.0, 0.5625, 32768, 2048) == (2.0 / 0.5625) * 16.0


def test_compact_gathers_labelled_rows():
    B, T, H, d, K = 2, 50, 3, 8, 7
    src = np.zeros((B, T, H, d), np.uint16)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                src[b, t, h, :] = b * 10000 + t * 10 + h
    rng = np.random.default_rng(0)
    keep = np.sort(np.stack([[rng.choice(T, K, replace=False) for _ in range(H)] for _ in range(B)]), -1).astype(np.int32)
    dst = oracle.compact(src, keep)
    for b in range(B):
        for k in range(K):
            for h in range(H):
                assert np.all(dst[b, k, h] == b * 10000 + keep[b, h, k] * 10 + h)


def test_bf16_helpers():
    # nearest-even on a tie: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1 (even)
    assert oracle.f32_to_bf16(np.float32(1 + 2.0**-8)).item() == 0x3F80
    assert oracle.f32_to_bf16(np.float32(1 + 3 * 2.0**-8)).item() == 0x3F82
    assert oracle.f32_to_bf16(np.float32(-1.5)).item() == 0xBFC0
    assert float(oracle.bf16_to_f32(np.array([0x4049], np.uint16))[0]) == 3.140625


# ------------------------------------------------ eviction on the 4-bit cache --

def _gather_tokens(X, keep):
    """X [B][T][H][d], keep [B][H][K] -> [B][K][H][d] (plain fancy indexing)."""
    B, T, H, d = X.shape
    out = np.empty((B, keep.shape[-1], H, d), X.dtype)
    for b in range(B):
        for h in range(H):
            out[b, :, h] = X[b, keep[b, h], h]
    return out


def _assert_same_cache(a, b):
    for k in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_res", "v_res"):
        assert a[k].shape == b[k].shape, k
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("T,R,g", [(300, 44, 64), (256, 0, 32), (128 * 3 + 5, 5, 128)])
def test_evict_keep_all_is_identity(T, R, g):
    B, H, d = 2, 2, 128
    Kb, Vb = _c2_like(B, T, H, d, seed=T)
    c = oracle.int4_quant(Kb, Vb, g, R)
    keep = np.broadcast_to(np.arange(T, dtype=np.int32), (B, H, T)).copy()
    _assert_same_cache(oracle.int4_evict(c, keep, R), c)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_evict_whole_groups_equals_quantizing_the_kept_tokens(g):
    # Eviction that keeps whole K groups (any of them, a different set per head) and the
    # residual: every group is a function of its own values only, so the result must be
    # the quantization of the gathered input.
    B, H, d = 2, 3, 128
    ng, R = 6, 40
    T = ng * g + 17 + R            # a partial last K group of 17 tokens
    Kb, Vb = _c2_like(B, T, H, d, seed=g + 1)
    c = oracle.int4_quant(Kb, Vb, g, R)
    rng = np.random.default_rng(g)
    keep = np.empty((B, H, 3 * g + 17 + R), np.int32)
    for b in range(B):
        for h in range(H):
            groups = np.sort(rng.choice(ng, 3, replace=False))
            toks = [np.arange(j * g, (j + 1) * g) for j in groups]
            toks.append(np.arange(ng * g, T))          # the partial group and the residual
            keep[b, h] = np.concatenate(toks)
    got = oracle.int4_evict(c, keep, R)
    want = oracle.int4_quant(_gather_tokens(Kb, keep), _gather_tokens(Vb, keep), g, R)
    _assert_same_cache(got, want)


@pytest.mark.parametrize("g,R2", [(64, 0), (64, 37), (32, 5), (128, 0)])
def test_evict_from_the_bf16_window_equals_the_quantizer(g, R2):
    # A cache held entirely in the bf16 residual: the kept tokens' values are their bf16
    # inputs, so every new group (K across tokens, V across channels) and the new residual
    # must be exactly what the quantizer makes of the gathered tokens.
    B, H, d, T = 1, 2, 128, 400
    Kb, Vb = _c2_like(B, T, H, d, seed=g + R2)
    c = oracle.int4_quant(Kb, Vb, g, T)
    rng = np.random.default_rng(R2)
    K = 3 * g + 11 + R2
    keep = np.sort(np.stack([[rng.choice(T, K, replace=False) for _ in range(H)] for _ in range(B)]), -1)
    keep = keep.astype(np.int32)
    got = oracle.int4_evict(c, keep, R2)
    want = oracle.int4_quant(_gather_tokens(Kb, keep), _gather_tokens(Vb, keep), g, R2)
    _assert_same_cache(got, want)


def _check_evicted(c, keep, R2, e):
    """Properties every eviction result has, whatever the kept set."""
    B, T, H, d, g, R = (c[k] for k in ("B", "T", "H", "d", "g", "R"))
    K = keep.shape[-1]
    Tq, Tq2 = T - R, K - R2
    gk = _gather_tokens(oracle.int4_dequant(c, "k"), keep)
    gv = _gather_tokens(oracle.int4_dequant(c, "v"), keep)
    # V: kept quantized rows come back exactly
    ev = oracle.int4_dequant(e, "v")
    from_q = (keep < Tq).transpose(0, 2, 1)[:, :Tq2]               # [B][Tq2][H]
    assert np.array_equal(ev[:, :Tq2][from_q], gv[:, :Tq2][from_q])
    # K: every new group keeps each value within half of its (new) step, on the nearest level
    ek = oracle.int4_dequant(e, "k")[:, :Tq2].astype(np.float64)
    x = gk[:, :Tq2].astype(np.float64)
    q, s, z = _levels_and_ids(e, "k")
    assert np.all(np.abs(x - ek) <= s / 2)
    levels = (np.arange(16)[None, None, None, None, :] - z[..., None]) * s[..., None]
    dist = np.abs(x[..., None] - levels)
    assert np.all(np.take_along_axis(dist, q[..., None], -1)[..., 0] == dist.min(-1))
    # a requantized group's scale is the smallest bf16 at or above (max - min) / 15 of its
    # values; a group copied whole is one whose tokens are exactly an old aligned group
    n_copied = 0
    for b in range(B):
        for h in range(H):
            for j in range(-(-Tq2 // g)):
                toks = keep[b, h, j * g:min((j + 1) * g, Tq2)]
                t0 = int(toks[0])
                old_n = min(g, Tq - t0) if t0 < Tq else -1
                whole = t0 % g == 0 and len(toks) == old_n and np.array_equal(toks, np.arange(t0, t0 + old_n))
                if whole:
                    n_copied += 1
                    assert np.array_equal(e["k_scale"][b, h, j], c["k_scale"][b, h, t0 // g])
                    assert np.array_equal(e["k_zero"][b, h, j], c["k_zero"][b, h, t0 // g])
                    continue
                vals = x[b, j * g:(j + 1) * g, h]
                floor = np.maximum(vals.max(0) - vals.min(0), np.float32(1e-8)).astype(np.float32) / np.float32(15)
                assert np.all(f32(e["k_scale"][b, h, j]) >= floor)
                assert np.all(f32(e["k_scale"][b, h, j] - np.uint16(1)) < floor)
    # residual rows: the kept values rounded to the nearest bf16; torch's fp32 -> bf16
    # conversion (round to nearest, ties to even) is the independent rounding
    import torch
    for side, gx in (("k", gk), ("v", gv)):
        want = torch.from_numpy(np.ascontiguousarray(gx[:, Tq2:])).to(torch.bfloat16).view(torch.int16).numpy()
        assert np.array_equal(e[side + "_res"], want.view(np.uint16).transpose(0, 2, 1, 3))
    return n_copied


@pytest.mark.parametrize("g", [32, 64, 128])
def test_evict_requantized_groups_bound_nearest_level_and_residual_rounding(g):
    B, H, d, R = 1, 2, 128, 30
    T = 5 * g + 9 + R
    Kb, Vb = _c2_like(B, T, H, d, seed=3 * g)
    c = oracle.int4_quant(Kb, Vb, g, R)
    rng = np.random.default_rng(g + 7)
    K = 3 * g + 20
    keep = np.sort(np.stack([[rng.choice(T, K, replace=False) for _ in range(H)] for _ in range(B)]), -1)
    keep = keep.astype(np.int32)
    _check_evicted(c, keep, 13, oracle.int4_evict(c, keep, 13))


@pytest.mark.parametrize("g", [32, 64])
def test_evict_shifted_and_aligned_runs(g):
    # head 0 keeps a contiguous run that starts mid-group (every group must be requantized);
    # head 1 keeps two whole aligned groups and then the same kind of shifted run
    B, H, d, R = 1, 2, 128, 16
    T = 6 * g + R
    Kb, Vb = _c2_like(B, T, H, d, seed=g + 11)
    c = oracle.int4_quant(Kb, Vb, g, R)
    K = 4 * g
    keep = np.stack([np.arange(g // 2, g // 2 + K),
                     np.concatenate([np.arange(g, 3 * g), np.arange(3 * g + 5, 5 * g + 5)])])[None].astype(np.int32)
    e = oracle.int4_evict(c, keep, 0)
    assert _check_evicted(c, keep, 0, e) == 2


@pytest.mark.parametrize("g", [32, 128])
def test_evict_prefix_of_a_group_and_quantized_tokens_into_the_window(g):
    # keep the first 2g + 5 + 20 tokens with 20 bf16 rows: the new quantized part ends 5
    # tokens into old group 2 (a prefix of a group is not that group: requantized), and the
    # window receives 20 dequantized 4-bit tokens, rounded to bf16
    B, H, d, R = 1, 1, 128, 8
    T = 4 * g + R
    Kb, Vb = _c2_like(B, T, H, d, seed=g + 21)
    c = oracle.int4_quant(Kb, Vb, g, R)
    keep = np.arange(2 * g + 25, dtype=np.int32)[None, None]
    e = oracle.int4_evict(c, keep, 20)
    assert _check_evicted(c, keep, 20, e) == 2
    assert not np.array_equal(e["k_scale"][0, 0, 2], c["k_scale"][0, 0, 2])


def test_evict_rejects_bad_arguments():
    Kb, Vb = _c2_like(1, 100, 1, 64, seed=0)
    c = oracle.int4_quant(Kb, Vb, 64, 10)
    keep = np.arange(50, dtype=np.int32)[None, None]
    with pytest.raises(Exception):
        oracle.int4_evict(c, keep, 51)
    with pytest.raises(Exception):
        oracle.int4_evict(c, np.full((1, 1, 5), 100, np.int32), 0)


# ------------------------------------------------------ decode-time H2O scores --

def test_h2o_decode_two_tokens_closed_form_per_query_head():
    # two tokens, k_0 = 0, k_1 = a e_0; query head hq has q = (hq + 1) e_0, so its weight on
    # token 1 is e^{(hq+1) a} / (1 + e^{(hq+1) a}); the KV head's score adds those of its
    # query heads (4 query heads over 2 KV heads).
    d = 64
    K = np.zeros((1, 2, 2, d), np.float32)
    K[0, 1, :, 0] = 0.375
    V = np.ones((1, 2, 2, d), np.float32)
    Kb, Vb = bf16(K), bf16(V)
    a = float(f32(Kb)[0, 1, 0, 0])
    q = np.zeros((1, 4, d), np.float32)
    q[0, :, 0] = np.arange(1, 5)
    c = _all_residual_cache(Kb, Vb)
    _, probs = oracle.decode_attn_probs(c, bf16(q))
    acc0 = np.array([[[0.5, 0.25], [1.0, 2.0]]])
    acc = oracle.h2o_decode_scores(acc0, probs)
    w = lambda m: math.exp(m * a) / (1 + math.exp(m * a))
    for h in range(2):
        want1 = acc0[0, h, 1] + w(2 * h + 1) + w(2 * h + 2)
        want0 = acc0[0, h, 0] + (1 - w(2 * h + 1)) + (1 - w(2 * h + 2))
        assert abs(acc[0, h, 1] - want1) < 1e-14 and abs(acc[0, h, 0] - want0) < 1e-14


def test_h2o_decode_scores_sum_and_match_offline_colsum():
    # each decode step hands out exactly G = Hq / H units of weight per KV head; summed over
    # steps, the running score equals the offline H2O column sum of the same weights
    B, T, H, Hq, d, g = 1, 150, 2, 4, 64, 32
    Kb, Vb = _c2_like(B, T, H, d, seed=9)
    c = oracle.int4_quant(Kb, Vb, g, 22)
    rng = np.random.default_rng(9)
    acc = np.zeros((B, H, T))
    hist = []
    for step in range(5):
        q = bf16(rng.standard_normal((B, Hq, d)) / 8)
        _, probs = oracle.decode_attn_probs(c, q)
        new = oracle.h2o_decode_scores(acc, probs)
        assert np.allclose((new - acc).sum(-1), Hq // H, rtol=0, atol=1e-12)
        acc = new
        hist.append(probs.reshape(B, H, Hq // H, T))
    hist = np.concatenate(hist, axis=2).reshape(B * H, -1, T).astype(np.float32)
    assert np.allclose(oracle.colsum(hist), acc.reshape(B * H, T), rtol=1e-5, atol=1e-7)


# -------------------------------------------------- Hadamard-rotated 4-bit cache --

def _signs(d, seed):
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1, 1).astype(np.int8)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_is_the_sylvester_hadamard_matrix(d):
    from scipy.linalg import hadamard
    Hm = hadamard(d).astype(np.float64)
    s = _signs(d, d)
    rng = np.random.default_rng(d)
    x = rng.standard_normal((50, d)).astype(np.float32)
    ref = (x.astype(np.float64) * s) @ Hm.T / math.sqrt(d)
    y = oracle.rotate(x, s).astype(np.float64)
    assert np.allclose(y, ref, rtol=0, atol=2e-6 * np.abs(x).sum(-1, keepdims=True).max())
    # small integers: every butterfly sum is exact, so only the final scale rounds
    xi = rng.integers(-8, 9, (20, d)).astype(np.float32)
    exact = ((xi.astype(np.float64) * s) @ Hm.T).astype(np.float32)
    want = exact * np.float32(1.0 / math.sqrt(d))
    assert np.array_equal(oracle.rotate(xi, s), want)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_orthogonal_inverse_and_outlier_spreading(d):
    s = _signs(d, d + 1)
    # the basis vectors map to rows of +-1/sqrt(d), mutually orthogonal
    E = np.eye(d, dtype=np.float32)
    R = oracle.rotate(E, s).astype(np.float64)
    assert np.allclose(np.abs(R), 1 / math.sqrt(d), rtol=1e-6, atol=0)
    assert np.allclose(R @ R.T, np.eye(d), atol=1e-6)
    # one outlier channel of size a spreads into d coordinates of size a / sqrt(d)
    x = np.zeros((1, d), np.float32)
    x[0, 5] = 100.0
    assert np.allclose(np.abs(oracle.rotate(x, s)), 100.0 / math.sqrt(d), rtol=1e-6)
    # the inverse recovers the input and the norm is kept
    rng = np.random.default_rng(d)
    x = rng.standard_normal((40, d)).astype(np.float32) * (1 + 30 * (rng.random(d) < 0.05))
    y = oracle.rotate(x, s)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-5)
    assert np.allclose(oracle.unrotate(y, s), x, rtol=0, atol=1e-5 * np.abs(x).max())


def test_rotation_equalizes_coordinate_variance():
    # independent coordinates with variances lambda_i -> every rotated coordinate has variance mean(lambda)
    d, n = 128, 20000
    rng = np.random.default_rng(7)
    lam = np.exp(rng.uniform(-3, 4, d))
    x = (rng.standard_normal((n, d)) * np.sqrt(lam)).astype(np.float32)
    y = oracle.rotate(x, _signs(d, 7)).astype(np.float64)
    var = y.var(0)
    assert lam.max() / lam.min() > 500
    assert np.all(np.abs(var / lam.mean() - 1) < 0.06)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_rot_quant_round_trip_nearest_level_and_norm_bound(g):
    from scipy.linalg import hadamard
    B, T, H, d = 1, 40, 2, 128
    Kb, Vb = _c2_like(B, T, H, d, seed=g + 3)
    ks, vs = _signs(d, 1), _signs(d, 2)
    c = oracle.rot_quant(Kb, Vb, g, ks, vs)
    Hm = hadamard(d).astype(np.float64) / math.sqrt(d)
    for side, X, s in (("k", Kb, ks), ("v", Vb, vs)):
        x = f32(X).astype(np.float64)                          # [B][T][H][d]
        y = (x * s) @ Hm.T                                      # rotated, fp64
        codes = c[side + "_codes"]
        q = np.stack([codes & 15, codes >> 4], -1).reshape(B, H, T, d).transpose(0, 2, 1, 3).astype(np.int64)
        sc = np.repeat(f32(c[side + "_scale"]).astype(np.float64), g, -1).transpose(0, 2, 1, 3)
        z = np.repeat(f32(c[side + "_zero"]).astype(np.float64), g, -1).transpose(0, 2, 1, 3)
        yh = (q - z) * sc
        # each rotated value within half a step of its level, on the nearest level (away from ties)
        assert np.all(np.abs(y - yh) <= sc / 2 * (1 + 1e-5) + 1e-6)
        levels = (np.arange(16)[None, None, None, None, :] - z[..., None]) * sc[..., None]
        dist = np.abs(y[..., None] - levels)
        srt = np.sort(dist, -1)
        clear = srt[..., 1] - srt[..., 0] > 1e-5 * sc
        assert np.array_equal(np.argmin(dist, -1)[clear], q[clear])
        # back in the original coordinates the error norm equals the rotated one (orthogonality)
        xh = oracle.rot_dequant(c, side).astype(np.float64)
        e_orig = np.linalg.norm(x - xh, axis=-1)
        e_rot = np.linalg.norm(y - yh, axis=-1)
        assert np.allclose(e_orig, e_rot, rtol=1e-4, atol=1e-6)


def test_rotation_beats_plain_per_token_quantization_on_outlier_channels():
    # K with 4 outlier channels (x10): per-token 4-bit groups waste their range on the outliers
    # unless the rotation spreads them first
    B, T, H, d, g = 1, 256, 2, 128, 64
    Kb, Vb = _c2_like(B, T, H, d, seed=5)
    ident = np.ones(d, np.int8)
    c = oracle.rot_quant(Kb, Vb, g, _signs(d, 5), ident)
    x = f32(Kb).astype(np.float64)
    err_rot = np.sqrt(((x - oracle.rot_dequant(c, "k")) ** 2).mean())
    # plain per-token groups = the 4-bit V format of the KIVI quantizer applied to K
    plain = oracle.int4_quant(Vb, Kb, g, 0)
    err_plain = np.sqrt(((x - oracle.int4_dequant(plain, "v")) ** 2).mean())
    assert err_rot < 0.6 * err_plain


def test_rot_attention_is_attention_over_the_unrotated_cache():
    # softmax attention (numpy, fp64) over the dequantized cache taken back to the original
    # coordinates must equal the rotated-space attention with its output rotated back
    from scipy.linalg import hadamard
    B, T, H, Hq, d, g = 2, 70, 2, 8, 64, 32
    Kb, Vb = _c2_like(B, T, H, d, seed=8)
    ks, vs = _signs(d, 3), _signs(d, 4)
    c = oracle.rot_quant(Kb, Vb, g, ks, vs)
    rng = np.random.default_rng(8)
    q = bf16(rng.standard_normal((B, Hq, d)) / 8)
    out = oracle.rot_decode_attn(c, q, 0.5)
    Hm = hadamard(d).astype(np.float64) / math.sqrt(d)

    def levels(side):
        codes = c[side + "_codes"]
        qq = np.stack([codes & 15, codes >> 4], -1).reshape(B, H, T, d).astype(np.float64)
        sc = np.repeat(f32(c[side + "_scale"]).astype(np.float64), g, -1)
        z = np.repeat(f32(c[side + "_zero"]).astype(np.float64), g, -1)
        return (qq - z) * sc                                   # [B][H][T][d], rotated coordinates

    Kx = (levels("k") @ Hm) * ks                               # back to the original coordinates
    Vx = (levels("v") @ Hm) * vs
    qf = f32(q).astype(np.float64)
    for b in range(B):
        for hq in range(Hq):
            h = hq // (Hq // H)
            lg = 0.5 * Kx[b, h] @ qf[b, hq]
            p = np.exp(lg - lg.max())
            want = p @ Vx[b, h] / p.sum()
            assert np.allclose(out[b, hq], want, rtol=0, atol=1e-10)


# ------------------------------------------------------ per-token mixed precision --

def _mixed_case(N, Cc, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, Cc)).astype(np.float32) * np.exp(rng.uniform(-2, 2, (N, 1))).astype(np.float32)
    x[rng.random(N) < 0.1, :] += 3.0          # some rows offset from zero
    tags = rng.integers(0, 4, N).astype(np.uint8)
    return bf16(x), tags


def _unpack(codes, bits, Cc):
    per = 8 // bits
    out = np.zeros((codes.shape[0], Cc), np.int64)
    for i in range(per):
        v = (codes.astype(np.int64) >> (bits * i)) & ((1 << bits) - 1)
        v = np.where(v >= (1 << (bits - 1)), v - (1 << bits), v)
        out[:, i::per] = v
    return out


def test_mixed_tag_packing_and_slots_bruteforce():
    rng = np.random.default_rng(1)
    tags = rng.integers(0, 4, 1001).astype(np.uint8)
    packed = oracle.pack_tags(tags)
    assert len(packed) == 251
    for r in (0, 1, 2, 3, 4, 999, 1000):
        assert (packed[r // 4] >> (2 * (r % 4))) & 3 == tags[r]
    slot, counts = oracle.mixed_plan(packed, len(tags))
    seen = [0, 0, 0, 0]
    for r, t in enumerate(tags):
        assert slot[r] == seen[t]
        seen[t] += 1
    assert list(counts) == seen == list(np.bincount(tags, minlength=4))


@pytest.mark.parametrize("Cc", [64, 128, 4096])
def test_mixed_rows_equal_the_per_channel_quantizers_on_one_row(Cc):
    # a row quantized at 2 / 4 bits is the symmetric quantizer of Walkthrough §1.1 applied to that
    # row as one channel; at 8 bits the asymmetric one of §1.2 with [-128, 127]; 16 bits keeps the bits
    N = 60
    xb, tags = _mixed_case(N, Cc, seed=Cc)
    m = oracle.mixed_quant(xb, oracle.pack_tags(tags))
    codes = {0: _unpack(m["q2"], 2, Cc), 1: _unpack(m["q4"], 4, Cc)}
    for r in range(N):
        t, k = int(tags[r]), int(m["slot"][r])
        col = xb[r][:, None]                          # the row as one channel of Cc "rows"
        if t in (0, 1):
            q = np.zeros((Cc, 1), np.int8)
            s = np.zeros(1, np.float32)
            oracle.lib().orc_quant_sym(oracle._p(np.ascontiguousarray(col)), 1, 1, Cc, 1, 2 if t == 0 else 4,
                                       oracle._p(q), oracle._p(s), None)
            assert np.array_equal(codes[t][k], q[:, 0].astype(np.int64)), (r, t)
            assert m["s2" if t == 0 else "s4"][k] == s[0]
        elif t == 2:
            q = np.zeros((Cc, 1), np.int8)
            s = np.zeros(1, np.float32)
            z = np.zeros(1, np.int8)
            oracle.lib().orc_quant_asym(oracle._p(np.ascontiguousarray(col)), 1, 1, Cc, 1, -128, 127,
                                        oracle._p(q), oracle._p(s), oracle._p(z))
            assert np.array_equal(m["q8"][k], q[:, 0]) and m["s8"][k] == s[0] and m["z8"][k] == z[0]
        else:
            assert np.array_equal(m["x16"][k], xb[r])


def test_mixed_round_trip_bounds_and_levels():
    N, Cc = 200, 128
    xb, tags = _mixed_case(N, Cc, seed=2)
    m = oracle.mixed_quant(xb, oracle.pack_tags(tags))
    x = f32(xb).astype(np.float64)
    xh = oracle.mixed_dequant(m).astype(np.float64)
    for r in range(N):
        t, k = int(tags[r]), int(m["slot"][r])
        if t == 3:
            assert np.array_equal(xh[r], x[r])
            continue
        s = float({0: m["s2"], 1: m["s4"], 2: m["s8"]}[t][k])
        qmax = {0: 1, 1: 7, 2: None}[t]
        if qmax is not None:
            # symmetric: s = absmax / qmax exactly as fp32 quotient; every value within s/2 of its level
            assert np.float32(max(np.abs(x[r]).max(), np.float32(1e-8))) / np.float32(qmax) == np.float32(s)
        # half a level, plus the fp32 rounding of the quotient x / s that the codes are taken from
        # (a quotient that rounds onto a half-integer then rounds to even)
        e = np.abs(x[r] - xh[r]) - 2.0**-22 * np.abs(x[r])
        if t == 2:
            # the rounded zero point can push the row's extremes one level past the code range:
            # codes away from the bounds are within s/2, clipped ones within 3s/2
            q = m["q8"][k].astype(np.int64)
            inner = (q > -128) & (q < 127)
            assert np.all(e[inner] <= s / 2) and np.all(e <= 1.5 * s), r
        else:
            assert np.all(e <= s / 2), (r, t)
    # worst-case error shrinks with the width: mean |error| / row scale orders 2 > 4 > 8 bits
    err = {t: np.mean([np.abs(x[r] - xh[r]).mean() / np.abs(x[r]).max() for r in range(N) if tags[r] == t])
           for t in (0, 1, 2)}
    assert err[0] > err[1] > err[2]


def test_mixed_bytes_closed_form():
    # counts (10, 20, 30, 40) of 2/4/8/16-bit rows of 128 channels, 100 rows
    data, meta, tagb = oracle.mixed_bytes([10, 20, 30, 40], 100, 128)
    assert data == 10 * 32 + 20 * 64 + 30 * 128 + 40 * 256
    assert meta == 10 * 4 + 20 * 4 + 30 * 5
    assert tagb == 25                                    # 2 bits per token
    # tags are 2 bits of 2*128*8 = 2048 bits of a bf16 token row: 1/1024 of the unquantized store
    assert oracle.mixed_bytes([0, 0, 0, 8192], 8192, 128)[2] / (8192 * 256) == 1 / 1024
