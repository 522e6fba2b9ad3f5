"""Property-based pins of the CPU oracle (Hypothesis): generated inputs, each checked against
what the method guarantees rather than against a re-typed formula.

- INT4 groups (Explainer (KV cache 压缩：把历史装得更小), quantization and grouping-axis
  sections): every element lies within half a stored step of its level, its code is the
  nearest of the 16 levels (exact ties to the even integer), codes never decrease as the
  value grows, and the zero point is an integer that bf16 holds exactly.
- Per-channel INT8-style codes (Walkthrough (KV Compression 公式到源码对照) §1.1, §1.2): codes
  in range, the nearest integer to the exact quotient wherever that is not within rounding
  of a tie, monotone in the value; dequantization rounds the exact (q - z) s once.
- TopK union (Walkthrough §3.2): the kept set equals a rank count over the masked scores
  (NaN and signed zeros included), sorted, unique, window included, of the stated size.
- Error statistics and compaction against exact rational sums and a plain gather.

Inputs are drawn with a fixed derandomized seed so every run checks the same cases.
"""
import math
from fractions import Fraction

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = dict(deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])


def bf16(x):
    return oracle.f32_to_bf16(np.asarray(x, np.float32))


def f32(b):
    return oracle.bf16_to_f32(b)


# ------------------------------------------------------------------ INT4 ----

@st.composite
def int4_layer(draw):
    """bf16 K, V [1][T][2][d] with one group's worth of structure drawn per call: a base
    distribution at a drawn magnitude, an offset far from zero relative to the spread, constant
    channels / tokens, exact zeros, and a ragged last K group."""
    g = draw(st.sampled_from([32, 64, 128]))
    d = draw(st.sampled_from([128, 256])) if g == 128 else draw(st.sampled_from([64, 128, 256]))
    T = g * draw(st.integers(1, 2)) + draw(st.integers(0, g - 1))
    seed = draw(st.integers(0, 2**31 - 1))
    e = draw(st.integers(-30, 30))                 # magnitude 10^e
    spread = draw(st.sampled_from([1.0, 1e-2, 1e-4]))
    offset = draw(st.sampled_from([0.0, 1.0, -1.0, 37.5, -300.0]))
    dist = draw(st.sampled_from(["normal", "uniform", "heavy", "signs"]))
    rng = np.random.default_rng(seed)
    arrs = []
    for _ in range(2):
        if dist == "normal":
            x = rng.standard_normal((1, T, 2, d))
        elif dist == "uniform":
            x = rng.uniform(-1, 1, (1, T, 2, d))
        elif dist == "heavy":
            x = rng.standard_t(2, (1, T, 2, d))
        else:
            x = np.sign(rng.standard_normal((1, T, 2, d)))
        x = (offset + spread * x) * 10.0 ** e
        if draw(st.booleans()):
            x[0, :, 0, rng.integers(0, d)] = x[0, 0, 0, 0]        # a constant K channel
            x[0, rng.integers(0, T), 1, :] = 0.0                   # an all-zero V token
        xb = bf16(x.astype(np.float32))
        if not np.all(np.isfinite(f32(xb))):
            xb = bf16(np.nan_to_num(f32(xb), posinf=3e38, neginf=-3e38))
        arrs.append(xb)
    return arrs[0], arrs[1], g


def _groups(c, side):
    """(x index helpers) -> per element of the quantized region: code, scale, zero (fp64)."""
    B, T, H, d, g, R = (c[k] for k in ("B", "T", "H", "d", "g", "R"))
    Tq = T - R
    codes = c[side + "_codes"]
    q = np.stack([codes & 15, codes >> 4], -1).reshape(B, H, Tq, d).transpose(0, 2, 1, 3).astype(np.int64)
    s = f32(c[side + "_scale"]).astype(np.float64)
    z = f32(c[side + "_zero"]).astype(np.float64)
    if side == "k":
        s = np.repeat(s, g, axis=2)[:, :, :Tq].transpose(0, 2, 1, 3)
        z = np.repeat(z, g, axis=2)[:, :, :Tq].transpose(0, 2, 1, 3)
    else:
        s = np.repeat(s, g, axis=3).transpose(0, 2, 1, 3)
        z = np.repeat(z, g, axis=3).transpose(0, 2, 1, 3)
    return q, s, z


@settings(max_examples=60, **SETTINGS)
@given(int4_layer())
def test_int4_groups_bound_nearest_and_monotone(layer):
    K, V, g = layer
    c = oracle.int4_quant(K, V, g, 0)
    for side, X in (("k", K), ("v", V)):
        x = f32(X).astype(np.float64)
        q, s, z = _groups(c, side)
        # the zero point is an integer bf16 holds exactly, the scale a positive bf16
        assert np.all(z == np.round(z)) and np.all(np.abs(z) <= 256) and np.all(s > 0)
        # levels (k - z) s are exact in fp64; every element within half a step of its own
        lv = (q - z) * s
        assert np.all(np.abs(x - lv) <= s / 2), side
        # nearest of the 16 levels, exact ties to the even integer k - z
        levels = (np.arange(16) - z[..., None]) * s[..., None]
        dist = np.abs(x[..., None] - levels)
        best = dist.min(-1, keepdims=True)
        cand = dist == best
        even = ((np.arange(16) - z[..., None]) % 2) == 0
        pick = np.where(cand.sum(-1) > 1, np.argmax(cand & even, -1), np.argmax(cand, -1))
        assert np.array_equal(pick, q), side
        # inside one group a larger value never gets a smaller code
        if side == "k":
            xs, qs = x[0, :, 0, 0], q[0, :, 0, 0]            # channel 0 of head 0, its K groups
            for j0 in range(0, len(xs), g):
                o = np.argsort(xs[j0:j0 + g], kind="stable")
                assert np.all(np.diff(qs[j0:j0 + g][o]) >= 0)
        else:
            xs, qs = x[0, 0, 0, :g], q[0, 0, 0, :g]            # token 0, head 0, first V group
            o = np.argsort(xs, kind="stable")
            assert np.all(np.diff(qs[o]) >= 0)


# ------------------------------------------------------------ per channel ----

finite32 = st.floats(min_value=-1e6, max_value=1e6, allow_nan=False, allow_infinity=False, width=32)


@st.composite
def pc_matrix(draw):
    R = draw(st.integers(1, 9))
    C = draw(st.integers(1, 4))
    vals = draw(st.lists(finite32, min_size=R * C, max_size=R * C))
    x = np.array(vals, np.float32).reshape(R, C)
    if draw(st.booleans()):
        x[:, 0] = x[0, 0]                              # a constant channel
    return x


def _near_tie(r: Fraction) -> bool:
    frac = r - math.floor(r)
    return abs(frac - Fraction(1, 2)) <= Fraction(1, 2**20)


@settings(max_examples=150, **SETTINGS)
@given(pc_matrix(), st.integers(2, 8))
def test_per_channel_sym_nearest_integer_and_monotone(x, bits):
    q, s, z = oracle.quant_sym(x, bits)
    qmax = (1 << (bits - 1)) - 1
    q, s = q[0].astype(np.int64), s[0]
    assert np.all(z == 0) and np.all(s > 0)
    assert np.all(np.abs(q) <= qmax)
    for c in range(x.shape[1]):
        sc = Fraction(float(s[c]))
        for r in range(x.shape[0]):
            quo = Fraction(float(x[r, c])) / sc
            assert abs(quo - q[r, c]) <= Fraction(1, 2) + Fraction(1, 2**20)
            if not _near_tie(quo) and abs(quo) <= qmax:
                assert q[r, c] == round(quo)
        o = np.argsort(x[:, c], kind="stable")
        assert np.all(np.diff(q[o, c]) >= 0)
    # dequantization: the exact product q * s, rounded once to fp32
    xh = oracle.dequant_pc(q[None].astype(np.int8), s[None], None)[0]
    want = np.array([[np.float32(float(q[r, c]) * float(s[c])) for c in range(x.shape[1])]
                     for r in range(x.shape[0])], np.float32)
    assert np.array_equal(xh.view(np.uint32), want.view(np.uint32))


@settings(max_examples=150, **SETTINGS)
@given(pc_matrix(), st.sampled_from([(-128, 127), (0, 15), (-8, 7), (0, 127)]))
def test_per_channel_asym_range_monotone_and_dequant(x, qr):
    qmin, qmax = qr
    q, s, z = oracle.quant_asym(x, qmin, qmax)
    q, s, z = q[0].astype(np.int64), s[0], z[0].astype(np.int64)
    assert np.all(q >= qmin) and np.all(q <= qmax) and np.all(s > 0)
    for c in range(x.shape[1]):
        o = np.argsort(x[:, c], kind="stable")
        assert np.all(np.diff(q[o, c]) >= 0)
    xh = oracle.dequant_pc(q[None].astype(np.int8), s[None], z[None].astype(np.int8))[0]
    want = np.array([[np.float32(float(q[r, c] - z[c]) * float(s[c])) for c in range(x.shape[1])]
                     for r in range(x.shape[0])], np.float32)
    assert np.array_equal(xh.view(np.uint32), want.view(np.uint32))


# -------------------------------------------------------------- selection ---

SPECIAL = [math.nan, 0.0, -0.0, math.inf, -math.inf, 0.5, -0.5, 1.0]


def _above(a, b):
    """Score a ranks strictly above score b: numbers in IEEE order (-0 == +0), NaN lowest."""
    na, nb = math.isnan(a), math.isnan(b)
    if na or nb:
        return nb and not na
    return a > b


def _same(a, b):
    return (math.isnan(a) and math.isnan(b)) or a == b


@settings(max_examples=300, **SETTINGS)
@given(st.lists(st.sampled_from(SPECIAL), min_size=1, max_size=14), st.integers(0, 16), st.integers(0, 7))
def test_select_is_a_rank_count_over_the_masked_scores(vals, budget, window):
    T = len(vals)
    sc = np.array(vals, np.float32)
    keep = oracle.select(sc[None], budget, window)[0].tolist()
    rs = max(0, T - window)
    k = min(max(0, budget - (T - rs)), T)

    def ranks_above(j, i):
        if (j >= rs) != (i >= rs):          # the window's masked tokens rank below every other
            return i >= rs
        a, b = float(sc[j]), float(sc[i])
        if j >= rs:
            a = b = -math.inf
        return _above(a, b) or (_same(a, b) and j < i)

    heavy = {i for i in range(T) if sum(1 for j in range(T) if ranks_above(j, i)) < k}
    assert keep == sorted(set(range(rs, T)) | heavy)
    assert keep == sorted(set(keep))
    assert len(keep) == oracle.keep_count(T, budget, window) == min(T, max(budget, min(window, T)))


# ------------------------------------------------ statistics and compaction ---

@settings(max_examples=100, **SETTINGS)
@given(st.lists(st.tuples(finite32, finite32), min_size=1, max_size=40))
def test_err_stats_are_the_exact_sums_rounded(pairs):
    x = np.array([p[0] for p in pairs], np.float32)
    xh = np.array([p[1] for p in pairs], np.float32)
    ss, sa, mx = oracle.err_stats(x, xh)
    e = [Fraction(float(a)) - Fraction(float(b)) for a, b in zip(x, xh)]
    ex_ss = sum(v * v for v in e)
    ex_sa = sum(abs(v) for v in e)
    n = len(e)
    # each difference is rounded once to fp64 (relative 2^-53), then n terms are accumulated:
    # relative error at most about (n + 2) * 2^-52
    tol = Fraction(n + 2, 2**51)
    assert abs(Fraction(ss) - ex_ss) <= tol * ex_ss
    assert abs(Fraction(sa) - ex_sa) <= tol * ex_sa
    ex_mx = max(abs(v) for v in e)
    assert abs(Fraction(mx) - ex_mx) <= Fraction(1, 2**53) * ex_mx


@settings(max_examples=80, **SETTINGS)
@given(st.integers(1, 3), st.integers(1, 20), st.integers(1, 3), st.sampled_from([8, 16]), st.data())
def test_compact_is_a_gather(B, T, H, d, data):
    rng = np.random.default_rng(data.draw(st.integers(0, 2**31 - 1)))
    src = rng.integers(0, 65536, (B, T, H, d), dtype=np.uint16)
    Kk = data.draw(st.integers(1, T))
    keep = np.stack([np.stack([np.sort(rng.choice(T, Kk, replace=False)) for _ in range(H)]) for _ in range(B)])
    keep = keep.astype(np.int32)
    dst = oracle.compact(src, keep)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(dst[b, :, h], src[b, keep[b, h], h])
