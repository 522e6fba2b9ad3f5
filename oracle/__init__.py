"""TEST INFRASTRUCTURE ONLY: ctypes wrapper around the plain C oracle (liboracle.so).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It never touches the GPU library and the GPU library
never touches it.  Arrays are numpy; bf16 data travels as its raw uint16 bits.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "kvq_oracle.c")

# -ffp-contract=off: every fp32 step is its own IEEE operation; no -ffast-math, no -march
# (the default x86-64 target has no FMA); single-threaded.
GCC_CMD = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB_PATH, SRC_PATH, "-lm"]


def build() -> str:
    subprocess.run(GCC_CMD, check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


P = C.c_void_p
I64 = C.c_int64


def _declare(L):
    L.orc_quant_sym.argtypes = [P, C.c_int, I64, I64, I64, C.c_int, P, P, P]
    L.orc_quant_asym.argtypes = [P, C.c_int, I64, I64, I64, C.c_int, C.c_int, P, P, P]
    L.orc_dequant_pc.argtypes = [P, P, P, I64, I64, I64, P]
    L.orc_dequant_pc.restype = None
    L.orc_err_stats.argtypes = [P, C.c_int, P, C.c_int, I64, P]
    L.orc_err_stats.restype = None
    L.orc_stats_finalize.argtypes = [P, I64, P, P, P]
    L.orc_stats_finalize.restype = None
    L.orc_int4_quant.argtypes = [P, P, I64, I64, I64, I64, I64, I64] + [P] * 8
    L.orc_int4_dequant.argtypes = [C.c_int, P, P, P, P, I64, I64, I64, I64, I64, I64, P]
    L.orc_int4_dequant.restype = None
    L.orc_decode_attn.argtypes = [P] * 8 + [I64] * 6 + [P, I64, C.c_double, P]
    L.orc_decode_attn_rows.argtypes = [P] * 8 + [I64] * 6 + [P, I64, C.c_double, P, P, I64, P, P]
    L.orc_int4_evict.argtypes = [P] * 8 + [I64] * 6 + [P, I64, I64] + [P] * 8
    L.orc_rotate_f32.argtypes = [P, P, I64, I64, P]
    L.orc_rotate_f32.restype = None
    L.orc_unrotate_f32.argtypes = [P, P, I64, I64, P]
    L.orc_unrotate_f32.restype = None
    L.orc_rot_quant.argtypes = [P, P] + [I64] * 5 + [P, P] + [P] * 6
    L.orc_rot_dequant.argtypes = [P, P, P, P] + [I64] * 5 + [P]
    L.orc_rot_dequant.restype = None
    L.orc_rot_decode_attn.argtypes = [P] * 8 + [I64] * 5 + [P, I64, C.c_double, P]
    L.orc_mixed_plan.argtypes = [P, I64, P, P]
    L.orc_mixed_plan.restype = None
    L.orc_mixed_quant.argtypes = [P, I64, I64, P, P] + [P] * 8
    L.orc_mixed_dequant.argtypes = [I64, I64, P, P] + [P] * 8 + [P]
    L.orc_mixed_dequant.restype = None
    L.orc_mixed_bytes.argtypes = [P, I64, I64, P]
    L.orc_mixed_bytes.restype = None
    L.orc_colsum.argtypes = [P, I64, I64, I64, P]
    L.orc_colsum.restype = None
    L.orc_keep_count.argtypes = [I64, I64, I64]
    L.orc_keep_count.restype = I64
    L.orc_select.argtypes = [P, I64, I64, I64, I64, P]
    L.orc_h2o_select.argtypes = [P, I64, I64, I64, I64, I64, P, P]
    L.orc_compact.argtypes = [P, I64, I64, I64, I64, P, I64, P]
    L.orc_compact.restype = None
    L.orc_int4_bytes.argtypes = [C.c_uint64, C.c_uint64]
    L.orc_int4_bytes.restype = C.c_uint64
    L.orc_int4_cache_sizes.argtypes = [I64] * 6 + [P, P]
    L.orc_compression_ratio.argtypes = [C.c_uint64] * 4
    L.orc_compression_ratio.restype = C.c_double
    L.orc_token_ratio.argtypes = [I64, I64, P]
    L.orc_total_gain.argtypes = [C.c_double, C.c_double, I64, I64]
    L.orc_total_gain.restype = C.c_double
    L.orc_kv_bytes.argtypes = [C.c_uint64] * 5
    L.orc_kv_bytes.restype = C.c_uint64
    L.orc_f32_to_bf16.argtypes = [C.c_float]
    L.orc_f32_to_bf16.restype = C.c_uint16
    L.orc_bf16_to_f32.argtypes = [C.c_uint16]
    L.orc_bf16_to_f32.restype = C.c_float
    L.orc_f32_to_bf16_array.argtypes = [P, I64, P]
    L.orc_f32_to_bf16_array.restype = None


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _x(a: np.ndarray):
    """Pointer + bf16 flag for an fp32 or bf16(uint16) array."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, 0
    if a.dtype == np.uint16:
        return a, 1
    raise TypeError(f"oracle takes float32 or bf16-as-uint16, got {a.dtype}")


class OracleError(ValueError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle rejected the arguments (rc={rc})")


# ------------------------------------------------------------ per-channel --

def quant_sym(x: np.ndarray, bits: int):
    """x: [nb][R][C] or [R][C] fp32/bf16 -> (q int8, scale fp32 [nb][C], zp int8 [nb][C])."""
    x3 = x.reshape((-1,) + x.shape[-2:]) if x.ndim >= 2 else x.reshape(1, -1, 1)
    x3, isb = _x(x3)
    nb, R, Cc = x3.shape
    q = np.empty((nb, R, Cc), np.int8)
    s = np.empty((nb, Cc), np.float32)
    z = np.empty((nb, Cc), np.int8)
    _check(lib().orc_quant_sym(_p(x3), isb, nb, R, Cc, bits, _p(q), _p(s), _p(z)), "quant_sym")
    return q, s, z


def quant_asym(x: np.ndarray, qmin: int, qmax: int):
    x3 = x.reshape((-1,) + x.shape[-2:])
    x3, isb = _x(x3)
    nb, R, Cc = x3.shape
    q = np.empty((nb, R, Cc), np.int8)
    s = np.empty((nb, Cc), np.float32)
    z = np.empty((nb, Cc), np.int8)
    _check(lib().orc_quant_asym(_p(x3), isb, nb, R, Cc, qmin, qmax, _p(q), _p(s), _p(z)), "quant_asym")
    return q, s, z


def dequant_pc(q: np.ndarray, scale: np.ndarray, zp):
    q = np.ascontiguousarray(q, np.int8)
    nb, R, Cc = q.shape
    scale = np.ascontiguousarray(scale, np.float32)
    out = np.empty((nb, R, Cc), np.float32)
    if zp is None:
        lib().orc_dequant_pc(_p(q), _p(scale), None, nb, R, Cc, _p(out))
    else:
        zp = np.ascontiguousarray(zp, np.int8)
        lib().orc_dequant_pc(_p(q), _p(scale), _p(zp), nb, R, Cc, _p(out))
    return out


def err_stats(x: np.ndarray, xh: np.ndarray):
    """-> (sum_sq, sum_abs, max_abs) in fp64."""
    x, xb = _x(x.reshape(-1))
    xh, hb = _x(xh.reshape(-1))
    assert x.size == xh.size
    out = np.zeros(3, np.float64)
    lib().orc_err_stats(_p(x), xb, _p(xh), hb, x.size, _p(out))
    return float(out[0]), float(out[1]), float(out[2])


def stats_finalize(raw, n: int):
    a = np.asarray(raw, np.float64)
    r, m, mean = C.c_double(), C.c_double(), C.c_double()
    lib().orc_stats_finalize(_p(a), n, C.byref(r), C.byref(m), C.byref(mean))
    return r.value, m.value, mean.value


# ------------------------------------------------------------------ INT4 ----

def int4_cache_sizes(B, T, H, d, g, R):
    sect = np.zeros(8, np.uint64)
    tot = C.c_uint64()
    _check(lib().orc_int4_cache_sizes(B, T, H, d, g, R, _p(sect), C.byref(tot)), "int4_cache_sizes")
    return [int(v) for v in sect], int(tot.value)


def int4_quant(K: np.ndarray, V: np.ndarray, g: int, R: int):
    """K, V bf16-as-uint16 [B][T][H][d] -> dict of the cache sections."""
    K = np.ascontiguousarray(K, np.uint16)
    V = np.ascontiguousarray(V, np.uint16)
    B, T, H, d = K.shape
    Tq = T - R
    nKg = -(-Tq // g) if Tq > 0 else 0
    c = dict(
        k_codes=np.zeros((B, H, Tq, d // 2), np.uint8),
        k_scale=np.zeros((B, H, nKg, d), np.uint16),
        k_zero=np.zeros((B, H, nKg, d), np.uint16),
        v_codes=np.zeros((B, H, Tq, d // 2), np.uint8),
        v_scale=np.zeros((B, H, Tq, d // g), np.uint16),
        v_zero=np.zeros((B, H, Tq, d // g), np.uint16),
        k_res=np.zeros((B, H, R, d), np.uint16),
        v_res=np.zeros((B, H, R, d), np.uint16),
    )
    rc = lib().orc_int4_quant(_p(K), _p(V), B, T, H, d, g, R,
                              _p(c["k_codes"]), _p(c["k_scale"]), _p(c["k_zero"]),
                              _p(c["v_codes"]), _p(c["v_scale"]), _p(c["v_zero"]),
                              _p(c["k_res"]), _p(c["v_res"]))
    _check(rc, "int4_quant")
    c.update(B=B, T=T, H=H, d=d, g=g, R=R)
    return c


def int4_dequant(c: dict, side: str):
    """side 'k' or 'v' -> fp32 [B][T][H][d]."""
    B, T, H, d, g, R = (c[k] for k in ("B", "T", "H", "d", "g", "R"))
    out = np.empty((B, T, H, d), np.float32)
    s = side.lower()
    lib().orc_int4_dequant(1 if s == "k" else 0, _p(c[s + "_codes"]), _p(c[s + "_scale"]),
                           _p(c[s + "_zero"]), _p(c[s + "_res"]), B, T, H, d, g, R, _p(out))
    return out


def _cache_ptrs(c):
    return [_p(np.ascontiguousarray(c[k])) for k in
            ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_res", "v_res")]


def decode_attn(c: dict, q: np.ndarray, sm_scale: float = 1.0, rows=None):
    """q bf16-as-uint16 [B][Hq][d] -> fp64 [B][Hq][d] (or [n_rows][d] for rows=[(b,hq),...])."""
    q = np.ascontiguousarray(q, np.uint16)
    B, Hq, d = q.shape
    args = _cache_ptrs(c) + [c["B"], c["T"], c["H"], c["d"], c["g"], c["R"], _p(q), Hq, float(sm_scale)]
    if rows is None:
        out = np.empty((B, Hq, d), np.float64)
        _check(lib().orc_decode_attn(*args, _p(out)), "decode_attn")
        return out
    rb = np.ascontiguousarray([r[0] for r in rows], np.int64)
    rh = np.ascontiguousarray([r[1] for r in rows], np.int64)
    out = np.empty((len(rows), d), np.float64)
    _check(lib().orc_decode_attn_rows(*args, _p(rb), _p(rh), len(rows), _p(out), None), "decode_attn_rows")
    return out


def decode_attn_probs(c: dict, q: np.ndarray, sm_scale: float = 1.0):
    """Attention output fp64 [B][Hq][d] and the attention weights fp64 [B][Hq][T]."""
    q = np.ascontiguousarray(q, np.uint16)
    B, Hq, d = q.shape
    T = c["T"]
    rb = np.repeat(np.arange(B, dtype=np.int64), Hq)
    rh = np.tile(np.arange(Hq, dtype=np.int64), B)
    out = np.empty((B, Hq, d), np.float64)
    probs = np.empty((B, Hq, T), np.float64)
    args = _cache_ptrs(c) + [c["B"], T, c["H"], c["d"], c["g"], c["R"], _p(q), Hq, float(sm_scale)]
    _check(lib().orc_decode_attn_rows(*args, _p(rb), _p(rh), B * Hq, _p(out), _p(probs)), "decode_attn_probs")
    return out, probs


def h2o_decode_scores(acc: np.ndarray, probs: np.ndarray) -> np.ndarray:
    """[Walkthrough §3.1] cumulative attention, one decode step at a time: the score of
    token i grows by the weight this step's query puts on it.  READING (GQA): the query
    heads that share a KV head are that head's observations in the step, so their weights
    add up.  acc [B][H][T], probs [B][Hq][T] (consecutive query heads share a KV head);
    fp64."""
    B, H, T = acc.shape
    G = probs.shape[1] // H
    grouped = np.asarray(probs, np.float64).reshape(B, H, G, T)
    step = np.zeros((B, H, T), np.float64)
    for j in range(G):
        step += grouped[:, :, j]
    return np.asarray(acc, np.float64) + step


def int4_evict(c: dict, keep: np.ndarray, R2: int) -> dict:
    """Eviction on a dense oracle cache dict; keep int32 [B][H][K] -> new cache dict (K tokens, R2 bf16)."""
    keep = np.ascontiguousarray(keep, np.int32)
    B, T, H, d, g, R = (c[k] for k in ("B", "T", "H", "d", "g", "R"))
    K = keep.shape[-1]
    Tq2 = K - R2
    nKg2 = -(-Tq2 // g) if Tq2 > 0 else 0
    o = dict(
        k_codes=np.zeros((B, H, Tq2, d // 2), np.uint8),
        k_scale=np.zeros((B, H, nKg2, d), np.uint16),
        k_zero=np.zeros((B, H, nKg2, d), np.uint16),
        v_codes=np.zeros((B, H, Tq2, d // 2), np.uint8),
        v_scale=np.zeros((B, H, Tq2, d // g), np.uint16),
        v_zero=np.zeros((B, H, Tq2, d // g), np.uint16),
        k_res=np.zeros((B, H, R2, d), np.uint16),
        v_res=np.zeros((B, H, R2, d), np.uint16),
    )
    rc = lib().orc_int4_evict(*_cache_ptrs(c), B, T, H, d, g, R, _p(keep), K, R2,
                              *[_p(o[k]) for k in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale",
                                                   "v_zero", "k_res", "v_res")])
    _check(rc, "int4_evict")
    o.update(B=B, T=K, H=H, d=d, g=g, R=R2)
    return o


# -------------------------------------------------------------- selection ---

def keep_count(T, budget, window) -> int:
    return int(lib().orc_keep_count(T, budget, window))


def colsum(hist: np.ndarray):
    hist = np.ascontiguousarray(hist, np.float32)
    rows, T_obs, T = hist.shape
    out = np.empty((rows, T), np.float32)
    lib().orc_colsum(_p(hist), rows, T_obs, T, _p(out))
    return out


def select(scores: np.ndarray, budget: int, window: int):
    scores = np.ascontiguousarray(scores, np.float32)
    if scores.ndim == 1:
        scores = scores[None]
    rows, T = scores.shape
    K = keep_count(T, budget, window)
    keep = np.empty((rows, K), np.int32)
    _check(lib().orc_select(_p(scores), rows, T, budget, window, _p(keep)), "select")
    return keep


def h2o_select(hist: np.ndarray, budget: int, window: int):
    hist = np.ascontiguousarray(hist, np.float32)
    rows, T_obs, T = hist.shape
    K = keep_count(T, budget, window)
    keep = np.empty((rows, K), np.int32)
    scores = np.empty((rows, T), np.float32)
    _check(lib().orc_h2o_select(_p(hist), rows, T_obs, T, budget, window, _p(scores), _p(keep)), "h2o_select")
    return keep, scores


def compact(src: np.ndarray, keep: np.ndarray):
    """src bf16-as-uint16 [B][T][H][d], keep int32 [B][H][K] -> [B][K][H][d]."""
    src = np.ascontiguousarray(src, np.uint16)
    keep = np.ascontiguousarray(keep, np.int32)
    B, T, H, d = src.shape
    K = keep.shape[-1]
    dst = np.empty((B, K, H, d), np.uint16)
    lib().orc_compact(_p(src), B, T, H, d, _p(keep), K, _p(dst))
    return dst


# ----------------------------------------------- Hadamard-rotated cache ---

def _signs(s, d):
    s = np.ascontiguousarray(s, np.int8)
    if s.shape != (d,) or not np.all(np.abs(s.astype(np.int64)) == 1):
        raise ValueError("signs must be d entries in {+1, -1}")
    return s


def rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """fp32 rows [..., d] -> (1/sqrt(d)) H (signs * x), fp32 butterflies in the fixed order."""
    x = np.ascontiguousarray(x, np.float32)
    d = x.shape[-1]
    s = _signs(signs, d)
    y = np.empty_like(x)
    lib().orc_rotate_f32(_p(x), _p(s), x.size // d, d, _p(y))
    return y


def unrotate(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    d = y.shape[-1]
    s = _signs(signs, d)
    x = np.empty_like(y)
    lib().orc_unrotate_f32(_p(y), _p(s), y.size // d, d, _p(x))
    return x


def rot_quant(K: np.ndarray, V: np.ndarray, g: int, k_signs, v_signs) -> dict:
    """K, V bf16-as-uint16 [B][T][H][d] -> rotated per-token 4-bit cache dict."""
    K = np.ascontiguousarray(K, np.uint16)
    V = np.ascontiguousarray(V, np.uint16)
    B, T, H, d = K.shape
    ks, vs = _signs(k_signs, d), _signs(v_signs, d)
    c = dict(k_codes=np.zeros((B, H, T, d // 2), np.uint8), k_scale=np.zeros((B, H, T, d // g), np.uint16),
             k_zero=np.zeros((B, H, T, d // g), np.uint16), v_codes=np.zeros((B, H, T, d // 2), np.uint8),
             v_scale=np.zeros((B, H, T, d // g), np.uint16), v_zero=np.zeros((B, H, T, d // g), np.uint16))
    rc = lib().orc_rot_quant(_p(K), _p(V), B, T, H, d, g, _p(ks), _p(vs),
                             *[_p(c[k]) for k in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")])
    _check(rc, "rot_quant")
    c.update(B=B, T=T, H=H, d=d, g=g, k_signs=ks.copy(), v_signs=vs.copy())
    return c


def rot_dequant(c: dict, side: str) -> np.ndarray:
    """One side back in the original coordinates, fp32 [B][T][H][d]."""
    B, T, H, d, g = (c[k] for k in ("B", "T", "H", "d", "g"))
    s = side.lower()
    out = np.empty((B, T, H, d), np.float32)
    lib().orc_rot_dequant(_p(c[s + "_codes"]), _p(c[s + "_scale"]), _p(c[s + "_zero"]), _p(c[s + "_signs"]),
                          B, T, H, d, g, _p(out))
    return out


def rot_decode_attn(c: dict, q: np.ndarray, sm_scale: float = 1.0) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint16)
    B, Hq, d = q.shape
    out = np.empty((B, Hq, d), np.float64)
    rc = lib().orc_rot_decode_attn(*[_p(c[k]) for k in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale",
                                                         "v_zero", "k_signs", "v_signs")],
                                   c["B"], c["T"], c["H"], c["d"], c["g"], _p(q), Hq, float(sm_scale), _p(out))
    _check(rc, "rot_decode_attn")
    return out


# ---------------------------------------------- per-token mixed precision ---

MIXED_BITS = (2, 4, 8, 16)   # tag 0, 1, 2, 3


def pack_tags(tags: np.ndarray) -> np.ndarray:
    """tag values 0..3 per row -> packed bytes (row r in bits 2(r%4) of byte r/4)."""
    t = np.asarray(tags, np.uint8) & 3
    n = len(t)
    pad = np.zeros(-(-n // 4) * 4, np.uint8)
    pad[:n] = t
    q = pad.reshape(-1, 4)
    return (q[:, 0] | (q[:, 1] << 2) | (q[:, 2] << 4) | (q[:, 3] << 6)).astype(np.uint8)


def mixed_plan(tags_packed: np.ndarray, N: int):
    tags_packed = np.ascontiguousarray(tags_packed, np.uint8)
    slot = np.empty(N, np.int32)
    counts = np.empty(4, np.int64)
    lib().orc_mixed_plan(_p(tags_packed), N, _p(slot), _p(counts))
    return slot, counts


def mixed_quant(x: np.ndarray, tags_packed: np.ndarray) -> dict:
    """x bf16-as-uint16 [N][C] -> dict with the slot plan, the counts and the four pools."""
    x = np.ascontiguousarray(x, np.uint16)
    N, Cc = x.shape
    tags_packed = np.ascontiguousarray(tags_packed, np.uint8)
    slot, counts = mixed_plan(tags_packed, N)
    n2, n4, n8, n16 = (int(v) for v in counts)
    m = dict(q2=np.zeros((n2, Cc // 4), np.uint8), s2=np.zeros(n2, np.float32),
             q4=np.zeros((n4, Cc // 2), np.uint8), s4=np.zeros(n4, np.float32),
             q8=np.zeros((n8, Cc), np.int8), s8=np.zeros(n8, np.float32), z8=np.zeros(n8, np.int8),
             x16=np.zeros((n16, Cc), np.uint16))
    rc = lib().orc_mixed_quant(_p(x), N, Cc, _p(tags_packed), _p(slot),
                               *[_p(m[k]) for k in ("q2", "s2", "q4", "s4", "q8", "s8", "z8", "x16")])
    _check(rc, "mixed_quant")
    m.update(N=N, C=Cc, tags=tags_packed, slot=slot, counts=counts)
    return m


def mixed_dequant(m: dict) -> np.ndarray:
    out = np.empty((m["N"], m["C"]), np.float32)
    lib().orc_mixed_dequant(m["N"], m["C"], _p(m["tags"]), _p(m["slot"]),
                            *[_p(m[k]) for k in ("q2", "s2", "q4", "s4", "q8", "s8", "z8", "x16")], _p(out))
    return out


def mixed_bytes(counts, N: int, Cc: int):
    cnt = np.ascontiguousarray(counts, np.int64)
    out = np.empty(3, np.uint64)
    lib().orc_mixed_bytes(_p(cnt), N, Cc, _p(out))
    return [int(v) for v in out]


# ------------------------------------------------------------- accounting ---

def int4_bytes(N, g) -> int:
    return int(lib().orc_int4_bytes(N, g))


def compression_ratio(orig, data, scale, zp) -> float:
    return float(lib().orc_compression_ratio(orig, data, scale, zp))


def token_ratio(T, K) -> float:
    out = C.c_double()
    _check(lib().orc_token_ratio(T, K, C.byref(out)), "token_ratio")
    return out.value


def total_gain(s_old, s_new, T, K) -> float:
    return float(lib().orc_total_gain(s_old, s_new, T, K))


def kv_bytes(L, T, Cst, b, metadata=0) -> int:
    return int(lib().orc_kv_bytes(L, T, Cst, b, metadata))


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_p(x), x.size, _p(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widening is exact: the bf16 bits become the top half of an fp32."""
    b = np.ascontiguousarray(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)
