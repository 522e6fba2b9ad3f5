"""Thin ctypes binding of libkvq (include/kvq.h).  Argument marshalling only: every step
of the computation runs in the library's HIP kernels.  torch provides device memory
(including the workspaces the library asks for) and the current stream.

The library must be built (``python -m kv_cache_compression_channel_amd.build``); if it
is missing, loading fails loudly -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_EALIGN, KVQ_EHIP = 0, -1, -2, -3
KVQ_FP32, KVQ_BF16 = 0, 1
KVQ_FMT_PER_CHANNEL, KVQ_FMT_INT4_K, KVQ_FMT_INT4_V = 1, 2, 3

EXPORTED = [
    "kvq_last_error", "kvq_abi_version",
    "kvq_quant_pc_ws", "kvq_quant_sym", "kvq_quant_asym",
    "kvq_int4_cache_sizes", "kvq_group_quant_int4", "kvq_int4_append", "kvq_int4_evict", "kvq_dequant",
    "kvq_err_stats_ws", "kvq_err_stats", "kvq_stats_finalize",
    "kvq_compression_ratio", "kvq_int4_bytes", "kvq_token_ratio", "kvq_total_gain", "kvq_kv_bytes",
    "kvq_keep_count",
    "kvq_decode_attn_int4_ws", "kvq_decode_attn_int4", "kvq_decode_attn_int4_h2o_ws", "kvq_decode_attn_int4_h2o",
    "kvq_select_ws", "kvq_h2o_select", "kvq_snapkv_select", "kvq_compact",
    "kvq_rot_cache_sizes", "kvq_rot_quant_int4", "kvq_rot_dequant", "kvq_rot_decode_attn_ws", "kvq_rot_decode_attn",
    "kvq_mixed_plan_ws", "kvq_mixed_plan", "kvq_mixed_quant", "kvq_mixed_dequant", "kvq_mixed_bytes",
    "kvq_bw_probe", "kvq_decode_attn_int4_noalloc",
]


class KVQError(ValueError):
    """A nonzero status from libkvq (KVQ_EINVAL / KVQ_EALIGN / KVQ_EHIP)."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"libkvq status {code}: {msg}")
        self.code = code


class Int4Desc(C.Structure):
    _fields_ = [("B", C.c_int64), ("T", C.c_int64), ("H", C.c_int64), ("d", C.c_int64), ("g", C.c_int64),
                ("R", C.c_int64),
                ("k_codes", C.c_void_p), ("k_scale", C.c_void_p), ("k_zero", C.c_void_p),
                ("v_codes", C.c_void_p), ("v_scale", C.c_void_p), ("v_zero", C.c_void_p),
                ("k_res", C.c_void_p), ("v_res", C.c_void_p), ("cap", C.c_int64), ("rcap", C.c_int64)]


class RotDesc(C.Structure):
    _fields_ = [("B", C.c_int64), ("T", C.c_int64), ("H", C.c_int64), ("d", C.c_int64), ("g", C.c_int64),
                ("k_codes", C.c_void_p), ("k_scale", C.c_void_p), ("k_zero", C.c_void_p),
                ("v_codes", C.c_void_p), ("v_scale", C.c_void_p), ("v_zero", C.c_void_p)]


class MixedDesc(C.Structure):
    _fields_ = [("N", C.c_int64), ("C", C.c_int64), ("tags", C.c_void_p), ("slot", C.c_void_p),
                ("cap", C.c_int64 * 4),
                ("q2", C.c_void_p), ("s2", C.c_void_p), ("q4", C.c_void_p), ("s4", C.c_void_p),
                ("q8", C.c_void_p), ("s8", C.c_void_p), ("z8", C.c_void_p), ("x16", C.c_void_p)]


class PcDesc(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scale", C.c_void_p), ("zp", C.c_void_p),
                ("nb", C.c_int64), ("R", C.c_int64), ("C", C.c_int64)]


class QDesc(C.Structure):
    _fields_ = [("kind", C.c_int), ("desc", C.c_void_p)]


_lib = None


def lib():
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libkvq.so is not built ({LIB_PATH}); run python -m kv_cache_compression_channel_amd.build")
    L = C.CDLL(LIB_PATH)
    P, I, I64, SZ, D = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.c_double
    L.kvq_last_error.restype = C.c_char_p
    L.kvq_abi_version.restype = I
    L.kvq_quant_pc_ws.argtypes = [I64, I64, I64]
    L.kvq_quant_pc_ws.restype = SZ
    L.kvq_quant_sym.argtypes = [P, I, I64, I64, I64, I64, I64, I, P, P, P, P, SZ, P]
    L.kvq_quant_asym.argtypes = [P, I, I64, I64, I64, I64, I64, I, I, P, P, P, P, SZ, P]
    L.kvq_int4_cache_sizes.argtypes = [I64] * 6 + [P, P]
    L.kvq_group_quant_int4.argtypes = [P, P, P, P]
    L.kvq_int4_append.argtypes = [P, P, P, I64, I64, P]
    L.kvq_int4_evict.argtypes = [P, P, P, P]
    L.kvq_rot_cache_sizes.argtypes = [I64] * 5 + [P, P]
    L.kvq_mixed_plan_ws.argtypes = [I64]
    L.kvq_mixed_plan_ws.restype = SZ
    L.kvq_mixed_plan.argtypes = [P, I64, P, P, P, SZ, P]
    L.kvq_mixed_quant.argtypes = [P, P, P]
    L.kvq_mixed_dequant.argtypes = [P, P, I, P]
    L.kvq_mixed_bytes.argtypes = [P, I64, I64, P]
    L.kvq_rot_quant_int4.argtypes = [P, P, P, P, P, P]
    L.kvq_rot_dequant.argtypes = [P, I, P, P, I, P]
    L.kvq_rot_decode_attn_ws.argtypes = [P, I64]
    L.kvq_rot_decode_attn_ws.restype = SZ
    L.kvq_rot_decode_attn.argtypes = [P, P, P, P, I64, C.c_float, P, I, P, SZ, P]
    L.kvq_dequant.argtypes = [P, P, I, P]
    L.kvq_err_stats_ws.argtypes = [I64]
    L.kvq_err_stats_ws.restype = SZ
    L.kvq_err_stats.argtypes = [P, I, P, I, I64, P, P, SZ, P]
    L.kvq_stats_finalize.argtypes = [P, I64, P, P, P]
    L.kvq_compression_ratio.argtypes = [C.c_uint64] * 4
    L.kvq_compression_ratio.restype = D
    L.kvq_int4_bytes.argtypes = [C.c_uint64, C.c_uint64]
    L.kvq_int4_bytes.restype = C.c_uint64
    L.kvq_token_ratio.argtypes = [I64, I64, P]
    L.kvq_total_gain.argtypes = [D, D, I64, I64, P]
    L.kvq_kv_bytes.argtypes = [C.c_uint64] * 5
    L.kvq_kv_bytes.restype = C.c_uint64
    L.kvq_keep_count.argtypes = [I64, I64, I64]
    L.kvq_keep_count.restype = I64
    L.kvq_decode_attn_int4_ws.argtypes = [P, I64]
    L.kvq_decode_attn_int4_ws.restype = SZ
    L.kvq_decode_attn_int4.argtypes = [P, P, I64, C.c_float, P, I, P, SZ, P]
    L.kvq_decode_attn_int4_h2o_ws.argtypes = [P, I64]
    L.kvq_decode_attn_int4_h2o_ws.restype = SZ
    L.kvq_decode_attn_int4_h2o.argtypes = [P, P, I64, C.c_float, P, I, P, I64, P, SZ, P]
    L.kvq_select_ws.argtypes = [I64, I64]
    L.kvq_select_ws.restype = SZ
    L.kvq_h2o_select.argtypes = [P, I64, I64, I64, I64, I64, P, P, P, SZ, P]
    L.kvq_snapkv_select.argtypes = [P, I64, I64, I64, I64, P, P, SZ, P]
    L.kvq_compact.argtypes = [P, P, I64, I64, I64, I64, P, I64, P, P, P]
    L.kvq_bw_probe.argtypes = [P, C.c_uint64, P, C.c_uint64, I, I, P]
    L.kvq_decode_attn_int4_noalloc.argtypes = [P, P, I64, C.c_float, P, I, P]
    _lib = L
    return L


def _check(rc: int):
    if rc != KVQ_OK:
        raise KVQError(rc, lib().kvq_last_error().decode())


def _stream(t: torch.Tensor):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KVQ_FP32
    if t.dtype == torch.bfloat16:
        return KVQ_BF16
    raise TypeError(f"libkvq takes float32 or bfloat16 tensors, got {t.dtype}")


def _ws(nbytes: int, device, ws: torch.Tensor | None = None):
    if nbytes == 0:
        return None, 0
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws, ws.numel() * ws.element_size()
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return t, nbytes


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libkvq tensors must live on the GPU")


# ------------------------------------------------------------- per-channel --

def _pc_view(x: torch.Tensor):
    """[nb][R][C] view of x with its row and slice strides (elements); channels dense."""
    x3 = x if x.dim() == 3 else x.reshape(1, *x.shape[-2:])
    nb, R, Cc = x3.shape
    if Cc > 1 and x3.stride(2) != 1:
        raise ValueError("channels must be the innermost, dense dimension")
    ldx = x3.stride(1) if R > 1 else Cc
    bsx = x3.stride(0) if nb > 1 else R * ldx
    return x3, ldx, bsx


def quant_pc_ws_bytes(nb, R, Cc) -> int:
    return int(lib().kvq_quant_pc_ws(nb, R, Cc))


def _pc_outs(x: torch.Tensor, nb, R, Cc, out, need_zp: bool):
    """Caller-supplied (q, scale, zp) checked for shape and dtype, or new ones."""
    if out is None:
        q = torch.empty((nb, R, Cc), dtype=torch.int8, device=x.device)
        s = torch.empty((nb, Cc), dtype=torch.float32, device=x.device)
        z = torch.empty((nb, Cc), dtype=torch.int8, device=x.device) if need_zp else None
        return q, s, z
    q, s, z = out
    _need_cuda(q, s, z)
    if q.dtype != torch.int8 or q.numel() != nb * R * Cc or not q.is_contiguous():
        raise ValueError("q must be a contiguous int8 tensor of nb * R * C elements")
    if s.dtype != torch.float32 or s.numel() != nb * Cc or not s.is_contiguous():
        raise ValueError("scale must be a contiguous fp32 tensor of nb * C elements")
    if z is not None and (z.dtype != torch.int8 or z.numel() != nb * Cc or not z.is_contiguous()):
        raise ValueError("zp must be a contiguous int8 tensor of nb * C elements")
    if need_zp and z is None:
        raise ValueError("the asymmetric quantizer needs a zp tensor")
    return q, s, z


def quant_sym(x: torch.Tensor, bits: int = 8, ws=None, with_zp: bool = True, out=None):
    """x: [nb][R][C] (or [R][C]) fp32/bf16 on the GPU, rows = tokens, columns = channels.
    Returns (q int8 [nb][R][C], scale fp32 [nb][C], zp int8 [nb][C] of zeros or None).
    out: optional caller-owned (q, scale, zp) to write into (zp may be None)."""
    _need_cuda(x)
    x3, ldx, bsx = _pc_view(x)
    nb, R, Cc = x3.shape
    q, s, z = _pc_outs(x, nb, R, Cc, out, with_zp)
    w, wb = _ws(quant_pc_ws_bytes(nb, R, Cc), x.device, ws)
    _check(lib().kvq_quant_sym(_p(x3), _dt(x3), nb, R, Cc, ldx, bsx, bits, _p(q), _p(s), _p(z), _p(w), wb,
                               _stream(x)))
    return q, s, z


def quant_asym(x: torch.Tensor, qmin: int = -128, qmax: int = 127, ws=None, out=None):
    """As quant_sym, with codes in [qmin, qmax] and an int8 zero point per channel."""
    _need_cuda(x)
    x3, ldx, bsx = _pc_view(x)
    nb, R, Cc = x3.shape
    q, s, z = _pc_outs(x, nb, R, Cc, out, True)
    w, wb = _ws(quant_pc_ws_bytes(nb, R, Cc), x.device, ws)
    _check(lib().kvq_quant_asym(_p(x3), _dt(x3), nb, R, Cc, ldx, bsx, qmin, qmax, _p(q), _p(s),
                                _p(z), _p(w), wb, _stream(x)))
    return q, s, z


def dequant_pc(q: torch.Tensor, scale: torch.Tensor, zp, out_dtype=torch.float32, out=None):
    _need_cuda(q, scale, zp)
    nb, R, Cc = q.shape
    if out is None:
        out = torch.empty((nb, R, Cc), dtype=out_dtype, device=q.device)
    desc = PcDesc(q.data_ptr(), scale.data_ptr(), zp.data_ptr() if zp is not None else None, nb, R, Cc)
    qd = QDesc(KVQ_FMT_PER_CHANNEL, C.cast(C.pointer(desc), C.c_void_p))
    _check(lib().kvq_dequant(C.byref(qd), _p(out), _dt(out), _stream(q)))
    return out


# -------------------------------------------------------------------- INT4 --

def int4_cache_sizes(B, T, H, d, g, R):
    sect = (C.c_size_t * 8)()
    tot = C.c_size_t()
    _check(lib().kvq_int4_cache_sizes(B, T, H, d, g, R, sect, C.byref(tot)))
    return [int(v) for v in sect], int(tot.value)


@dataclass
class Int4Cache:
    """The eight sections of a KIVI-style INT4 cache (device tensors) and its shape."""
    B: int
    T: int
    H: int
    d: int
    g: int
    R: int
    k_codes: torch.Tensor
    k_scale: torch.Tensor
    k_zero: torch.Tensor
    v_codes: torch.Tensor
    v_scale: torch.Tensor
    v_zero: torch.Tensor
    k_res: torch.Tensor
    v_res: torch.Tensor
    cap: int = 0     # quantized-token rows per (b, h) in the sections (0: dense, T - R)
    rcap: int = 0    # residual rows per (b, h) in the sections (0: dense, R)

    SECTIONS = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_res", "v_res")

    @staticmethod
    def empty(B, T, H, d, g, R, device):
        Tq = T - R
        nKg = -(-Tq // g) if Tq > 0 else 0
        u8, bf = torch.uint8, torch.bfloat16

        def e(shape, dt):
            return torch.empty(shape, dtype=dt, device=device)
        return Int4Cache(B, T, H, d, g, R,
                         e((B, H, Tq, d // 2), u8), e((B, H, nKg, d), bf), e((B, H, nKg, d), bf),
                         e((B, H, Tq, d // 2), u8), e((B, H, Tq, d // g), bf), e((B, H, Tq, d // g), bf),
                         e((B, H, R, d), bf), e((B, H, R, d), bf))

    @staticmethod
    def empty_stream(B, H, d, g, cap, rcap, device):
        """An empty growable cache: sections sized for cap quantized and rcap residual tokens."""
        u8, bf = torch.uint8, torch.bfloat16

        def e(shape, dt):
            return torch.empty(shape, dtype=dt, device=device)
        nKg = -(-cap // g)
        return Int4Cache(B, 0, H, d, g, 0,
                         e((B, H, cap, d // 2), u8), e((B, H, nKg, d), bf), e((B, H, nKg, d), bf),
                         e((B, H, cap, d // 2), u8), e((B, H, cap, d // g), bf), e((B, H, cap, d // g), bf),
                         e((B, H, rcap, d), bf), e((B, H, rcap, d), bf), cap, rcap)

    def valid(self, section: str) -> torch.Tensor:
        """The rows of a section in use (all of it for a dense cache)."""
        t = getattr(self, section)
        Tq = self.T - self.R
        if section in ("k_scale", "k_zero"):
            return t[:, :, :-(-Tq // self.g) if Tq > 0 else 0]
        if section in ("k_res", "v_res"):
            return t[:, :, :self.R]
        return t[:, :, :Tq]

    def desc(self) -> Int4Desc:
        def p(t):
            return t.data_ptr() if t.numel() else None
        return Int4Desc(self.B, self.T, self.H, self.d, self.g, self.R,
                        p(self.k_codes), p(self.k_scale), p(self.k_zero), p(self.v_codes), p(self.v_scale),
                        p(self.v_zero), p(self.k_res), p(self.v_res), self.cap, self.rcap)

    def nbytes(self) -> int:
        return sum(getattr(self, s).numel() * getattr(self, s).element_size() for s in self.SECTIONS)


def group_quant_int4(K: torch.Tensor, V: torch.Tensor, g: int = 64, R: int = 128, cache: Int4Cache | None = None):
    """K, V bf16 [B][T][H][d] on the GPU -> Int4Cache (codes, bf16 scale/zero, bf16 residual)."""
    _need_cuda(K, V)
    if K.dtype != torch.bfloat16 or V.dtype != torch.bfloat16:
        raise TypeError("K and V must be bfloat16")
    if K.shape != V.shape or K.dim() != 4 or not K.is_contiguous() or not V.is_contiguous():
        raise ValueError("K and V must be contiguous [B][T][H][d] of the same shape")
    B, T, H, d = K.shape
    if cache is None:
        cache = Int4Cache.empty(B, T, H, d, g, R, K.device)
    desc = cache.desc()
    _check(lib().kvq_group_quant_int4(_p(K), _p(V), C.byref(desc), _stream(K)))
    return cache


def int4_append(cache: Int4Cache, k_new: torch.Tensor, v_new: torch.Tensor, r_keep: int) -> Int4Cache:
    """Append n <= g tokens (bf16 [B][n][H][d]) to a growable cache in place; flushes the oldest g
    residual tokens to INT4 when the residual reaches r_keep + g.  Updates cache.T and cache.R."""
    _need_cuda(k_new, v_new)
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise TypeError("k_new and v_new must be bfloat16")
    if k_new.shape != v_new.shape or k_new.dim() != 4 or not k_new.is_contiguous() or not v_new.is_contiguous():
        raise ValueError("k_new and v_new must be contiguous [B][n][H][d] of the same shape")
    if (k_new.shape[0], k_new.shape[2], k_new.shape[3]) != (cache.B, cache.H, cache.d):
        raise ValueError("k_new does not match the cache's B, H, d")
    desc = cache.desc()
    _check(lib().kvq_int4_append(C.byref(desc), _p(k_new), _p(v_new), k_new.shape[1], r_keep, _stream(k_new)))
    cache.T, cache.R = int(desc.T), int(desc.R)
    return cache


def int4_evict(cache: Int4Cache, keep: torch.Tensor, r2: int, out: Int4Cache | None = None) -> Int4Cache:
    """Keep the tokens keep[b][h][:] (int32 [B][H][K], indices into the cache's T tokens) of every
    (b, h): a new cache of K tokens whose last r2 are bf16.  Kept V rows and whole kept K groups
    are copied; other K groups are requantized from their current values.  ``out`` (dense or
    growable, not overlapping ``cache``) receives the result; its T and R become K and r2."""
    _need_cuda(keep)
    if keep.dtype != torch.int32 or keep.dim() != 3 or not keep.is_contiguous():
        raise ValueError("keep must be contiguous int32 [B][H][K]")
    if (keep.shape[0], keep.shape[1]) != (cache.B, cache.H):
        raise ValueError("keep does not match the cache's B, H")
    K = keep.shape[2]
    if out is None:
        out = Int4Cache.empty(cache.B, K, cache.H, cache.d, cache.g, r2, keep.device)
        sd, dd = cache.desc(), out.desc()
    else:
        before = (out.T, out.R)
        out.T, out.R = K, r2
        sd, dd = cache.desc(), out.desc()
        out.T, out.R = before
    _check(lib().kvq_int4_evict(C.byref(sd), _p(keep), C.byref(dd), _stream(keep)))
    out.T, out.R = K, r2
    return out


def dequant_int4(cache: Int4Cache, side: str, out_dtype=torch.bfloat16, out=None):
    kind = KVQ_FMT_INT4_K if side.lower() == "k" else KVQ_FMT_INT4_V
    dev = cache.k_codes.device if cache.k_codes.numel() else cache.k_res.device
    if out is None:
        out = torch.empty((cache.B, cache.T, cache.H, cache.d), dtype=out_dtype, device=dev)
    desc = cache.desc()
    qd = QDesc(kind, C.cast(C.pointer(desc), C.c_void_p))
    _check(lib().kvq_dequant(C.byref(qd), _p(out), _dt(out), _stream(out)))
    return out


# ----------------------------------------------- Hadamard-rotated cache --

@dataclass
class RotCache:
    """Per-token 4-bit codes of Hadamard-rotated K and V (device tensors) and their shape."""
    B: int
    T: int
    H: int
    d: int
    g: int
    k_codes: torch.Tensor
    k_scale: torch.Tensor
    k_zero: torch.Tensor
    v_codes: torch.Tensor
    v_scale: torch.Tensor
    v_zero: torch.Tensor

    SECTIONS = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")

    @staticmethod
    def empty(B, T, H, d, g, device):
        def e(shape, dt):
            return torch.empty(shape, dtype=dt, device=device)
        u8, bf = torch.uint8, torch.bfloat16
        return RotCache(B, T, H, d, g, e((B, H, T, d // 2), u8), e((B, H, T, d // g), bf), e((B, H, T, d // g), bf),
                        e((B, H, T, d // 2), u8), e((B, H, T, d // g), bf), e((B, H, T, d // g), bf))

    def desc(self) -> RotDesc:
        return RotDesc(self.B, self.T, self.H, self.d, self.g, *[getattr(self, s).data_ptr() for s in self.SECTIONS])

    def nbytes(self) -> int:
        return sum(getattr(self, s).numel() * getattr(self, s).element_size() for s in self.SECTIONS)


def _signs_host(s, d) -> torch.Tensor:
    t = torch.as_tensor(s, dtype=torch.int8).contiguous().cpu()
    if t.shape != (d,):
        raise ValueError(f"signs must have d = {d} entries")
    return t


def rot_quant_int4(K: torch.Tensor, V: torch.Tensor, g: int, k_signs, v_signs, cache: RotCache | None = None):
    """K, V bf16 [B][T][H][d] -> RotCache (each row rotated by (1/sqrt(d)) H diag(signs), then
    per-token 4-bit groups of g).  Signs: d host values in {+1, -1} per side."""
    _need_cuda(K, V)
    if K.dtype != torch.bfloat16 or V.dtype != torch.bfloat16 or K.shape != V.shape or K.dim() != 4 \
            or not K.is_contiguous() or not V.is_contiguous():
        raise ValueError("K and V must be contiguous bfloat16 [B][T][H][d] of the same shape")
    B, T, H, d = K.shape
    ks, vs = _signs_host(k_signs, d), _signs_host(v_signs, d)
    if cache is None:
        cache = RotCache.empty(B, T, H, d, g, K.device)
    desc = cache.desc()
    _check(lib().kvq_rot_quant_int4(_p(K), _p(V), ks.data_ptr(), vs.data_ptr(), C.byref(desc), _stream(K)))
    return cache


def rot_dequant(cache: RotCache, side: str, signs, out_dtype=torch.bfloat16, out=None):
    """One side back in the original coordinates, [B][T][H][d]."""
    if out is None:
        out = torch.empty((cache.B, cache.T, cache.H, cache.d), dtype=out_dtype, device=cache.k_codes.device)
    sg = _signs_host(signs, cache.d)
    desc = cache.desc()
    _check(lib().kvq_rot_dequant(C.byref(desc), 0 if side.lower() == "k" else 1, sg.data_ptr(), _p(out), _dt(out),
                                 _stream(out)))
    return out


def rot_decode_attn(cache: RotCache, q: torch.Tensor, k_signs, v_signs, sm_scale: float = 1.0, out=None, ws=None,
                    out_dtype=torch.bfloat16):
    """GQA decode attention over the rotated cache; q bf16 [B][Hq][d] -> out [B][Hq][d]."""
    _need_cuda(q)
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise TypeError("q must be a contiguous bfloat16 [B][Hq][d] tensor")
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
    ks, vs = _signs_host(k_signs, d), _signs_host(v_signs, d)
    desc = cache.desc()
    w, wb = _ws(int(lib().kvq_rot_decode_attn_ws(C.byref(desc), Hq)), q.device, ws)
    _check(lib().kvq_rot_decode_attn(C.byref(desc), ks.data_ptr(), vs.data_ptr(), _p(q), Hq, float(sm_scale), _p(out),
                                     _dt(out), _p(w), wb, _stream(q)))
    return out


def rot_attn_ws_bytes(cache: RotCache, Hq: int) -> int:
    desc = cache.desc()
    return int(lib().kvq_rot_decode_attn_ws(C.byref(desc), Hq))


# ---------------------------------------------- per-token mixed precision --

@dataclass
class MixedStore:
    """Rows of N x C at 2/4/8/16 bits per their tags: the plan (slot, counts) and the four pools."""
    N: int
    C: int
    tags: torch.Tensor      # uint8 [ceil(N/4)], four 2-bit tags per byte
    slot: torch.Tensor      # int32 [N]
    cap: tuple
    q2: torch.Tensor
    s2: torch.Tensor
    q4: torch.Tensor
    s4: torch.Tensor
    q8: torch.Tensor
    s8: torch.Tensor
    z8: torch.Tensor
    x16: torch.Tensor

    POOLS = ("q2", "s2", "q4", "s4", "q8", "s8", "z8", "x16")

    def desc(self) -> MixedDesc:
        def p(t):
            return t.data_ptr() if t.numel() else None
        d = MixedDesc(self.N, self.C, self.tags.data_ptr(), self.slot.data_ptr())
        for i in range(4):
            d.cap[i] = int(self.cap[i])
        for f in self.POOLS:
            setattr(d, f, p(getattr(self, f)))
        return d

    def nbytes(self) -> int:
        return sum(getattr(self, f).numel() * getattr(self, f).element_size() for f in self.POOLS)


def mixed_plan(tags: torch.Tensor, N: int, slot=None, counts=None, ws=None):
    """Slots (int32 [N]) and rows per tag (int64 [4]) on the device."""
    _need_cuda(tags)
    if slot is None:
        slot = torch.empty(N, dtype=torch.int32, device=tags.device)
    if counts is None:
        counts = torch.empty(4, dtype=torch.int64, device=tags.device)
    w, wb = _ws(int(lib().kvq_mixed_plan_ws(N)), tags.device, ws)
    _check(lib().kvq_mixed_plan(_p(tags), N, _p(slot), _p(counts), _p(w), wb, _stream(tags)))
    return slot, counts


def mixed_store_empty(N: int, Cc: int, tags: torch.Tensor, slot: torch.Tensor, cap, device) -> MixedStore:
    n2, n4, n8, n16 = (int(v) for v in cap)

    def e(shape, dt):
        return torch.empty(shape, dtype=dt, device=device)
    return MixedStore(N, Cc, tags, slot, (n2, n4, n8, n16), e((n2, Cc // 4), torch.uint8), e(n2, torch.float32),
                      e((n4, Cc // 2), torch.uint8), e(n4, torch.float32), e((n8, Cc), torch.int8), e(n8, torch.float32),
                      e(n8, torch.int8), e((n16, Cc), torch.bfloat16))


def mixed_quant(x: torch.Tensor, store: MixedStore) -> MixedStore:
    """x bf16 [N][C] -> the store's pools (slots and capacities as planned)."""
    _need_cuda(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous() or tuple(x.shape) != (store.N, store.C):
        raise ValueError("x must be contiguous bfloat16 [N][C] matching the store")
    d = store.desc()
    _check(lib().kvq_mixed_quant(_p(x), C.byref(d), _stream(x)))
    return store


def mixed_quantize(x: torch.Tensor, tags: torch.Tensor) -> MixedStore:
    """Plan, size the pools from the counts (one device-to-host copy), quantize."""
    N, Cc = x.shape
    slot, counts = mixed_plan(tags, N)
    cap = [int(v) for v in counts.cpu()]
    return mixed_quant(x, mixed_store_empty(N, Cc, tags, slot, cap, x.device))


def mixed_dequant(store: MixedStore, out_dtype=torch.bfloat16, out=None):
    if out is None:
        out = torch.empty((store.N, store.C), dtype=out_dtype, device=store.slot.device)
    d = store.desc()
    _check(lib().kvq_mixed_dequant(C.byref(d), _p(out), _dt(out), _stream(out)))
    return out


# ------------------------------------------------------------------- stats --

def err_stats(x: torch.Tensor, xh: torch.Tensor, out=None, ws=None) -> torch.Tensor:
    """-> fp64 device tensor [sum (x-xh)^2, sum |x-xh|, max |x-xh|]."""
    _need_cuda(x, xh)
    if not (x.is_contiguous() and xh.is_contiguous()):
        raise ValueError("err_stats reads x and x_hat as dense arrays; pass contiguous tensors")
    n = x.numel()
    if xh.numel() != n:
        raise ValueError("x and x_hat differ in size")
    if out is None:
        out = torch.empty(3, dtype=torch.float64, device=x.device)
    w, wb = _ws(int(lib().kvq_err_stats_ws(n)), x.device, ws)
    _check(lib().kvq_err_stats(_p(x), _dt(x), _p(xh), _dt(xh), n, _p(out), _p(w), wb, _stream(x)))
    return out


def stats_finalize(raw, n: int):
    a = (C.c_double * 3)(*[float(v) for v in raw])
    r, m, mean = C.c_double(), C.c_double(), C.c_double()
    _check(lib().kvq_stats_finalize(a, n, C.byref(r), C.byref(m), C.byref(mean)))
    return r.value, m.value, mean.value


def compression_ratio(orig, data, scale, zp) -> float:
    return float(lib().kvq_compression_ratio(orig, data, scale, zp))


def int4_bytes(N, g) -> int:
    return int(lib().kvq_int4_bytes(N, g))


def token_ratio(T, K) -> float:
    out = C.c_double()
    _check(lib().kvq_token_ratio(T, K, C.byref(out)))
    return out.value


def total_gain(s_old, s_new, T, K) -> float:
    out = C.c_double()
    _check(lib().kvq_total_gain(s_old, s_new, T, K, C.byref(out)))
    return out.value


def kv_bytes(L, T, Cst, b, metadata=0) -> int:
    return int(lib().kvq_kv_bytes(L, T, Cst, b, metadata))


def keep_count(T, budget, window) -> int:
    return int(lib().kvq_keep_count(T, budget, window))


# -------------------------------------------------------- decode attention --

def decode_attn_ws_bytes(cache: Int4Cache, Hq: int) -> int:
    desc = cache.desc()
    return int(lib().kvq_decode_attn_int4_ws(C.byref(desc), Hq))


def decode_attn_h2o_ws_bytes(cache: Int4Cache, Hq: int) -> int:
    desc = cache.desc()
    return int(lib().kvq_decode_attn_int4_h2o_ws(C.byref(desc), Hq))


def decode_attn_int4(cache: Int4Cache, q: torch.Tensor, sm_scale: float = 1.0, out=None, ws=None,
                     out_dtype=torch.bfloat16):
    """q bf16 [B][Hq][d] -> out [B][Hq][d] (bf16 = the fp32 result rounded to nearest even, or fp32)."""
    _need_cuda(q)
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise TypeError("q must be a contiguous bfloat16 [B][Hq][d] tensor")
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
    desc = cache.desc()
    w, wb = _ws(int(lib().kvq_decode_attn_int4_ws(C.byref(desc), Hq)), q.device, ws)
    _check(lib().kvq_decode_attn_int4(C.byref(desc), _p(q), Hq, float(sm_scale), _p(out), _dt(out), _p(w), wb,
                                      _stream(q)))
    return out


ATTN_SCRATCH_BYTES = 16 << 20   # KVQ_ATTN_SCRATCH_BYTES


def decode_attn_int4_noalloc(cache: Int4Cache, q: torch.Tensor, sm_scale: float = 1.0, out=None,
                             out_dtype=torch.bfloat16):
    """decode_attn_int4 with the split partials in the library's per-device scratch array instead of a
    workspace (the library call allocates nothing; out is allocated here unless given).  Calls that
    overlap on one GPU race."""
    _need_cuda(q)
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise TypeError("q must be a contiguous bfloat16 [B][Hq][d] tensor")
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
    desc = cache.desc()
    _check(lib().kvq_decode_attn_int4_noalloc(C.byref(desc), _p(q), Hq, float(sm_scale), _p(out), _dt(out),
                                              _stream(q)))
    return out


def decode_attn_int4_h2o(cache: Int4Cache, q: torch.Tensor, acc: torch.Tensor, sm_scale: float = 1.0, out=None,
                         ws=None, out_dtype=torch.bfloat16):
    """Decode attention (as decode_attn_int4) that also adds this step's attention weights to the
    running H2O scores: acc fp32 [B][H][L] with L >= cache.T, updated in place for t < cache.T
    (the weights of the Hq/H query heads of a KV head summed)."""
    _need_cuda(q, acc)
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise TypeError("q must be a contiguous bfloat16 [B][Hq][d] tensor")
    if acc.dtype != torch.float32 or acc.dim() != 3 or not acc.is_contiguous() or \
            acc.shape[0] != cache.B or acc.shape[1] != cache.H:
        raise ValueError("acc must be contiguous float32 [B][H][L]")
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
    desc = cache.desc()
    w, wb = _ws(int(lib().kvq_decode_attn_int4_h2o_ws(C.byref(desc), Hq)), q.device, ws)
    _check(lib().kvq_decode_attn_int4_h2o(C.byref(desc), _p(q), Hq, float(sm_scale), _p(out), _dt(out), _p(acc),
                                          acc.shape[2], _p(w), wb, _stream(q)))
    return out


# --------------------------------------------------------------- selection --

def h2o_select(hist: torch.Tensor, budget: int, window: int, scores: torch.Tensor | None = None,
               keep: torch.Tensor | None = None, ws=None):
    """hist fp32 [rows][T_obs][T] -> keep int32 [rows][K] (scores written when given)."""
    _need_cuda(hist)
    if hist.dtype != torch.float32 or hist.dim() != 3 or not hist.is_contiguous():
        raise TypeError("hist must be a contiguous float32 [rows][T_obs][T] tensor")
    rows, T_obs, T = hist.shape
    K = keep_count(T, budget, window)
    if keep is None:
        keep = torch.empty((rows, max(K, 0)), dtype=torch.int32, device=hist.device)
    w, wb = (None, 0) if scores is not None else _ws(int(lib().kvq_select_ws(rows, T)), hist.device, ws)
    _check(lib().kvq_h2o_select(_p(hist), rows, T_obs, T, budget, window, _p(scores), _p(keep), _p(w), wb,
                                _stream(hist)))
    return keep


def snapkv_select(scores: torch.Tensor, budget: int, window: int, keep: torch.Tensor | None = None):
    _need_cuda(scores)
    if scores.dtype != torch.float32 or not scores.is_contiguous():
        raise TypeError("scores must be a contiguous float32 [rows][T] tensor")
    s2 = scores if scores.dim() == 2 else scores.reshape(1, -1)
    rows, T = s2.shape
    K = keep_count(T, budget, window)
    if keep is None:
        keep = torch.empty((rows, max(K, 0)), dtype=torch.int32, device=scores.device)
    _check(lib().kvq_snapkv_select(_p(s2), rows, T, budget, window, _p(keep), None, 0, _stream(scores)))
    return keep


def compact(k_src: torch.Tensor, v_src: torch.Tensor | None, keep: torch.Tensor, k_dst=None, v_dst=None):
    """k_src, v_src bf16 [B][T][H][d]; keep int32 [B][H][K] -> (k_dst, v_dst) [B][K][H][d]."""
    _need_cuda(k_src, v_src, keep)
    B, T, H, d = k_src.shape
    K = keep.shape[-1]
    if keep.dtype != torch.int32 or tuple(keep.shape) != (B, H, K) or not keep.is_contiguous():
        raise ValueError("keep must be a contiguous int32 [B][H][K] tensor")
    if k_dst is None:
        k_dst = torch.empty((B, K, H, d), dtype=k_src.dtype, device=k_src.device)
    if v_src is not None and v_dst is None:
        v_dst = torch.empty((B, K, H, d), dtype=v_src.dtype, device=v_src.device)
    _check(lib().kvq_compact(_p(k_src), _p(v_src), B, T, H, d, _p(keep), K, _p(k_dst), _p(v_dst), _stream(k_src)))
    return k_dst, v_dst


# ------------------------------------------------------- bandwidth probe --

def bw_probe(src: torch.Tensor | None, read_bytes: int, dst: torch.Tensor, write_bytes: int, nt: bool = True,
             depth: int = 8):
    """Stream read_bytes of src and write_bytes into dst (device buffers) in one of the probe's
    read:write mixes, depth times the mix's accesses per thread; see kvq_bw_probe."""
    _need_cuda(dst)
    if src is not None and src.numel() * src.element_size() < read_bytes:
        raise ValueError("src is smaller than read_bytes")
    if dst.numel() * dst.element_size() < max(write_bytes, 16):
        raise ValueError("dst is smaller than write_bytes (or 16 bytes)")
    _check(lib().kvq_bw_probe(_p(src) if src is not None else None, read_bytes, _p(dst), write_bytes, int(nt),
                              int(depth), _stream(dst)))
