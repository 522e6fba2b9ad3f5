"""CPU tests of the C ABI: the library loads without a GPU, exports every function the
header declares, its host-only helpers agree with the pages' closed forms, and every
argument check fails with KVQ_EINVAL / KVQ_EALIGN before anything is enqueued."""
import ctypes as C
import os
import re

import pytest

from kv_cache_compression_channel_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

FAKE = C.c_void_p(0x100000)        # aligned, never dereferenced: validation fails first
MISALIGNED = C.c_void_p(0x100004)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    return kvq.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), f"{n} declared in kvq.h but not exported"
    assert sorted(kvq.EXPORTED) == names
    assert L.kvq_abi_version() == 1


def test_host_helpers_closed_forms(L):
    assert kvq.int4_bytes(1048576, 64) == 589824
    for g, bpn in ((32, 0.625), (64, 0.5625), (128, 0.53125)):
        assert kvq.int4_bytes(g * 1000, g) == g * 1000 * bpn
    assert kvq.int4_bytes(65, 64) == 41 and kvq.int4_bytes(7, 0) == 0
    assert kvq.compression_ratio(131072, 32768, 512, 128) == 131072 / 33408
    assert kvq.compression_ratio(1, 0, 0, 0) == 0.0
    assert kvq.token_ratio(32768, 2048) == 16.0
    assert kvq.total_gain(2.0, 0.5625, 32768, 2048) == (2.0 / 0.5625) * 16
    assert kvq.kv_bytes(32, 8192, 2 * 32 * 128, 2) == 4 * 2**30
    sect, tot = kvq.int4_cache_sizes(1, 8192, 8, 128, 64, 128)
    assert tot == 9_814_016 and sect == [4128768, 258048, 258048, 4128768, 258048, 258048, 262144, 262144]
    for T, B, W, want in ((32768, 2048, 256, 2048), (100, 200, 10, 100), (100, 5, 10, 10), (5, 0, 0, 0),
                          (10, 3, 20, 10)):
        assert kvq.keep_count(T, B, W) == want
    assert L.kvq_keep_count(0, 1, 1) == -1


def test_host_helpers_match_oracle():
    import oracle
    for T, B, W in ((1, 0, 0), (7, 3, 2), (300, 64, 256), (32768, 2048, 256), (50, 100, 0)):
        assert kvq.keep_count(T, B, W) == oracle.keep_count(T, B, W)
    for B, T, H, d, g, R in ((1, 8192, 8, 128, 64, 128), (4, 100, 2, 64, 32, 7), (2, 128, 3, 256, 128, 128)):
        assert kvq.int4_cache_sizes(B, T, H, d, g, R) == oracle.int4_cache_sizes(B, T, H, d, g, R)
    for N in (1, 63, 64, 65, 10**6 + 3):
        for g in (32, 64, 128):
            assert kvq.int4_bytes(N, g) == oracle.int4_bytes(N, g)


def test_ratio_errors(L):
    for T, K in ((0, 1), (10, 0), (10, 11)):
        with pytest.raises(kvq.KVQError) as e:
            kvq.token_ratio(T, K)
        assert e.value.code == kvq.KVQ_EINVAL
    with pytest.raises(kvq.KVQError):
        kvq.total_gain(2.0, 0.0, 10, 5)


def _rc(fn, *args):
    return fn(*args)


def test_quant_pc_validation(L):
    ws = FAKE
    big = 1 << 30
    cases = [
        (L.kvq_quant_sym, (None, 0, 1, 4, 4, 4, 16, 8, FAKE, FAKE, None, ws, big, None)),      # NULL x
        (L.kvq_quant_sym, (FAKE, 0, 1, 4, 4, 4, 16, 9, FAKE, FAKE, None, ws, big, None)),      # bits 9
        (L.kvq_quant_sym, (FAKE, 0, 1, 4, 4, 4, 16, 1, FAKE, FAKE, None, ws, big, None)),      # bits 1
        (L.kvq_quant_sym, (FAKE, 2, 1, 4, 4, 4, 16, 8, FAKE, FAKE, None, ws, big, None)),      # dtype
        (L.kvq_quant_sym, (FAKE, 0, 0, 4, 4, 4, 16, 8, FAKE, FAKE, None, ws, big, None)),      # nb 0
        (L.kvq_quant_sym, (FAKE, 0, 1, 4, 4, 3, 16, 8, FAKE, FAKE, None, ws, big, None)),      # ldx < C
        (L.kvq_quant_sym, (FAKE, 0, 2, 4, 4, 4, 15, 8, FAKE, FAKE, None, ws, big, None)),      # bsx < R*ldx
        (L.kvq_quant_sym, (FAKE, 0, 1, 4, 4, 4, 16, 8, FAKE, FAKE, None, ws, 8, None)),        # short ws
        (L.kvq_quant_asym, (FAKE, 0, 1, 4, 4, 4, 16, 0, 0, FAKE, FAKE, FAKE, ws, big, None)),  # qmin == qmax
        (L.kvq_quant_asym, (FAKE, 0, 1, 4, 4, 4, 16, -129, 0, FAKE, FAKE, FAKE, ws, big, None)),
        (L.kvq_quant_asym, (FAKE, 0, 1, 4, 4, 4, 16, -128, 127, FAKE, FAKE, None, ws, big, None)),  # no zp
    ]
    for fn, args in cases:
        assert fn(*args) == kvq.KVQ_EINVAL, args
        assert L.kvq_last_error()
    assert L.kvq_quant_sym(MISALIGNED, 0, 1, 4, 4, 4, 16, 8, FAKE, FAKE, None, ws, big, None) == kvq.KVQ_EALIGN


def _desc(**kw):
    base = dict(B=1, T=128, H=2, d=128, g=64, R=0, cap=0, rcap=0)
    base.update(kw)
    d = kvq.Int4Desc(base["B"], base["T"], base["H"], base["d"], base["g"], base["R"])
    for f in kvq.Int4Cache.SECTIONS:
        setattr(d, f, kw.get(f, 0x200000))
    d.cap, d.rcap = base["cap"], base["rcap"]
    return d


def test_int4_growable_layout_validation(L):
    # cap must cover T - R and be a multiple of g; rcap must cover R
    for kw in (dict(cap=64), dict(cap=130), dict(R=100, rcap=50)):
        d = _desc(**kw)
        assert L.kvq_group_quant_int4(FAKE, FAKE, C.byref(d), None) == kvq.KVQ_EINVAL, kw
        assert L.kvq_decode_attn_int4(C.byref(d), FAKE, 2, 1.0, FAKE, 1, FAKE, 1 << 30, None) == kvq.KVQ_EINVAL
    ok = dict(T=192, R=64, cap=256, rcap=256)          # T - R = 128, two groups of 64
    app = L.kvq_int4_append
    cases = [
        (dict(ok, cap=0), 1, 64),                       # dense layout cannot grow
        (dict(ok, rcap=0), 1, 64),
        (dict(ok, T=200), 1, 64),                       # T - R not a multiple of g
        (dict(ok, cap=200), 1, 64),                     # cap not a multiple of g
        (ok, 0, 64),                                    # n = 0
        (ok, 65, 64),                                   # n > g
        (dict(ok, R=128, T=256), 1, 64),                # R >= r_keep + g
        (dict(ok, rcap=64), 1, 64),                     # rcap < R + n
        (dict(ok, cap=128), 64, 64),                    # a flush with the quantized rows full
        (dict(ok, d=96), 1, 64),
        (dict(ok, k_res=None), 1, 64),
    ]
    for kw, n, r_keep in cases:
        d = _desc(**kw)
        T0, R0 = d.T, d.R
        assert app(C.byref(d), FAKE, FAKE, n, r_keep, None) == kvq.KVQ_EINVAL, (kw, n, r_keep)
        assert (d.T, d.R) == (T0, R0), "a rejected append left the descriptor changed"
        assert L.kvq_last_error()
    d = _desc(**ok)
    assert app(C.byref(d), None, FAKE, 1, 64, None) == kvq.KVQ_EINVAL
    assert app(None, FAKE, FAKE, 1, 64, None) == kvq.KVQ_EINVAL
    assert app(C.byref(d), MISALIGNED, FAKE, 1, 64, None) == kvq.KVQ_EALIGN


def test_int4_evict_validation(L):
    src = dict(T=512, R=64)
    far = {f: 0x40000000 + 0x1000000 * i for i, f in enumerate(kvq.Int4Cache.SECTIONS)}
    ev = L.kvq_int4_evict
    cases = [
        (src, dict(far, T=600, R=0)),                 # more kept tokens than src holds
        (src, dict(far, T=128, R=129)),               # R2 > K
        (src, dict(far, T=128, R=0, d=64)),           # d differs
        (src, dict(far, T=128, R=0, g=32)),           # g differs
        (src, dict(far, T=128, R=0, H=3)),            # H differs
        (src, dict(T=128, R=0)),                      # dst sections overlap the src sections
        (src, dict(far, T=128, R=0, cap=64)),         # dst cap below its quantized rows
        (dict(src, cap=100), dict(far, T=128, R=0)),  # src cap not a multiple of g
    ]
    for skw, dkw in cases:
        s_, d_ = _desc(**skw), _desc(**dkw)
        assert ev(C.byref(s_), FAKE, C.byref(d_), None) == kvq.KVQ_EINVAL, (skw, dkw)
        assert L.kvq_last_error()
    s_, d_ = _desc(**src), _desc(**dict(far, T=128, R=0))
    assert ev(C.byref(s_), None, C.byref(d_), None) == kvq.KVQ_EINVAL
    assert ev(None, FAKE, C.byref(d_), None) == kvq.KVQ_EINVAL
    assert ev(C.byref(s_), FAKE, None, None) == kvq.KVQ_EINVAL
    d_ = _desc(**dict(far, T=128, R=0, k_codes=0x40000008))
    assert ev(C.byref(s_), FAKE, C.byref(d_), None) == kvq.KVQ_EALIGN


def test_int4_validation(L):
    bad = [dict(d=96), dict(d=32), dict(g=16), dict(g=256), dict(d=64, g=128), dict(R=129), dict(R=-1),
           dict(B=0), dict(T=0), dict(H=0), dict(k_codes=None), dict(v_zero=None)]
    for kw in bad:
        d = _desc(**kw)
        assert L.kvq_group_quant_int4(FAKE, FAKE, C.byref(d), None) == kvq.KVQ_EINVAL, kw
    d = _desc()
    assert L.kvq_group_quant_int4(None, FAKE, C.byref(d), None) == kvq.KVQ_EINVAL
    assert L.kvq_group_quant_int4(MISALIGNED, FAKE, C.byref(d), None) == kvq.KVQ_EALIGN
    d = _desc(k_scale=0x200008)
    assert L.kvq_group_quant_int4(FAKE, FAKE, C.byref(d), None) == kvq.KVQ_EALIGN
    # residual sections may be NULL only when R == 0, INT4 sections only when T == R
    d = _desc(R=128, k_codes=None, k_scale=None, k_zero=None, v_codes=None, v_scale=None, v_zero=None, k_res=None)
    assert L.kvq_group_quant_int4(FAKE, FAKE, C.byref(d), None) == kvq.KVQ_EINVAL
    sect = (C.c_size_t * 8)()
    tot = C.c_size_t()
    assert L.kvq_int4_cache_sizes(1, 10, 1, 64, 48, 0, sect, C.byref(tot)) == kvq.KVQ_EINVAL


def test_dequant_and_stats_validation(L):
    qd = kvq.QDesc(99, FAKE)
    assert L.kvq_dequant(C.byref(qd), FAKE, 0, None) == kvq.KVQ_EINVAL
    d = _desc(d=100)
    qd = kvq.QDesc(kvq.KVQ_FMT_INT4_K, C.cast(C.pointer(d), C.c_void_p))
    assert L.kvq_dequant(C.byref(qd), FAKE, 0, None) == kvq.KVQ_EINVAL
    d = _desc()
    qd = kvq.QDesc(kvq.KVQ_FMT_INT4_V, C.cast(C.pointer(d), C.c_void_p))
    assert L.kvq_dequant(C.byref(qd), FAKE, 7, None) == kvq.KVQ_EINVAL
    pc = kvq.PcDesc(0x100000, 0x100000, None, 1, 0, 4)
    qd = kvq.QDesc(kvq.KVQ_FMT_PER_CHANNEL, C.cast(C.pointer(pc), C.c_void_p))
    assert L.kvq_dequant(C.byref(qd), FAKE, 0, None) == kvq.KVQ_EINVAL
    assert L.kvq_err_stats(FAKE, 0, FAKE, 0, 0, FAKE, FAKE, 1 << 20, None) == kvq.KVQ_EINVAL
    assert L.kvq_err_stats(FAKE, 0, FAKE, 3, 10, FAKE, FAKE, 1 << 20, None) == kvq.KVQ_EINVAL
    assert L.kvq_err_stats(FAKE, 0, FAKE, 0, 10, FAKE, FAKE, 8, None) == kvq.KVQ_EINVAL
    assert L.kvq_err_stats_ws(0) == 0


def test_attn_validation(L):
    d = _desc(H=8)
    for Hq in (0, 12, 8 * 32):
        assert L.kvq_decode_attn_int4(C.byref(d), FAKE, Hq, 1.0, FAKE, 1, FAKE, 1 << 30, None) == kvq.KVQ_EINVAL
    assert L.kvq_decode_attn_int4(C.byref(d), FAKE, 32, 1.0, FAKE, 1, FAKE, 16, None) == kvq.KVQ_EINVAL
    assert L.kvq_decode_attn_int4(C.byref(d), None, 32, 1.0, FAKE, 1, FAKE, 1 << 30, None) == kvq.KVQ_EINVAL
    assert L.kvq_decode_attn_int4(C.byref(d), FAKE, 32, 1.0, FAKE, 5, FAKE, 1 << 30, None) == kvq.KVQ_EINVAL
    assert L.kvq_decode_attn_int4_ws(None, 4) == 0


def test_attn_h2o_validation(L):
    d = _desc(H=8)                                   # T = 128
    f = L.kvq_decode_attn_int4_h2o
    big = 1 << 30
    assert f(C.byref(d), FAKE, 32, 1.0, FAKE, 1, None, 128, FAKE, big, None) == kvq.KVQ_EINVAL      # NULL acc
    assert f(C.byref(d), FAKE, 32, 1.0, FAKE, 1, FAKE, 127, FAKE, big, None) == kvq.KVQ_EINVAL      # ld_acc < T
    assert f(C.byref(d), FAKE, 32, 1.0, FAKE, 1, MISALIGNED, 128, FAKE, big, None) == kvq.KVQ_EALIGN
    assert f(C.byref(d), FAKE, 12, 1.0, FAKE, 1, FAKE, 128, FAKE, big, None) == kvq.KVQ_EINVAL      # Hq % H
    assert f(None, FAKE, 32, 1.0, FAKE, 1, FAKE, 128, FAKE, big, None) == kvq.KVQ_EINVAL
    # the workspace covers the attention's and the logits of every query head
    need = L.kvq_decode_attn_int4_h2o_ws(C.byref(d), 32)
    assert need >= L.kvq_decode_attn_int4_ws(C.byref(d), 32) + 32 * 128 * 4
    assert f(C.byref(d), FAKE, 32, 1.0, FAKE, 1, FAKE, 128, FAKE, need - 1, None) == kvq.KVQ_EINVAL
    assert L.kvq_decode_attn_int4_h2o_ws(None, 4) == 0


def test_rot_validation(L):
    import numpy as np
    def rd(**kw):
        base = dict(B=1, T=16, H=2, d=128, g=64)
        base.update(kw)
        return kvq.RotDesc(base["B"], base["T"], base["H"], base["d"], base["g"],
                           *[kw.get(f, 0x200000) for f in kvq.RotCache.SECTIONS])
    good = np.ones(128, np.int8)
    bad = good.copy()
    bad[7] = 0
    gp, bp = good.ctypes.data, bad.ctypes.data
    q = L.kvq_rot_quant_int4
    for kw in (dict(d=96), dict(g=16), dict(d=64, g=128), dict(T=0), dict(k_scale=None)):
        assert q(FAKE, FAKE, gp, gp, C.byref(rd(**kw)), None) == kvq.KVQ_EINVAL, kw
    assert q(FAKE, FAKE, bp, gp, C.byref(rd()), None) == kvq.KVQ_EINVAL          # a zero sign
    assert q(FAKE, FAKE, gp, None, C.byref(rd()), None) == kvq.KVQ_EINVAL
    assert q(None, FAKE, gp, gp, C.byref(rd()), None) == kvq.KVQ_EINVAL
    assert q(MISALIGNED, FAKE, gp, gp, C.byref(rd()), None) == kvq.KVQ_EALIGN
    dq = L.kvq_rot_dequant
    assert dq(C.byref(rd()), 2, gp, FAKE, 0, None) == kvq.KVQ_EINVAL             # side
    assert dq(C.byref(rd()), 0, gp, FAKE, 7, None) == kvq.KVQ_EINVAL             # ot
    assert dq(C.byref(rd()), 0, bp, FAKE, 0, None) == kvq.KVQ_EINVAL
    at = L.kvq_rot_decode_attn
    need = L.kvq_rot_decode_attn_ws(C.byref(rd()), 8)
    assert need > 0
    assert at(C.byref(rd()), gp, gp, FAKE, 6, 1.0, FAKE, 1, FAKE, need, None) == kvq.KVQ_EINVAL     # Hq % H
    assert at(C.byref(rd()), gp, gp, FAKE, 64, 1.0, FAKE, 1, FAKE, 1 << 30, None) == kvq.KVQ_EINVAL  # Hq / H = 32
    assert at(C.byref(rd()), gp, gp, FAKE, 8, 1.0, FAKE, 1, FAKE, need - 1, None) == kvq.KVQ_EINVAL
    assert at(C.byref(rd()), gp, bp, FAKE, 8, 1.0, FAKE, 1, FAKE, need, None) == kvq.KVQ_EINVAL
    sect = (C.c_size_t * 6)()
    tot = C.c_size_t()
    assert L.kvq_rot_cache_sizes(2, 10, 3, 128, 64, sect, C.byref(tot)) == kvq.KVQ_OK
    assert list(sect) == [2 * 3 * 10 * 64, 2 * 3 * 10 * 2 * 2, 2 * 3 * 10 * 2 * 2] * 2 and tot.value == sum(sect)


def test_mixed_validation(L):
    def md(**kw):
        d = kvq.MixedDesc(kw.get("N", 100), kw.get("C", 128), kw.get("tags", 0x200000), kw.get("slot", 0x200000))
        for i, c in enumerate(kw.get("cap", (10, 20, 30, 40))):
            d.cap[i] = c
        for f in kvq.MixedStore.POOLS:
            setattr(d, f, kw.get(f, 0x200000))
        return d
    for kw in (dict(N=0), dict(C=100), dict(C=32), dict(C=16384), dict(tags=None), dict(slot=None),
               dict(cap=(10, -1, 0, 0)), dict(q4=None), dict(z8=None), dict(x16=None)):
        assert L.kvq_mixed_quant(FAKE, C.byref(md(**kw)), None) == kvq.KVQ_EINVAL, kw
        assert L.kvq_mixed_dequant(C.byref(md(**kw)), FAKE, 0, None) == kvq.KVQ_EINVAL, kw
    # a pool that holds no rows may be NULL
    assert L.kvq_mixed_quant(None, C.byref(md(cap=(0, 5, 0, 0), q2=None, s2=None)), None) == kvq.KVQ_EINVAL
    assert L.kvq_mixed_dequant(C.byref(md()), FAKE, 9, None) == kvq.KVQ_EINVAL
    assert L.kvq_mixed_quant(MISALIGNED, C.byref(md()), None) == kvq.KVQ_EALIGN
    need = L.kvq_mixed_plan_ws(5000)
    assert need >= 5 * 24
    assert L.kvq_mixed_plan(FAKE, 5000, FAKE, FAKE, FAKE, need - 1, None) == kvq.KVQ_EINVAL
    assert L.kvq_mixed_plan(FAKE, 0, FAKE, FAKE, FAKE, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_mixed_plan(None, 5000, FAKE, FAKE, FAKE, need, None) == kvq.KVQ_EINVAL
    out = (C.c_uint64 * 3)()
    cnt = (C.c_int64 * 4)(10, 20, 30, 40)
    assert L.kvq_mixed_bytes(cnt, 100, 128, out) == kvq.KVQ_OK
    assert list(out) == [10 * 32 + 20 * 64 + 30 * 128 + 40 * 256, 10 * 4 + 20 * 4 + 30 * 5, 25]


def test_select_and_compact_validation(L):
    big = 1 << 30
    h2o = L.kvq_h2o_select
    assert h2o(None, 1, 1, 10, 4, 2, None, FAKE, FAKE, big, None) == kvq.KVQ_EINVAL
    assert h2o(FAKE, 0, 1, 10, 4, 2, None, FAKE, FAKE, big, None) == kvq.KVQ_EINVAL
    assert h2o(FAKE, 1, 0, 10, 4, 2, None, FAKE, FAKE, big, None) == kvq.KVQ_EINVAL
    assert h2o(FAKE, 1, 1, 10, -1, 2, None, FAKE, FAKE, big, None) == kvq.KVQ_EINVAL
    assert h2o(FAKE, 1, 1, 10, 4, -2, None, FAKE, FAKE, big, None) == kvq.KVQ_EINVAL
    assert h2o(FAKE, 1, 1, 10, 4, 2, None, FAKE, None, 0, None) == kvq.KVQ_EINVAL   # needs ws for scores
    assert h2o(FAKE, 1, 1, 1 << 31, 4, 2, None, FAKE, FAKE, big, None) == kvq.KVQ_EINVAL
    assert L.kvq_snapkv_select(FAKE, 1, 0, 4, 2, FAKE, None, 0, None) == kvq.KVQ_EINVAL
    assert L.kvq_snapkv_select(MISALIGNED, 1, 10, 4, 2, FAKE, None, 0, None) == kvq.KVQ_EALIGN
    cp = L.kvq_compact
    assert cp(FAKE, None, 1, 10, 1, 128, FAKE, 11, FAKE, None, None) == kvq.KVQ_EINVAL   # K > T
    assert cp(FAKE, None, 1, 10, 1, 12, FAKE, 5, FAKE, None, None) == kvq.KVQ_EINVAL    # d % 8
    assert cp(FAKE, FAKE, 1, 10, 1, 128, FAKE, 5, FAKE, None, None) == kvq.KVQ_EINVAL   # v pair
    assert cp(FAKE, None, 1, 10, 1, 128, None, 5, FAKE, None, None) == kvq.KVQ_EINVAL   # keep NULL
    assert cp(FAKE, None, 1, 10, 1, 128, FAKE, 0, FAKE, None, None) == kvq.KVQ_EINVAL   # K 0


def test_bw_probe_validation(L):
    bw = L.kvq_bw_probe
    assert bw(FAKE, 64, None, 0, 1, 8, None) == kvq.KVQ_EINVAL            # no sink
    assert bw(None, 64, FAKE, 0, 1, 8, None) == kvq.KVQ_EINVAL            # no source
    assert bw(FAKE, 0, FAKE, 0, 1, 8, None) == kvq.KVQ_EINVAL             # nothing to move
    assert bw(FAKE, 24, FAKE, 0, 1, 8, None) == kvq.KVQ_EINVAL            # not a multiple of 16
    assert bw(FAKE, 48, FAKE, 16, 1, 8, None) == kvq.KVQ_EINVAL           # 3:1 is not a probe mix
    for depth in (0, 3, 16):
        assert bw(FAKE, 64, FAKE, 0, 1, depth, None) == kvq.KVQ_EINVAL    # depth 1, 2, 4 or 8
    assert bw(FAKE, 32 * 16, FAKE, 9 * 16, 1, 2, None) == kvq.KVQ_EINVAL  # 32:9 takes depth 1
    assert bw(MISALIGNED, 64, FAKE, 0, 1, 8, None) == kvq.KVQ_EALIGN


def test_library_has_no_oracle_dependency():
    """The product library and binding never load the oracle."""
    import subprocess
    import sys
    code = ("import sys; import kv_cache_compression_channel_amd as k; k.lib(); "
            "assert 'oracle' not in sys.modules, 'binding imported the oracle'")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)
    out = subprocess.run(["ldd", kvq.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out
    src_dir = os.path.join(ROOT, "kv_cache_compression_channel_amd")
    for dirpath, _, files in os.walk(src_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"import oracle|from oracle|liboracle|\borc_", text), f


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_gpu_visible(), reason="needs a host with no GPU: the arguments are fake pointers that "
                                           "pass validation, so on a GPU they would reach a kernel")
def test_hip_errors_map_to_EHIP(L):
    """With no device, every call that gets past its argument checks fails in the HIP runtime:
    the status is KVQ_EHIP and kvq_last_error names the entry point and the runtime's message.
    Covers launches (the probe, INT4 dequantization) and the device query of the
    no-allocation attention."""
    L.kvq_last_error.restype = C.c_char_p
    assert L.kvq_bw_probe(FAKE, 4096, FAKE, 4096, 0, 8, None) == kvq.KVQ_EHIP
    assert L.kvq_last_error().startswith(b"kvq_bw_probe")
    d = _desc(H=8)
    qd = kvq.QDesc(kvq.KVQ_FMT_INT4_K, C.cast(C.pointer(d), C.c_void_p))
    assert L.kvq_dequant(C.byref(qd), FAKE, 0, None) == kvq.KVQ_EHIP
    assert L.kvq_decode_attn_int4_noalloc(C.byref(d), FAKE, 32, 1.0, FAKE, 1, None) == kvq.KVQ_EHIP
    msg = L.kvq_last_error()
    assert b"kvq_decode_attn_int4_noalloc" in msg and len(msg) > len(b"kvq_decode_attn_int4_noalloc: ")
    # a host-only call after the failures still succeeds
    assert kvq.keep_count(32768, 2048, 256) == 2048
