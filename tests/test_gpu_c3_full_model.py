"""GPU parity at full size: the whole-model cache (batch 4 x 32 layers, 8192 tokens, 32 KV
heads, d=128, bf16, per-channel K scales 10^U(-1,1)) through INT4 group quantization at
g = 32 / 64 / 128 and per-channel symmetric INT8, dequantized back to bf16.  The GPU runs
every slice in the same launches the benchmark times; the oracle checks sampled (b, l)
slices and heads element by element, and per-slice error statistics."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_channel_amd import kvq, synth
from tests.gpu_helpers import DEV, STATS_RTOL, assert_bits_equal, assert_rel, need_gpu, np_, say, u16

pytestmark = pytest.mark.gpu

BATCH, LAYERS, T, H, D = 4, 32, 8192, 32, 128
SAMPLES = [(0, 0, 0), (1, 17, 13), (3, 31, 31)]   # (b, l, head)


@pytest.fixture(scope="module")
def cache_kv():
    need_gpu()
    say("full-model cache generation", (BATCH * LAYERS, T, H, D))
    K, V, _ = synth.full_model_cache(BATCH, LAYERS, T, H, D, seed=0, device=DEV)
    torch.cuda.synchronize()
    yield K, V
    del K, V
    torch.cuda.empty_cache()


@pytest.mark.parametrize("g", [32, 64, 128])
def test_int4_sweep_sampled(cache_kv, g):
    K, V = cache_kv
    say("C3 int4", "g", g)
    cache = kvq.group_quant_int4(K, V, g=g, R=0)
    kh = kvq.dequant_int4(cache, "k", torch.bfloat16)
    vh = kvq.dequant_int4(cache, "v", torch.bfloat16)
    torch.cuda.synchronize()
    # exact compression ratio of the quantized cache vs bf16: 2 / (0.5 + 4/g)
    ratio = (K.numel() + V.numel()) * 2 / cache.nbytes()
    assert abs(ratio - 2 / (0.5 + 4 / g)) < 1e-12
    kmax = 0.0
    for b, l, h in SAMPLES:
        s = b * LAYERS + l
        Kb = u16(K[s:s + 1, :, h:h + 1])
        Vb = u16(V[s:s + 1, :, h:h + 1])
        want = oracle.int4_quant(Kb, Vb, g, 0)
        for sec in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
            t = getattr(cache, sec)[s:s + 1, h:h + 1]
            got = u16(t) if t.dtype == torch.bfloat16 else np_(t)
            assert_bits_equal(got, want[sec], f"{sec} slice {(b, l, h)} g={g}")
        for side, Xb, Xh in (("k", Kb, kh), ("v", Vb, vh)):
            oxf = oracle.int4_dequant(want, side)
            got = u16(Xh[s:s + 1, :, h:h + 1])
            assert_bits_equal(got, oracle.f32_to_bf16(oxf), f"{side} dequant slice {(b, l, h)}")
            st = np_(kvq.err_stats(gpu_slice(Xb), Xh[s:s + 1, :, h:h + 1].contiguous()))
            assert_rel(st, oracle.err_stats(Xb, oracle.f32_to_bf16(oxf)), STATS_RTOL, f"{side} stats {(b, l, h)}")
            if side == "k":
                kmax = max(kmax, st[2])
    # whole-tensor statistics bound the sampled ones
    full = np_(kvq.err_stats(K, kh))
    assert full[2] >= kmax and full[0] > 0


@pytest.mark.parametrize("g", [32, 64, 128])
def test_int4_whole_slice_every_head(cache_kv, g):
    """One whole (b, l) slice, all 32 heads, every section and both dequantized sides
    element by element (the sampled test above covers one head of three slices)."""
    K, V = cache_kv
    b, l = 2, 5
    s = b * LAYERS + l
    say("C3 int4 whole slice", (b, l), "g", g)
    cache = kvq.group_quant_int4(K, V, g=g, R=0)
    kh = kvq.dequant_int4(cache, "k", torch.bfloat16)
    vh = kvq.dequant_int4(cache, "v", torch.bfloat16)
    torch.cuda.synchronize()
    Kb, Vb = u16(K[s:s + 1]), u16(V[s:s + 1])
    want = oracle.int4_quant(Kb, Vb, g, 0)
    for sec in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        t = getattr(cache, sec)[s:s + 1]
        got = u16(t) if t.dtype == torch.bfloat16 else np_(t)
        assert_bits_equal(got, want[sec], f"{sec} slice {(b, l)} g={g}")
    for side, Xh in (("k", kh), ("v", vh)):
        assert_bits_equal(u16(Xh[s:s + 1]), oracle.f32_to_bf16(oracle.int4_dequant(want, side)),
                          f"{side} dequant slice {(b, l)} g={g}")


def gpu_slice(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def test_int8_per_channel_sampled(cache_kv):
    K, V = cache_kv
    say("C3 int8 per-channel")
    x = K.view(BATCH * LAYERS, T, H * D)           # channels = every (head, dim) of the layer
    q, s, _ = kvq.quant_sym(x, bits=8, with_zp=True)
    xh = kvq.dequant_pc(q, s, None, torch.bfloat16)
    torch.cuda.synchronize()
    for b, l, _h in SAMPLES:
        sl = b * LAYERS + l
        xb = u16(x[sl:sl + 1])
        oq, os_, _ = oracle.quant_sym(xb, 8)
        assert_bits_equal(np_(q[sl:sl + 1]), oq, f"int8 codes slice {sl}")
        assert_bits_equal(np_(s[sl:sl + 1]).view(np.uint32), os_.view(np.uint32), f"int8 scales slice {sl}")
        oxh = oracle.dequant_pc(oq, os_, None)
        assert_bits_equal(u16(xh[sl:sl + 1]), oracle.f32_to_bf16(oxh), f"int8 dequant slice {sl}")
    # ratio with scale and zero-point bytes: 2T*C / (T*C + 4C + C)
    r = kvq.compression_ratio(x.numel() * 2, q.numel(), s.numel() * 4, s.numel())
    assert abs(r - 2 * T / (T + 5)) < 1e-12
