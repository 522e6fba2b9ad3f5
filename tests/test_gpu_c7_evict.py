"""GPU parity: eviction on the INT4 cache against the oracle, bit for bit.

The source cache is the oracle's quantization of seeded K, V (uploaded), the keep lists are
seeded (random subsets, the selector's recent-window + TopK union, aligned and shifted
runs, unsorted lists with repeats); the kernel's result must equal the oracle's eviction in
every section.  The full-size case quantizes and evicts on the GPU at batch 16, 8 KV heads,
context 32768 (budget 2048, window 256) and checks sampled heads: their source sections
against the oracle's quantization of the same input slice, then their evicted sections
against the oracle's eviction of that slice.

Cases: every (d, g); bf16 window sizes 0, the old one, and ones that pull quantized tokens
into it; identity (keep all); whole aligned groups (copied) next to shifted runs
(requantized); all-window sources; one kept token; growable source and destination;
out-of-range indices (clamped)."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_channel_amd import kvq, synth
from tests.gpu_helpers import ATTN_ROW_RTOL, DEV, assert_bits_equal, gpu_cache, need_gpu, np_, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def valid_np(cache) -> dict:
    d = {}
    for s in cache.SECTIONS:
        t = cache.valid(s)
        d[s] = u16(t) if t.dtype == torch.bfloat16 else np_(t)
    return d


def compare(got_cache, want: dict, what: str):
    got = valid_np(got_cache)
    assert (got_cache.T, got_cache.R) == (want["T"], want["R"])
    for s in kvq.Int4Cache.SECTIONS:
        assert_bits_equal(got[s], want[s], f"{what}: {s}")


def src_cache(B, T, H, d, g, R, seed):
    K, V, _ = synth.kv_layer(B, T, H, d, seed=seed)
    return oracle.int4_quant(u16(K), u16(V), g, R)


def random_keep(B, H, T, K, seed):
    rng = np.random.default_rng(seed)
    return np.sort(np.stack([[rng.choice(T, K, replace=False) for _ in range(H)] for _ in range(B)]), -1).astype(np.int32)


def run(c: dict, keep: np.ndarray, R2: int, what: str, src_cap=0, src_rcap=0, dst=None):
    say("evict", dict(what=what, B=c["B"], T=c["T"], H=c["H"], d=c["d"], g=c["g"], R=c["R"], K=keep.shape[-1], R2=R2,
                      src_cap=src_cap, src_rcap=src_rcap))
    src = gpu_cache(c, src_cap, src_rcap)
    out = kvq.int4_evict(src, torch.from_numpy(np.ascontiguousarray(keep)).to(DEV), R2, out=dst)
    torch.cuda.synchronize()
    want = oracle.int4_evict(c, keep, R2)
    compare(out, want, what)
    return out, want


@pytest.mark.parametrize("d,g", [(64, 32), (64, 64), (128, 32), (128, 64), (128, 128), (256, 32), (256, 64),
                                 (256, 128)])
def test_shapes_and_window_sizes(d, g):
    B, H, R = 2, 3, 17
    T = 5 * g + 37 + R
    c = src_cache(B, T, H, d, g, R, seed=d + g)
    K = 3 * g + 29
    keep = random_keep(B, H, T, K, seed=d * g)
    for R2 in (R, 0, K - 2 * g, K):
        run(c, keep, R2, f"random R2={R2}")


def test_selector_keep_lists():
    B, H, d, g, R, T = 2, 4, 128, 64, 128, 4096 + 128
    c = src_cache(B, T, H, d, g, R, seed=3)
    rng = np.random.default_rng(3)
    scores = rng.random((B * H, T)).astype(np.float32)
    for budget, window in ((1024, 256), (1000, 256), (700, 64)):
        keep = oracle.select(scores, budget, window).reshape(B, H, -1)
        K = keep.shape[-1]
        # the old window kept whole; and a window that makes the quantized part a multiple of g
        for R2 in (min(R, K), min(K, R + (K - R) % g)):
            run(c, keep, R2, f"select budget={budget} window={window} R2={R2}")


def test_identity_whole_groups_and_shifted_runs():
    B, H, d, g, R = 1, 3, 128, 64, 40
    T = 6 * g + 17 + R
    c = src_cache(B, T, H, d, g, R, seed=11)
    every = np.broadcast_to(np.arange(T, dtype=np.int32), (B, H, T)).copy()
    _, want = run(c, every, R, "identity")
    for s in kvq.Int4Cache.SECTIONS:
        assert np.array_equal(want[s], c[s]), s
    K = 3 * g + 17 + R
    keep = np.stack([
        np.concatenate([np.arange(0, g), np.arange(2 * g, 4 * g), np.arange(6 * g, T)]),        # whole groups
        np.concatenate([np.arange(g // 2, g // 2 + 3 * g), np.arange(6 * g, T)]),               # shifted run
        np.concatenate([np.arange(g, 2 * g), np.arange(3 * g + 1, 5 * g + 1), np.arange(6 * g, T)]),
    ])[None].astype(np.int32)
    assert keep.shape[-1] == K
    run(c, keep, R, "whole and shifted")
    run(c, keep, R + 17, "whole and shifted, partial group into the window")


def test_edges():
    d, g = 128, 64
    c = src_cache(2, 300, 2, d, g, 44, seed=21)
    one = np.array([[[5], [299]], [[256], [0]]], np.int32)
    run(c, one, 0, "one token quantized")
    run(c, one, 1, "one token bf16")
    allres = src_cache(2, 200, 2, d, g, 200, seed=22)          # every token in the bf16 window
    keep = random_keep(2, 2, 200, 150, seed=22)
    run(allres, keep, 0, "window source, all quantized")
    run(allres, keep, 50, "window source, mixed")
    noquant = src_cache(1, 256, 2, d, g, 0, seed=23)           # no window in the source
    run(noquant, random_keep(1, 2, 256, 256, seed=23), 0, "K = T")


def test_unsorted_repeats_and_out_of_range_indices():
    B, H, d, g, R, T = 2, 2, 128, 32, 20, 400
    c = src_cache(B, T, H, d, g, R, seed=31)
    rng = np.random.default_rng(31)
    keep = rng.integers(0, T, (B, H, 150)).astype(np.int32)      # unsorted, with repeats
    run(c, keep, 30, "unsorted with repeats")
    wild = keep.copy()
    wild[0, 0, :7] = [-5, T, T + 1000, -(2**31), 2**31 - 1, 0, T - 1]
    say("evict", "out-of-range indices")
    src = gpu_cache(c)
    out = kvq.int4_evict(src, torch.from_numpy(wild).to(DEV), 30)
    torch.cuda.synchronize()
    compare(out, oracle.int4_evict(c, np.clip(wild, 0, T - 1).astype(np.int32), 30), "clamped")


def test_growable_source_and_destination_serve_attention():
    B, H, Hq, d, g, R = 2, 2, 8, 128, 64, 128
    T = 2048 + R
    c = src_cache(B, T, H, d, g, R, seed=41)
    keep = oracle.select(np.random.default_rng(41).random((B * H, T)).astype(np.float32), 600, 256).reshape(B, H, -1)
    K = keep.shape[-1]
    R2 = R + (K - R) % g
    dst = kvq.Int4Cache.empty_stream(B, H, d, g, 1024, R2 + 2 * g, DEV)
    out, want = run(c, keep, R2, "growable", src_cap=T - R + 3 * g, src_rcap=R + 64, dst=dst)
    q = synth.decode_query(B, Hq, d, seed=42)
    o = kvq.decode_attn_int4(out, q.to(DEV), 1.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decode_attn(want, u16(q), 1.0)
    got = np_(o).astype(np.float64)
    err = np.abs(got - ref).max(-1) / np.abs(ref).max(-1)
    assert err.max() <= ATTN_ROW_RTOL, f"attention on the evicted cache: {err.max():.3e}"
    # the evicted growable cache keeps growing
    Kn, Vn, _ = synth.kv_layer(B, 1, H, d, seed=43)
    kvq.int4_append(out, Kn.to(DEV), Vn.to(DEV), r_keep=R2)
    torch.cuda.synchronize()
    assert (out.T, out.R) == (K + 1, R2 + 1)


def test_full_size_sampled_heads():
    B, H, d, T, g, R = 16, 8, 128, 32768, 64, 128
    budget, window = 2048, 256
    say("evict full", dict(B=B, H=H, d=d, T=T, budget=budget, window=window))
    K_, V_, _ = synth.kv_layer(B, T, H, d, seed=0, device=DEV, n_outlier=0)
    cache = kvq.group_quant_int4(K_, V_, g=g, R=R)
    # one-shot observation scores (a softmax row per (b, h)) and the selector's keep lists
    scores = np_(synth.attention_history(B * H, 1, T, seed=5)[:, 0])
    keep_np = oracle.select(scores, budget, window).reshape(B, H, -1)
    Kk = keep_np.shape[-1]
    R2 = R + (Kk - R) % g
    out = kvq.int4_evict(cache, torch.from_numpy(keep_np).to(DEV), R2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    heads = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, B, 4), rng.integers(0, H, 4))} | {(B - 1, H - 1)})
    for (b, h) in heads:
        Ks = u16(K_[b:b + 1, :, h:h + 1])
        Vs = u16(V_[b:b + 1, :, h:h + 1])
        ref_src = oracle.int4_quant(Ks, Vs, g, R)
        for s in kvq.Int4Cache.SECTIONS:
            t = getattr(cache, s)[b:b + 1, h:h + 1]
            assert_bits_equal(u16(t) if t.dtype == torch.bfloat16 else np_(t), ref_src[s], f"source ({b},{h}) {s}")
        want = oracle.int4_evict(ref_src, keep_np[b:b + 1, h:h + 1], R2)
        for s in kvq.Int4Cache.SECTIONS:
            t = getattr(out, s)[b:b + 1, h:h + 1]
            assert_bits_equal(u16(t) if t.dtype == torch.bfloat16 else np_(t), want[s], f"evicted ({b},{h}) {s}")
