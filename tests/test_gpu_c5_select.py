"""GPU parity: H2O cumulative scores, recent-window + TopK selection (ties to the lower
index), SnapKV selection and compaction of the kept KV rows, bit-exact against the oracle.
Cases: the full configuration (8 x 32 rows, 64 observed steps, 32768 tokens, W=256,
B=2048; sampled rows of the 2 GiB history), small rows, tie-heavy scores, T < W, T <= B,
budget 0, window 0, T beyond the register-resident limit, and -inf / NaN scores."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_channel_amd import kvq, synth
from tests.gpu_helpers import DEV, assert_bits_equal, need_gpu, np_, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def check_h2o(hist: torch.Tensor, budget: int, window: int):
    rows, T_obs, T = hist.shape
    say("h2o", dict(rows=rows, T_obs=T_obs, T=T, budget=budget, window=window))
    scores = torch.empty((rows, T), dtype=torch.float32, device=DEV)
    keep = kvq.h2o_select(hist.to(DEV), budget, window, scores=scores)
    keep2 = kvq.h2o_select(hist.to(DEV), budget, window)     # scores in the workspace
    torch.cuda.synchronize()
    okeep, oscores = oracle.h2o_select(hist.numpy(), budget, window)
    assert_bits_equal(np_(scores).view(np.uint32), oscores.view(np.uint32), "H2O scores")
    assert_bits_equal(np_(keep), okeep, "H2O keep")
    assert_bits_equal(np_(keep2), okeep, "H2O keep (workspace scores)")
    return keep


def check_snapkv(scores: torch.Tensor, budget: int, window: int):
    rows, T = scores.shape
    say("snapkv", dict(rows=rows, T=T, budget=budget, window=window))
    keep = kvq.snapkv_select(scores.to(DEV), budget, window)
    torch.cuda.synchronize()
    assert_bits_equal(np_(keep), oracle.select(scores.numpy(), budget, window), "SnapKV keep")


@pytest.mark.parametrize("T,budget,window", [(3000, 512, 256), (300, 64, 256), (200, 300, 16), (200, 200, 0),
                                             (200, 0, 8), (200, 0, 0), (1, 1, 1), (5, 3, 0), (1025, 100, 1)])
def test_h2o_small(T, budget, window):
    hist = synth.attention_history(4, 8, T, seed=T + budget)
    check_h2o(hist, budget, window)


def test_tie_heavy_snapkv():
    for levels in (1, 2, 3, 7):
        s = synth.tie_heavy_scores(6, 5000, levels, seed=levels)
        check_snapkv(s, 700, 64)
        check_snapkv(s, 4999, 1)


def test_special_values_snapkv():
    s = synth.tie_heavy_scores(3, 4000, 5, seed=1)
    s[0, ::7] = float("-inf")
    s[1, ::5] = float("nan")
    s[2, :100] = float("inf")
    s[2, 100:200] = -0.0
    s[2, 200:300] = 0.0
    check_snapkv(s, 1000, 128)
    check_snapkv(s, 3990, 0)
    # NaN scores before the window are needed to fill the budget: the window's masked tokens
    # rank below them, so the union still holds the full keep count
    check_snapkv(s, 3990, 128)
    check_snapkv(s, 3500, 600)
    n = torch.full((2, 700), float("nan"))
    n[0, ::3] = torch.arange(0, 700, 3, dtype=torch.float32)
    check_snapkv(n, 300, 50)
    check_snapkv(n, 690, 64)
    # a NaN in the history makes its token's H2O score NaN (fused path and the general one)
    hist = synth.attention_history(3, 4, 2048, seed=9)
    hist[0, 2, ::5] = float("nan")
    hist[2, 0, :1500] = float("nan")
    check_h2o(hist, 1900, 128)
    hist = synth.attention_history(2, 3, 2050, seed=10)
    hist[1, 1, 3::4] = float("nan")
    check_h2o(hist, 2000, 100)


def test_long_rows_beyond_register_path():
    s = synth.normal_fp32((2, 40000), seed=4)
    check_snapkv(s, 3000, 256)
    hist = synth.attention_history(1, 4, 33000, seed=5)
    check_h2o(hist, 2048, 256)


def test_compact_small():
    B, T, H, d = 2, 500, 3, 128
    K = synth.normal_bf16((B, T, H, d), seed=1)
    V = synth.normal_bf16((B, T, H, d), seed=2)
    hist = synth.attention_history(B * H, 4, T, seed=3)
    keep = check_h2o(hist, 96, 32).view(B, H, -1)
    kd, vd = kvq.compact(K.to(DEV), V.to(DEV), keep)
    kd1, vd1 = kvq.compact(K.to(DEV), None, keep)
    torch.cuda.synchronize()
    assert vd1 is None
    okeep = oracle.h2o_select(hist.numpy(), 96, 32)[0].reshape(B, H, -1)   # equal to keep (checked above)
    assert_bits_equal(u16(kd), oracle.compact(u16(K), okeep), "compact K")
    assert_bits_equal(u16(vd), oracle.compact(u16(V), okeep), "compact V")
    assert_bits_equal(u16(kd1), u16(kd), "compact K only")
    for dd in (8, 64, 256):
        K2 = synth.normal_bf16((1, 50, 2, dd), seed=dd)
        kp = torch.sort(torch.randperm(50)[:9].repeat(2, 1), dim=-1).values.to(torch.int32).view(1, 2, 9)
        kd2, _ = kvq.compact(K2.to(DEV), None, kp.to(DEV))
        torch.cuda.synchronize()
        assert_bits_equal(u16(kd2), oracle.compact(u16(K2), kp.numpy()), f"compact d={dd}")


def test_compact_out_of_range_indices_are_clamped():
    """Keep entries below 0 or at / past T move the row of the nearest valid index (the
    documented clamp), so a bad index never reads outside the source."""
    B, T, H, d = 2, 77, 3, 128
    K = synth.normal_bf16((B, T, H, d), seed=12)
    V = synth.normal_bf16((B, T, H, d), seed=13)
    keep = torch.randint(0, T, (B, H, 20), dtype=torch.int32)
    keep[0, 0, 3] = -1
    keep[0, 1, 0] = -(2 ** 31)
    keep[1, 2, 19] = T
    keep[1, 0, 7] = 2 ** 31 - 1
    say("compact clamp", dict(B=B, T=T, H=H, d=d))
    kd, vd = kvq.compact(K.to(DEV), V.to(DEV), keep.to(DEV))
    torch.cuda.synchronize()
    kc = keep.clamp(0, T - 1).numpy()
    assert_bits_equal(u16(kd), oracle.compact(u16(K), kc), "compact K, clamped indices")
    assert_bits_equal(u16(vd), oracle.compact(u16(V), kc), "compact V, clamped indices")


def test_config5_full_size_sampled_rows():
    Bb, Hh, T_obs, T, W, budget, d = 8, 32, 64, 32768, 256, 2048, 128
    rows = Bb * Hh
    say("select full", dict(rows=rows, T_obs=T_obs, T=T))
    hist = synth.attention_history(rows, T_obs, T, seed=0, device=DEV)
    scores = torch.empty((rows, T), dtype=torch.float32, device=DEV)
    keep = kvq.h2o_select(hist, budget, W, scores=scores)
    K = synth.normal_bf16((Bb, T, Hh, d), seed=1, device=DEV)
    V = synth.normal_bf16((Bb, T, Hh, d), seed=2, device=DEV)
    kd, vd = kvq.compact(K, V, keep.view(Bb, Hh, -1))
    torch.cuda.synchronize()
    assert keep.shape == (rows, 2048)
    rng = np.random.default_rng(0)
    for r in sorted(set(rng.integers(0, rows, 6).tolist()) | {0, rows - 1}):
        h_r = np_(hist[r:r + 1])
        okeep, oscores = oracle.h2o_select(h_r, budget, W)
        assert_bits_equal(np_(scores[r:r + 1]).view(np.uint32), oscores.view(np.uint32), f"scores row {r}")
        assert_bits_equal(np_(keep[r:r + 1]), okeep, f"keep row {r}")
        b, h = divmod(r, Hh)
        idx = torch.from_numpy(okeep[0]).long().to(DEV)
        assert torch.equal(kd[b, :, h], K[b, idx, h]) and torch.equal(vd[b, :, h], V[b, idx, h])
