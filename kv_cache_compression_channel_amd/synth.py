"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This module only draws numbers; it holds none of the compression arithmetic.
Every generator takes an explicit seed and a device.  Small inputs are drawn
on the CPU (so the oracle and the GPU path read identical bytes after a
copy); the large workloads are drawn directly on the GPU with torch's
counter-based generator and sampled slices are copied back for checking.

Workload shapes follow the pages:
  * per-channel INT8 on a single fp32 tensor [256 tokens][128 channels], N(0,1);
  * one layer of KV cache, bf16 [T=8192][Hkv=8][d=128] (the single-layer residual
    budget example of the KV-cache-compression explainer page) with 4 of 128 K
    channels scaled x10 to act as outlier channels (the page's "why the grouping
    axis matters for outliers" section suggests amplifying one K channel);
  * a full-model cache (32 layers, 32 KV heads, d=128, 8192 tokens, the page's
    "turn savings into bytes" example) at batch 4 with per-channel K scales drawn
    log-uniform in [0.1, 10];
  * GQA decode over INT4 KV at context 32768;
  * H2O / SnapKV selection on softmax-normalised attention histories.
"""
from __future__ import annotations

import math

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def worked_example() -> torch.Tensor:
    """The 4-value teaching example of the 4-bit section, as [4 tokens][1 channel] fp32."""
    return torch.tensor([[-1.0], [-0.2], [0.3], [1.0]], dtype=torch.float32)


def normal_fp32(shape, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    g = _gen(seed, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def normal_bf16(shape, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def kv_layer(B: int, T: int, H: int, d: int, seed: int, device="cpu",
             n_outlier: int = 4, outlier_scale: float = 10.0):
    """K, V bf16 [B][T][H][d], N(0,1); ``n_outlier`` distinct K channels (same in every
    head, drawn from the seed) multiplied by ``outlier_scale`` before rounding to bf16.
    Returns (K, V, outlier_channel_indices)."""
    g = _gen(seed, device)
    k = torch.randn(B, T, H, d, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(B, T, H, d, generator=g, device=device, dtype=torch.float32)
    gc = _gen(seed + 1000003, "cpu")
    idx = torch.randperm(d, generator=gc)[:n_outlier].sort().values
    if n_outlier:
        k[..., idx.to(device)] *= outlier_scale
    return k.to(torch.bfloat16), v.to(torch.bfloat16), idx


def full_model_cache(batch: int, layers: int, T: int, H: int, d: int, seed: int, device="cpu"):
    """K, V bf16 [batch*layers][T][H][d] (slice index = b*layers + l), N(0,1), with every
    K channel of every (layer, head) scaled by 10**U(-1, 1), shared across the batch."""
    g = _gen(seed, device)
    ks = torch.pow(10.0, torch.rand(layers, H, d, generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0)
    K = torch.empty(batch, layers, T, H, d, dtype=torch.bfloat16, device=device)
    V = torch.empty(batch, layers, T, H, d, dtype=torch.bfloat16, device=device)
    for b in range(batch):
        for l in range(layers):
            kk = torch.randn(T, H, d, generator=g, device=device, dtype=torch.float32)
            kk.mul_(ks[l])
            K[b, l].copy_(kk)
            V[b, l].copy_(torch.randn(T, H, d, generator=g, device=device, dtype=torch.float32))
            del kk
    return K.view(batch * layers, T, H, d), V.view(batch * layers, T, H, d), ks


def decode_query(B: int, Hq: int, d: int, seed: int, device="cpu") -> torch.Tensor:
    """Q bf16 [B][Hq][d] drawn N(0,1)/sqrt(d)."""
    g = _gen(seed, device)
    q = torch.randn(B, Hq, d, generator=g, device=device, dtype=torch.float32) / math.sqrt(d)
    return q.to(torch.bfloat16)


def attention_history(rows: int, T_obs: int, T: int, seed: int, device="cpu", var: float = 2.0) -> torch.Tensor:
    """fp32 [rows][T_obs][T]; each [row][t] vector is a softmax over T of N(0, var) logits
    (softmax taken in fp64 on the CPU, fp32 on the GPU for the large sizes)."""
    g = _gen(seed, device)
    out = torch.empty(rows, T_obs, T, dtype=torch.float32, device=device)
    sd = math.sqrt(var)
    for r in range(rows):
        logits = torch.randn(T_obs, T, generator=g, device=device, dtype=torch.float32) * sd
        if device == "cpu" or str(device) == "cpu":
            out[r] = torch.softmax(logits.double(), dim=-1).float()
        else:
            out[r] = torch.softmax(logits, dim=-1)
    return out


def tie_heavy_scores(rows: int, T: int, levels: int, seed: int, device="cpu") -> torch.Tensor:
    """fp32 [rows][T] scores taking only ``levels`` distinct values (k/levels), so that
    the TopK threshold almost always falls inside a run of equal scores."""
    g = _gen(seed, device)
    return torch.randint(0, levels, (rows, T), generator=g, device=device).to(torch.float32) / float(levels)
