"""GPU parity: per-channel symmetric / asymmetric quantization, dequantization and error
statistics (Walkthrough §1.1-§2) against the oracle, on fp32 [256 tokens][128 channels]
N(0,1), the 4-value worked example, bf16 multi-slice inputs with strides, and the
degenerate channels (all-zero, constant, all-positive)."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_channel_amd import kvq, synth
from tests.gpu_helpers import (DEV, STATS_RTOL, assert_bits_equal, assert_rel, need_gpu, np_, say, u16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _check_pc(x_gpu: torch.Tensor, x_host: np.ndarray, mode: str, bits=8, qmin=-128, qmax=127):
    say("per-channel", mode, tuple(x_gpu.shape), x_gpu.dtype, bits, qmin, qmax)
    if mode == "sym":
        q, s, z = kvq.quant_sym(x_gpu, bits)
        oq, os_, oz = oracle.quant_sym(x_host, bits)
    else:
        q, s, z = kvq.quant_asym(x_gpu, qmin, qmax)
        oq, os_, oz = oracle.quant_asym(x_host, qmin, qmax)
    torch.cuda.synchronize()
    assert_bits_equal(np_(q), oq.reshape(np_(q).shape), f"{mode} codes")
    assert_bits_equal(np_(s).view(np.uint32), os_.view(np.uint32), f"{mode} scales")
    assert_bits_equal(np_(z), oz, f"{mode} zero points")
    # dequantization: fp32 bit-exact, bf16 = round-to-nearest-even of the fp32 result
    xh = kvq.dequant_pc(q, s, z, torch.float32)
    xb = kvq.dequant_pc(q, s, z, torch.bfloat16)
    oxh = oracle.dequant_pc(oq, os_, oz)
    torch.cuda.synchronize()
    assert_bits_equal(np_(xh).view(np.uint32), oxh.view(np.uint32), f"{mode} dequant fp32")
    assert_bits_equal(u16(xb), oracle.f32_to_bf16(oxh), f"{mode} dequant bf16")
    # error statistics, fp64
    raw = np_(kvq.err_stats(x_gpu.contiguous(), xh))
    want = oracle.err_stats(x_host, oxh)
    assert_rel(raw, want, STATS_RTOL, f"{mode} stats")
    n = x_host.size
    assert_rel(kvq.stats_finalize(raw, n), oracle.stats_finalize(want, n), STATS_RTOL, f"{mode} finalize")
    return q, s, z


def test_config1_fp32_256x128_sym_asym():
    x = synth.normal_fp32((256, 128), seed=0)
    xg = x.to(DEV)
    q, s, z = _check_pc(xg, x.numpy(), "sym", bits=8)
    _check_pc(xg, x.numpy(), "asym")
    # compression ratio including scale and zero-point bytes
    r = kvq.compression_ratio(x.numel() * 4, q.numel(), s.numel() * 4, z.numel())
    assert f"{r:.6f}" == "3.923372"


def test_worked_example_on_gpu():
    x = synth.worked_example()
    q, s, _ = _check_pc(x.to(DEV), x.numpy(), "sym", bits=4)
    assert np_(q).ravel().tolist() == [-7, -1, 2, 7]
    assert np_(s).view(np.uint32)[0, 0] == 0x3E124925


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_sym_all_bit_widths(bits):
    x = synth.normal_fp32((3, 70, 24), seed=bits)
    _check_pc(x.to(DEV), x.numpy(), "sym", bits=bits)


@pytest.mark.parametrize("qmin,qmax", [(-128, 127), (0, 15), (-8, 7), (0, 255 // 2)])
def test_asym_ranges(qmin, qmax):
    x = synth.normal_fp32((2, 300, 40), seed=qmax)
    _check_pc(x.to(DEV), x.numpy(), "asym", qmin=qmin, qmax=qmax)


def test_bf16_slices_ragged_rows():
    # several slices, rows not a multiple of the 256-row chunk, vector (C % 8 == 0) and scalar paths
    for shape in ((5, 513, 256), (2, 257, 4096), (3, 33, 12), (1, 1, 8)):
        x = synth.normal_bf16(shape, seed=sum(shape))
        _check_pc(x.to(DEV), u16(x), "sym", bits=8)
        _check_pc(x.to(DEV), u16(x), "asym")


def test_strided_view():
    # [nb][R][C] view into a wider buffer: row stride ldx > C, slice stride > R*ldx
    big = synth.normal_fp32((4, 130, 160), seed=5)
    view = big[:, 1:129, 16:144]            # [4][128][128], ldx = 160
    assert view.stride() == (130 * 160, 160, 1)
    xg = big.to(DEV)[:, 1:129, 16:144]
    _check_pc(xg, np.ascontiguousarray(view.numpy()), "sym", bits=8)
    _check_pc(xg, np.ascontiguousarray(view.numpy()), "asym")


def test_degenerate_channels():
    x = synth.normal_fp32((256, 32), seed=9).numpy()
    x[:, 0] = 0.0                         # all zero: range floored at 1e-8
    x[:, 1] = 0.75                        # constant
    x[:, 2] = np.abs(x[:, 2]) + 1.0       # all positive: asym zero point saturates
    x[:, 3] = -np.abs(x[:, 3]) - 2.0      # all negative
    x[:, 4] = 1e-9                        # below the floor
    x[::2, 5] = 0.5                       # exact half quotients
    x[1::2, 5] = -0.5
    x[0, 5] = 7.0 / 127 * 127             # absmax 7: s = 7/127
    xt = torch.from_numpy(x)
    _check_pc(xt.to(DEV), x, "sym", bits=8)
    _check_pc(xt.to(DEV), x, "sym", bits=4)
    _check_pc(xt.to(DEV), x, "asym")


def test_exact_half_quotients():
    # absmax 7 at bits 4 -> s = 1: quotients are exact halves, which must round half to even
    col = np.array([7, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 4.5, -6.5] * 26, np.float32)
    x = np.stack([col, col * 2, col * 0.25], 1)
    _check_pc(torch.from_numpy(x).to(DEV), x, "sym", bits=4)
    # asym with s = 1 and an odd zero point (-1)
    col = np.array([-127, 128, 0.5, 2.5, -3.5, 5.5] * 40, np.float32)[:, None]
    _check_pc(torch.from_numpy(col).to(DEV), col, "asym")


@pytest.mark.parametrize("shape", [(2, 8192, 4096), (4, 1, 2048), (8, 128, 1024), (8, 129, 1024),
                                   (3, 5000, 2752), (2, 4999, 4096), (32, 2000, 4096)])
def test_bf16_wide_slices(shape):
    """bf16 slices with thousands of channels, as the full-model cache uses them: row counts of
    one, below, at and past a 128- and 256-row chunk, a whole 8192-token slice pair, and enough
    slices that the min/max pass takes 512-row chunks (the last one ragged), with all-zero,
    constant, all-positive, exact-half and far-from-zero channels."""
    x = synth.normal_bf16(shape, seed=sum(shape) + 1)
    xf = x.float()
    xf[0, :, 5] = 0.0                                   # all-zero channel
    xf[-1, :, 33] = 2.5                                 # constant channel
    xf[0, :, 64] = xf[0, :, 64].abs() + 1.0             # all positive
    # absmax 127/16 gives s = 1/16 exactly; every other value sits on a half step (k + 0.5) / 16
    xf[-1, :, 100] = (torch.arange(shape[1]) % 20 - 10 + 0.5) / 16
    xf[-1, 0, 100] = 127 / 16
    xf[0, :, 200] = 100 + 0.25 * xf[0, :, 200]         # far from zero: |x / s| > 250 under asym
    x = xf.to(torch.bfloat16)
    _check_pc(x.to(DEV), u16(x), "sym", bits=8)
    _check_pc(x.to(DEV), u16(x), "asym")
    if shape[1] <= 1000:
        _check_pc(x.to(DEV), u16(x), "sym", bits=3)
        _check_pc(x.to(DEV), u16(x), "asym", qmin=0, qmax=15)


def test_bf16_wide_strided_view():
    big = synth.normal_bf16((2, 300, 4160), seed=31)
    xg = big.to(DEV)[:, 3:260, 32:4128]                 # [2][257][4096], ldx = 4160
    assert xg.stride() == (300 * 4160, 4160, 1)
    host = np.ascontiguousarray(u16(big)[:, 3:260, 32:4128])
    _check_pc(xg, host, "sym", bits=8)
    _check_pc(xg, host, "asym")
