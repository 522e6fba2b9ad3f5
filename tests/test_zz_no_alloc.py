"""GPU check of the allocation-free decode attention (kvq_decode_attn_int4_noalloc, through the
C ABI): bit-identical to kvq_decode_attn_int4 with a caller-owned workspace, on two calls in a
row whose second is smaller (the scratch keeps the first call's contents), and the size limit
rejected before anything is launched."""
import numpy as np
import pytest
import torch

from kv_cache_compression_channel_amd import kvq, synth
from tests.gpu_helpers import DEV, need_gpu, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _case(B, T, H, Hq, d, g, R, seed):
    K, V, _ = synth.kv_layer(B, T, H, d, seed=seed, device=DEV, n_outlier=0)
    cache = kvq.group_quant_int4(K, V, g=g, R=R)
    q = synth.decode_query(B, Hq, d, seed=seed + 1, device=DEV)
    return cache, q


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_equals_workspace_call(order):
    cases = [(8, 9000, 8, 32, 128, 64, 128, 1),     # matrix-core path, 4 query heads per KV head
             (2, 1300, 2, 8, 64, 32, 40, 2)]        # VALU split path, smaller: second call reuses the scratch
    for (B, T, H, Hq, d, g, R, seed) in cases:
        say("noalloc attention", dict(B=B, T=T, H=H, Hq=Hq, d=d, g=g, R=R))
        cache, q = _case(B, T, H, Hq, d, g, R, seed)
        assert kvq.decode_attn_ws_bytes(cache, Hq) <= kvq.ATTN_SCRATCH_BYTES
        for dt in (torch.float32, torch.bfloat16):
            ref = kvq.decode_attn_int4(cache, q, 1.0, out_dtype=dt)
            got = kvq.decode_attn_int4_noalloc(cache, q, 1.0, out_dtype=dt)
            torch.cuda.synchronize()
            if dt == torch.float32:
                assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), "fp32 output differs"
            else:
                assert np.array_equal(u16(got), u16(ref)), "bf16 output differs"


def test_noalloc_rejects_oversized_partials():
    # 256 x 128 query rows x their split slots x 130 floats > 16 MiB: rejected before any launch
    cache = kvq.Int4Cache.empty(256, 1024, 8, 128, 64, 128, DEV)
    q = torch.zeros((256, 128, 128), dtype=torch.bfloat16, device=DEV)
    assert kvq.decode_attn_ws_bytes(cache, 128) > kvq.ATTN_SCRATCH_BYTES
    with pytest.raises(ValueError, match="scratch"):
        kvq.decode_attn_int4_noalloc(cache, q, 1.0)
