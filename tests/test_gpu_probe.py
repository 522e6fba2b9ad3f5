"""GPU check of the streaming bandwidth probe used to state the measured ceilings: every mix
runs at every depth, and a write-only probe writes exactly its bytes with the value each store
carries (thread t of a workgroup stores (t ^ i, t, t, t) as its i-th 16-byte chunk, chunk
(block * depth + i) * 256 + t)."""
import numpy as np
import pytest
import torch

from kv_cache_compression_channel_amd import kvq
from tests.gpu_helpers import DEV, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("depth", [1, 2, 4, 8])
def test_write_only_pattern_and_bounds(depth):
    n = 1 << 20
    dst = torch.zeros(n + 4096, dtype=torch.uint8, device=DEV)
    say("bw probe write", n, "depth", depth)
    kvq.bw_probe(None, 0, dst, n, nt=False, depth=depth)
    torch.cuda.synchronize()
    w = dst[:n].view(torch.int32).view(-1, 4).cpu().numpy()
    j = np.arange(n // 16, dtype=np.int32)
    t, i = j % 256, (j // 256) % depth
    assert np.array_equal(w[:, 0], t ^ i) and np.array_equal(w[:, 1], t) and np.array_equal(w[:, 3], t)
    assert int(dst[n:].abs().sum()) == 0          # nothing past the requested bytes


@pytest.mark.parametrize("a,b", [(1, 0), (1, 1), (2, 1), (1, 2), (32, 9), (9, 32)])
def test_every_mix_runs(a, b):
    unit = 1 << 16
    src = torch.ones(a * unit * 16 + 16, dtype=torch.uint8, device=DEV)
    dst = torch.zeros(max(b * unit * 16, 16) + 4096, dtype=torch.uint8, device=DEV)
    say("bw probe mix", a, b)
    for depth in ((1,) if a + b > 16 else (1, 2, 4, 8)):
        for nt in (False, True):
            kvq.bw_probe(src, a * unit * 16, dst, b * unit * 16, nt=nt, depth=depth)
    torch.cuda.synchronize()
    assert int(dst[max(b * unit * 16, 16):].abs().sum()) == 0
