"""GPU test of the streaming-read probe: it reads every 16-byte word exactly once, so the
XOR of its per-work-group words equals the XOR of all 32-bit words of the buffer (computed
with NumPy), for a size with a ragged tail and for the headline cache size."""
import numpy as np
import pytest
import torch

import rank_latent_kv_amd as R

from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 256 * 16 * 3 + 16 * 77, 167_772_160])
def test_read_probe_xor(nbytes):
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    say(f"read probe {nbytes} bytes")
    out = R.read_probe(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
