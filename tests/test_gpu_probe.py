"""sas_probe_read, the gather-ceiling measurement utility: each workgroup's
sink word is the XOR of every 16-byte word of its chunks, checked against
numpy on the host copy of the buffer (a ragged last workgroup included)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from learned_block_sparse_tok_amd import ops

pytestmark = pytest.mark.gpu
CHUNK = 16384


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()


@pytest.mark.parametrize("n,per", [(1, 1), (37, 3), (64, 64), (200, 8)])
def test_probe_read_xor_per_workgroup(n, per):
    rng = np.random.default_rng(7 + n)
    n_buf = 256
    host = rng.integers(0, 2**32, size=(n_buf, CHUNK // 4), dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    picks = rng.integers(0, n_buf, size=n)  # repeats allowed
    addr = torch.tensor(buf.data_ptr() + picks.astype(np.int64) * CHUNK, dtype=torch.int64, device="cuda")
    sink = ops.probe_read(addr, per)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    words = (n + per - 1) // per
    assert got.shape == (words, 4)
    for w in range(words):
        chunks = host[picks[w * per:(w + 1) * per]].reshape(-1, 4)
        expect = np.bitwise_xor.reduce(chunks, axis=0)
        assert np.array_equal(got[w], expect), (w, got[w], expect)
