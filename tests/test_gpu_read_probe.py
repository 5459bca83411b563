"""GPU: the streaming-read probe (pkv_debug_stream_read) reads exactly the
listed 4 KiB tiles: each workgroup's XOR of the dwords it read equals the XOR
numpy computes over the same tiles; ids outside the buffer are skipped."""

import numpy as np
import pytest
import torch

import paged_kv_cache_430_amd as pkv

from gpu_helpers import device

pytestmark = pytest.mark.gpu


def _expected(words, ids, nwg):
    n = len(ids)
    out = np.zeros(nwg, dtype=np.uint32)
    for i in range(nwg):
        lo, hi = n * i // nwg, n * (i + 1) // nwg
        acc = np.uint32(0)
        for t in ids[lo:hi]:
            if 0 <= t < words.shape[0]:
                acc ^= np.bitwise_xor.reduce(words[t])
        out[i] = acc
    return out


@pytest.mark.parametrize("n_buf,order,nwg", [(300, "perm", 7), (300, "contig", 1), (1000, "perm", 256),
                                             (64, "invalid", 5), (129, "contig", 130)])
def test_stream_read_reads_the_listed_tiles(n_buf, order, nwg):
    dev = device()
    rng = np.random.default_rng(n_buf + nwg)
    words = rng.integers(0, 2 ** 32, size=(n_buf, 1024), dtype=np.uint32)
    if order == "perm":
        ids = rng.permutation(n_buf)
    elif order == "contig":
        ids = np.arange(n_buf)
    else:   # repeats and ids outside the buffer, which are skipped
        ids = np.concatenate([rng.integers(-3, n_buf + 3, size=200), [-1, n_buf, 2 ** 30]])
    ids = ids.astype(np.int32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = pkv.pkv_debug_stream_read(buf, torch.from_numpy(ids).to(dev), nwg)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, _expected(words, ids, nwg))
