"""GPU parity of pkv_attn_decode_noalloc (the library's static split-KV
scratch, no workspace argument) against pkv_attn_decode with a caller's
workspace: identical outputs on two calls in a row, the second with a smaller
input, so the second call runs on scratch that still holds the first call's
partials. Plus the size limit, checked on the host before any launch."""

import numpy as np
import pytest
import torch

import paged_kv_cache_430_amd as pkv
import workloads

from gpu_helpers import build_cache, device, lens, tables

pytestmark = pytest.mark.gpu

STATIC_BYTES = 8 << 20


@pytest.mark.parametrize("cache_dtype,hq,hkv,dh", [("bf16", 32, 8, 128), ("fp8", 16, 2, 64), ("f32", 8, 2, 128)])
def test_noalloc_decode_matches_workspace_decode(cache_dtype, hq, hkv, dh):
    dev = device()
    big = workloads.decode_inputs("noalloc-a", 71 + dh, [4096, 1, 700, 2500, 33], hq, hkv, dh, cache_dtype, dev)
    small = workloads.decode_inputs("noalloc-b", 72 + dh, [300, 17], hq, hkv, dh, cache_dtype, dev)
    for w, pt in ((big, 64), (small, 16)):          # both split into several partitions
        need = pkv.pkv_attn_decode_workspace_bytes({"f32": 0, "bf16": 1, "fp8": 2}[cache_dtype],
                                                   w.batch, hq, hkv, dh, int(w.seq_lens.max()), pt)
        assert 0 < need <= STATIC_BYTES
        cache = build_cache(w, dev)
        bt, ln, msl = tables(w, dev), lens(w, dev), int(w.seq_lens.max())
        want = pkv.pkv_attn_decode(cache, w.q, bt, ln, msl, w.scale, partition_tokens=pt)
        got = torch.full_like(want, float("nan"))
        pkv.pkv_attn_decode_noalloc(cache, w.q, bt, ln, msl, w.scale, got, partition_tokens=pt)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{cache_dtype} pt{pt}"
        # the automatic partition as well
        want0 = pkv.pkv_attn_decode(cache, w.q, bt, ln, msl, w.scale)
        got0 = torch.full_like(want0, float("nan"))
        pkv.pkv_attn_decode_noalloc(cache, w.q, bt, ln, msl, w.scale, got0)
        torch.cuda.synchronize()
        assert torch.equal(got0, want0), f"{cache_dtype} auto"


def test_noalloc_decode_refuses_partials_beyond_the_static_scratch():
    """64 partitions of 16 tokens for 32 sequences × 32 heads × 128 need
    32·32·64·130·4 bytes (34 MB) of partials: refused before any launch, the
    output untouched."""
    dev = device()
    w = workloads.decode_inputs("noalloc-c", 73, [1024] * 32, 32, 8, 128, "bf16", dev)
    cache = build_cache(w, dev)
    need = pkv.pkv_attn_decode_workspace_bytes(1, 32, 32, 8, 128, 1024, 16)
    assert need == 32 * 32 * 64 * 130 * 4 > STATIC_BYTES
    out = torch.full((32, 32, 128), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(pkv.PKVError) as e:
        pkv.pkv_attn_decode_noalloc(cache, w.q, tables(w, dev), lens(w, dev), 1024, w.scale, out,
                                    partition_tokens=16)
    assert e.value.status == pkv.PKV_EWORKSPACE and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
