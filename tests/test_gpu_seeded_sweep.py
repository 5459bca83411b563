"""GPU: a seeded sweep of random shapes against the float64 oracle — decode
(both kernels, all cache dtypes, block sizes 16/32/64, explicit and automatic
partitions, with and without the fused append) and chunked prefill (both
kernels). Each case is drawn from numpy's default_rng(seed); the cases stay
small enough for the oracle."""

import numpy as np
import pytest
import torch

import paged_kv_cache_430_amd as pkv
import workloads

from gpu_helpers import NAN_FP8, build_cache, device, lens, tables
from test_gpu_decode import TOL, assert_close, decode_kernel, oracle_decode
from test_gpu_prefill import _prefill_case

pytestmark = pytest.mark.gpu

HEADS = [(32, 8), (8, 8), (16, 2), (32, 1), (24, 8), (64, 1), (4, 4)]


def _decode_case(seed):
    rng = np.random.default_rng(seed)
    cache_dtype = ["bf16", "fp8", "f32"][seed % 3]
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    dh = [64, 128][int(rng.integers(2))]
    bs = 16 if cache_dtype == "f32" else [16, 32, 64, 8][int(rng.integers(4))]
    b = int(rng.integers(1, 9))
    lens_ = [int(x) for x in rng.integers(1, 2500, b)]
    pt = [0, 16, 48, 256, 1024][int(rng.integers(5))]
    fused = bool(rng.integers(2)) and cache_dtype != "f32"
    return cache_dtype, hq, hkv, dh, bs, lens_, pt, fused


@pytest.mark.parametrize("seed", range(24))
def test_decode_seeded_shapes(seed):
    cache_dtype, hq, hkv, dh, bs, lens_, pt, fused = _decode_case(seed)
    dev = device()
    w = workloads.decode_inputs("sweep", 9000 + seed, lens_, hq, hkv, dh, cache_dtype, dev, block_size=bs)
    cache = build_cache(w, dev)
    ref = oracle_decode(w)
    msl = int(max(lens_))
    what = f"seed {seed}: {cache_dtype} {hq}/{hkv} dh{dh} bs{bs} pt{pt} fused={fused} lens={lens_}"
    kinv = vinv = None
    if cache_dtype == "fp8":
        kinv = torch.from_numpy(w.k_inv_scale).to(dev)
        vinv = torch.from_numpy(w.v_inv_scale).to(dev)
    kerns = ["matrix"] if bs != 16 else (["vector"] if cache_dtype == "f32" else ["vector", "matrix"])
    for kern in kerns:
        with decode_kernel(kern):
            if fused:   # the last token's slot starts as NaN; the call writes it
                last = torch.tensor([int(c) - 1 for c in w.cu_seqlens[1:]], device=dev)
                nan = NAN_FP8 if cache_dtype == "fp8" else float("nan")
                for i, t in enumerate(lens_):
                    phys, off = int(w.block_tables[0, i, (t - 1) // bs]), (t - 1) % bs
                    cache.k[phys, :, off, :] = nan
                    cache.v[phys, :, off, :] = nan
                out = pkv.pkv_attn_decode_append(cache, w.k[last].contiguous(), w.v[last].contiguous(), w.q,
                                                 tables(w, dev), lens(w, dev), msl, w.scale, partition_tokens=pt,
                                                 k_inv_scale=kinv, v_inv_scale=vinv)
            else:
                out = pkv.pkv_attn_decode(cache, w.q, tables(w, dev), lens(w, dev), msl, w.scale,
                                          partition_tokens=pt)
            torch.cuda.synchronize()
        assert_close(out.cpu().double().numpy(), ref, TOL[cache_dtype], f"{kern} {what}")


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("prefill_kernel", ["tiles", "tiles128", "tiles256", "columns"])
def test_prefill_seeded_shapes(seed, prefill_kernel, monkeypatch):
    monkeypatch.setenv("PKV_PREFILL_KERNEL", prefill_kernel)
    rng = np.random.default_rng(7000 + seed)
    hq, hkv = [(32, 8), (8, 8), (16, 8), (32, 4), (4, 1), (64, 8), (48, 4)][int(rng.integers(7))]
    dh = [64, 128][int(rng.integers(2))]
    n = int(rng.integers(1, 5))
    seqs = [(int(rng.integers(0, 1500)), int(rng.integers(1, 200))) for _ in range(n)]
    bs = [16, 32, 64, 8][seed % 4]
    err, rel = _prefill_case(device(), seqs, hq, hkv, dh, seed=7000 + seed, bs=bs)
    assert err <= 2e-3, f"seed {seed} {hq}/{hkv} dh{dh} bs{bs} {seqs}: max-abs {err:.3e}"
