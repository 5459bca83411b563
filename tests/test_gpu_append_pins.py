"""GPU parity of every path that writes the pool, pinned directly to the
oracle's paging (slot formula and per-token scatter) and fp8 codec: the
decode step's append fused into the decode launch (the benchmarked step),
the fused slot-mapping append (the prefill chunks' and the mixed step's
path), and a table entry too large for a 32-bit slot."""

import numpy as np
import pytest
import torch

import paged_kv_cache_430_amd as pkv
import workloads
from oracle import fp8 as ofp8
from oracle import paging

from gpu_helpers import NAN_FP8, bf16_bits, build_cache, device, lens, new_pools, tables

pytestmark = pytest.mark.gpu


def _pool_elems(t, cache_dtype):
    """Host copy of a pool in its stored element type (uint8 / uint16 / uint32)."""
    view = {"fp8": torch.uint8, "bf16": torch.int16, "f32": torch.int32}[cache_dtype]
    a = t.contiguous().view(view).cpu().numpy()
    return a.view({"fp8": np.uint8, "bf16": np.uint16, "f32": np.uint32}[cache_dtype])


def _stored(x, cache_dtype, inv=None):
    """Oracle's stored elements for new tokens x [N, Hkv, Dh] (torch, bf16 or f32):
    the bits themselves for a copy, per-head e4m3 codes for fp8."""
    if cache_dtype == "bf16":
        return bf16_bits(x)
    if cache_dtype == "f32":
        return x.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)
    hkv = x.shape[1]
    if x.dtype == torch.bfloat16:
        b = bf16_bits(x)
        return np.stack([ofp8.quantize_bf16_bits(b[:, h, :], inv[h]) for h in range(hkv)], axis=1)
    f = x.float().cpu().numpy()
    return np.stack([ofp8.quantize(f[:, h, :], inv[h]) for h in range(hkv)], axis=1)


@pytest.mark.parametrize("cache_dtype,in_dtype,hq,hkv,dh,bs", [
    ("bf16", "bf16", 32, 8, 128, 16), ("bf16", "bf16", 8, 2, 64, 8), ("bf16", "bf16", 32, 1, 128, 64),
    ("fp8", "bf16", 32, 8, 128, 16), ("fp8", "bf16", 16, 2, 64, 32), ("fp8", "f32", 16, 2, 64, 16),
    ("fp8", "bf16", 32, 8, 128, 8),
])
def test_decode_append_pool_bytes_match_oracle(cache_dtype, in_dtype, hq, hkv, dh, bs):
    """pkv_attn_decode_append (the matrix-core split kernel writing each new
    token itself) leaves the pool equal, byte for byte, to the oracle's append
    of the stored values at the slots of positions T_b − 1; every other byte
    is unchanged."""
    dev = device()
    lens_ = [1, 2, 16, 17, 33, 500, 1024]
    w = workloads.decode_inputs("pin", 501 + dh + hq + bs, lens_, hq, hkv, dh, cache_dtype, dev, block_size=bs)
    cache = build_cache(w, dev)
    last = torch.tensor([int(c) - 1 for c in w.cu_seqlens[1:]], device=dev)
    dt = torch.float32 if in_dtype == "f32" else torch.bfloat16
    k_new, v_new = w.k[last].to(dt).contiguous(), w.v[last].to(dt).contiguous()
    nan = NAN_FP8 if cache_dtype == "fp8" else float("nan")
    slots = []
    for b, t in enumerate(lens_):                 # the new token's slot holds NaN before the call
        s = paging.slot_of(w.block_tables[0, b], t - 1, bs)
        slots.append(s)
        cache.k[s // bs, :, s % bs, :] = nan
        cache.v[s // bs, :, s % bs, :] = nan
    want_k, want_v = _pool_elems(cache.k, cache_dtype), _pool_elems(cache.v, cache_dtype)
    kinv = vinv = None
    if cache_dtype == "fp8":
        kinv = torch.from_numpy(w.k_inv_scale).to(dev)
        vinv = torch.from_numpy(w.v_inv_scale).to(dev)
    paging.append(want_k, _stored(k_new, cache_dtype, w.k_inv_scale), slots, bs)
    paging.append(want_v, _stored(v_new, cache_dtype, w.v_inv_scale), slots, bs)
    out = pkv.pkv_attn_decode_append(cache, k_new, v_new, w.q, tables(w, dev), lens(w, dev), max(lens_), w.scale,
                                     partition_tokens=48, k_inv_scale=kinv, v_inv_scale=vinv)
    torch.cuda.synchronize()
    assert np.array_equal(_pool_elems(cache.k, cache_dtype), want_k)
    assert np.array_equal(_pool_elems(cache.v, cache_dtype), want_v)
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("cache_dtype,in_dtype,dh,bs", [("bf16", "bf16", 128, 16), ("f32", "f32", 64, 16),
                                                        ("fp8", "bf16", 128, 16), ("fp8", "f32", 64, 32),
                                                        ("bf16", "bf16", 64, 8), ("bf16", "bf16", 128, 64)])
def test_kv_append_paged_pool_bytes_match_oracle(cache_dtype, in_dtype, dh, bs):
    """pkv_kv_append_paged against the oracle's slot formula and append:
    ragged new-token counts (0 included), block crossings, positions on
    unallocated entries or past the table (skipped, slot −1)."""
    dev = device()
    rng = np.random.default_rng(600 + dh + bs)
    s, mb, hkv, nblocks = 9, 7, 2, 80
    tabs = np.full((s, mb), -1, dtype=np.int32)
    perm = rng.permutation(nblocks).astype(np.int32)
    firsts, news, k = [], [], 0
    for i in range(s):
        nb = int(rng.integers(1, mb + 1))
        tabs[i, :nb] = perm[k:k + nb]
        k += nb
        firsts.append(int(rng.integers(0, nb * bs)))
        news.append(int(rng.integers(0, 2 * bs + 8)) if i != 3 else 0)
    cu = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    n = int(cu[-1])
    dt = torch.float32 if in_dtype == "f32" else torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(8 + dh)
    kn = torch.randn(n, hkv, dh, generator=g, device=dev).to(dt)
    vn = torch.randn(n, hkv, dh, generator=g, device=dev).to(dt)
    kinv_h = np.array([1.7, 0.3], dtype=np.float32)
    vinv_h = np.array([0.9, 2.5], dtype=np.float32)
    kinv = vinv = ksc = vsc = None
    if cache_dtype == "fp8":
        kinv, vinv = torch.from_numpy(kinv_h).to(dev), torch.from_numpy(vinv_h).to(dev)
        ksc, vsc = 1.0 / kinv, 1.0 / vinv
    kp, vp = new_pools(nblocks, hkv, dh, cache_dtype, dev, block_size=bs)
    want_k, want_v = _pool_elems(kp, cache_dtype), _pool_elems(vp, cache_dtype)
    slots = []                                    # the oracle's slots; −1 where nothing is allocated
    for i in range(s):
        for j in range(news[i]):
            pos = firsts[i] + j
            lb = pos // bs
            slots.append(paging.slot_of(tabs[i], pos, bs) if lb < mb and tabs[i, lb] >= 0 else -1)
    paging.append(want_k, _stored(kn, cache_dtype, kinv_h), slots, bs)
    paging.append(want_v, _stored(vn, cache_dtype, vinv_h), slots, bs)
    out_slots = torch.full((n,), -7, dtype=torch.int32, device=dev)
    pkv.pkv_kv_append_paged(pkv.Cache(kp, vp, ksc, vsc), kn, vn, torch.from_numpy(tabs).to(dev),
                            torch.from_numpy(cu).to(dev), torch.tensor(firsts, dtype=torch.int32, device=dev),
                            max(news), kinv, vinv, out_slots)
    torch.cuda.synchronize()
    assert out_slots.cpu().numpy().tolist() == slots
    assert np.array_equal(_pool_elems(kp, cache_dtype), want_k)
    assert np.array_equal(_pool_elems(vp, cache_dtype), want_v)


@pytest.mark.parametrize("bs", [16, 64])
def test_table_id_too_large_for_a_32_bit_slot_is_skipped(bs):
    """A table entry whose slot id·bs + offset exceeds 2^31 − 1 (here one that
    would wrap, in 32-bit arithmetic, onto block 3 of the pool) names no pool
    block: its tokens get slot −1 and the pool is left unchanged."""
    dev = device()
    huge = (1 << 32) // bs + 3                    # huge·bs wraps to 3·bs modulo 2^32
    assert huge < 2 ** 31
    nblocks, hkv, dh = 8, 2, 64
    tabs = torch.tensor([[huge, 1], [2, huge]], dtype=torch.int32, device=dev)
    cu = torch.tensor([0, 3, 5], dtype=torch.int32, device=dev)
    first = torch.tensor([0, bs], dtype=torch.int32, device=dev)      # seq 1 writes into its entry 1 (huge)
    kn = torch.randn(5, hkv, dh, device=dev).to(torch.bfloat16)
    kp, vp = new_pools(nblocks, hkv, dh, "bf16", dev, block_size=bs)
    before = _pool_elems(kp, "bf16").copy()
    out_slots = torch.full((5,), -7, dtype=torch.int32, device=dev)
    pkv.pkv_kv_append_paged(pkv.Cache(kp, vp), kn, kn, tabs, cu, first, 3, out_slots=out_slots)
    dev_slots = pkv.pkv_slot_mapping_device(tabs, cu, first, 5, block_size=bs)
    torch.cuda.synchronize()
    assert out_slots.cpu().numpy().tolist() == [-1] * 5
    assert dev_slots.cpu().numpy().tolist() == [-1] * 5
    assert np.array_equal(_pool_elems(kp, "bf16"), before)
    assert np.array_equal(_pool_elems(vp, "bf16"), before)
