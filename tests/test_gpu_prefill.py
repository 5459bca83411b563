"""GPU parity: causal chunked prefill over a paged prefix, and the mixed
shared-prefix step (allocator + copy-on-write + append + prefill + decode)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_430_amd as pkv
import workloads
from oracle import attention

from gpu_helpers import device, new_pools, parity

pytestmark = pytest.mark.gpu

PREFILL_KERNELS = ["tiles", "tiles128", "tiles256", "tiles16", "columns"]


@pytest.fixture(params=PREFILL_KERNELS)
def prefill_kernel(request, monkeypatch):
    """Every prefill kernel (PKV_PREFILL_KERNEL): the key-stream tile kernel
    with 64, 128 and 256 query rows per workgroup (256: head dim 128; at 64
    the call runs 128), the 16-row tile kernel, and the matrix-core decode
    kernel with (head, query) columns."""
    monkeypatch.setenv("PKV_PREFILL_KERNEL", request.param)
    return request.param


def _bf16(shape, gen, dev):
    return torch.randn(*shape, generator=gen, device=dev).to(torch.bfloat16)


def _f64(t):
    return t.float().cpu().double().numpy()


def _prefill_case(dev, seqs, hq, hkv, dh, seed, bs=16, label=None, norm_tol=None, shape_q=None):
    """seqs: list of (prefix P, chunk C); bs: tokens per pool block. Checks
    max-abs <= 2e-3 (and the normalised error against norm_tol) and returns
    (max-abs error, normalised error). shape_q(i, q, k), if given, rewrites
    sequence i's queries (C, Hq, Dh) in place from its keys (P+C, Hkv, Dh)."""
    gen = torch.Generator(device=dev).manual_seed(seed)
    rng = np.random.default_rng(seed)
    total_blocks = sum(-(-(p + c) // bs) for p, c in seqs)
    perm = rng.permutation(total_blocks + 5).astype(np.int32)
    max_blocks = max(-(-(p + c) // bs) for p, c in seqs)
    bt = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
    kp, vp = new_pools(total_blocks + 5, hkv, dh, "bf16", dev, block_size=bs)
    cache = pkv.Cache(kp, vp)
    pos = 0
    qs, ks, vs = [], [], []
    for i, (p, c) in enumerate(seqs):
        nb = -(-(p + c) // bs)
        bt[i, :nb] = perm[pos:pos + nb]
        pos += nb
        k = _bf16((p + c, hkv, dh), gen, dev)
        v = _bf16((p + c, hkv, dh), gen, dev)
        slots = pkv.pkv_slot_mapping(bt[i], bs, 0, p + c)
        pkv.pkv_kv_append(cache, k, v, torch.from_numpy(slots).to(dev))
        qs.append(_bf16((c, hq, dh), gen, dev))
        if shape_q is not None:
            shape_q(i, qs[-1], k)
        ks.append(k)
        vs.append(v)
    q = torch.cat(qs).contiguous()
    q_start = np.concatenate([[0], np.cumsum([c for _, c in seqs])]).astype(np.int32)
    seq_lens = np.array([p + c for p, c in seqs], dtype=np.int32)
    scale = 1.0 / np.sqrt(dh)
    out = pkv.pkv_attn_prefill_chunk(cache, q, torch.from_numpy(q_start).to(dev), torch.from_numpy(bt).to(dev),
                                     torch.from_numpy(seq_lens).to(dev), max(c for _, c in seqs), scale)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    refs, gots = {}, {}
    for i, (p, c) in enumerate(seqs):
        refs[i] = attention.prefill_chunk(_f64(qs[i]), np.transpose(_f64(ks[i]), (1, 0, 2)),
                                          np.transpose(_f64(vs[i]), (1, 0, 2)), scale)
        gots[i] = got[q_start[i]:q_start[i + 1]]
    import os
    label = label or f"prefill {os.environ.get('PKV_PREFILL_KERNEL', 'auto')} {hq}/{hkv} dh{dh} bs{bs} {seqs}"
    return parity(label, gots, refs, 2e-3, norm_tol)


@pytest.mark.parametrize("hq,hkv,dh", [(32, 8, 128), (8, 8, 128), (16, 8, 64), (32, 4, 128), (4, 1, 64)])
def test_ragged_chunks_one_call(hq, hkv, dh, prefill_kernel):
    dev = device()
    seqs = [(0, 1), (0, 17), (5, 16), (100, 64), (33, 100), (2048, 3), (0, 130)]
    err, rel = _prefill_case(dev, seqs, hq, hkv, dh, seed=hq * 7 + dh)
    assert err <= 2e-3, f"max-abs {err:.3e}"


@pytest.mark.parametrize("seqs", [[(0, 2048)], [(100, 64), (0, 1), (3000, 700), (5, 1500)]])
@pytest.mark.parametrize("kernel", ["auto", "tiles"])
def test_tile_kernel_many_query_tiles(seqs, kernel, monkeypatch):
    """Chunks with rows enough for several rounds of tile kernel workgroups:
    the library's own choice (128 rows per workgroup for the first, 256 for
    the second) and the 64-row form."""
    if kernel == "auto":
        monkeypatch.delenv("PKV_PREFILL_KERNEL", raising=False)
    else:
        monkeypatch.setenv("PKV_PREFILL_KERNEL", kernel)
    dev = device()
    err, rel = _prefill_case(dev, seqs, 32, 8, 128, seed=11 + len(seqs))
    assert err <= 2e-3, f"max-abs {err:.3e}"


@pytest.mark.parametrize("kernel", ["tiles", "tiles128", "tiles256"])
@pytest.mark.parametrize("hq,hkv,dh", [(32, 8, 128), (16, 8, 64)])
def test_eight_token_blocks_every_stream_form(kernel, hq, hkv, dh, monkeypatch):
    """Pools of 8-token blocks under the key-stream kernel's 64-, 128- and
    256-row forms (256: head dim 128; at 64 the call runs 128): chunks long
    enough for several table batches (32 tiles each per stream), ragged
    prefixes and chunk ends inside blocks."""
    monkeypatch.setenv("PKV_PREFILL_KERNEL", kernel)
    dev = device()
    seqs = [(100, 64), (0, 1), (3000, 700), (5, 1500), (13, 29)]
    err, rel = _prefill_case(dev, seqs, hq, hkv, dh, seed=808 + dh, bs=8)
    assert err <= 2e-3, f"max-abs {err:.3e}"
    assert rel < 5e-2


def test_long_table_and_small_chunk(prefill_kernel):
    """A small chunk on a table longer than the column form takes (8192
    tokens): the library runs the tile kernel whatever PKV_PREFILL_KERNEL says."""
    dev = device()
    err, rel = _prefill_case(dev, [(9000, 20), (8170, 30)], 32, 8, 128, seed=77)
    assert err <= 2e-3, f"max-abs {err:.3e}"


def test_512_chunk_on_2048_tokens_full_size(prefill_kernel):
    dev = device()
    _prefill_case(dev, [(2048, 512)], 32, 8, 128, seed=4304, label=f"prefill {prefill_kernel} cfg4 chunk C=512 P=2048",
                  norm_tol=1e-4)


@pytest.mark.parametrize("bs", [8, 32, 64])
@pytest.mark.parametrize("hq,hkv,dh", [(32, 8, 128), (16, 8, 64), (4, 1, 64)])
def test_ragged_chunks_at_block_sizes_8_32_and_64(bs, hq, hkv, dh, prefill_kernel):
    """The prefill kernels on pools of 8-, 32- and 64-token blocks: a 16-row
    unit is part of a pool block (rows (u mod bs/16)·16 of entry u / (bs/16)),
    or with 8-token blocks the rows of entries 2u and 2u+1 (only the
    key-stream kernel takes those: the other settings of PKV_PREFILL_KERNEL
    fall back to it); chunks and prefixes that start and end inside blocks."""
    dev = device()
    seqs = [(0, 1), (0, 17), (5, 16), (100, 64), (33, 100), (2048, 3), (0, 130), (40, 9)]
    err, rel = _prefill_case(dev, seqs, hq, hkv, dh, seed=70 + bs + dh, bs=bs)
    assert err <= 2e-3, f"max-abs {err:.3e}"
    assert rel < 5e-2


def test_shared_prefix_mixed_step(prefill_kernel):
    """16 sequences share 1024 prefix tokens (64 full blocks, refcount 16), each
    owns 1024 more; S0 appends and attends a 512-token chunk; 64 other
    sequences append one token and decode. Blocks come from the library's
    allocator with a seeded free order."""
    dev = device()
    m = workloads.shared_prefix_mixed(device=dev)
    bs, hkv, hq, dh = 16, m.hkv, m.hq, m.head_dim
    alloc = pkv.BlockAllocator(m.num_blocks, bs, free_order=m.free_order)
    kp, vp = new_pools(m.num_blocks, hkv, dh, "bf16", dev)
    cache = pkv.Cache(kp, vp)
    max_blocks = (m.shared + m.private + m.chunk) // bs + 1

    def append(table, first, k, v):
        s = pkv.pkv_slot_mapping(table, bs, first, k.shape[0])
        pkv.pkv_kv_append(cache, k.contiguous(), v.contiguous(), torch.from_numpy(s).to(dev))

    # shared prefix, written once
    prefix = np.full(max_blocks, -1, dtype=np.int32)
    assert alloc.reserve_append(prefix, 0, m.shared) == []
    append(prefix, 0, *m.prefix_kv)
    n_pref = m.shared // bs
    tables = []
    for i in range(m.n_share):
        t = prefix.copy()
        if i > 0:
            alloc.incref(prefix[:n_pref])
        assert alloc.reserve_append(t, m.shared, m.private) == []     # block-aligned: no copy
        append(t, m.shared, *m.private_kv[i])
        tables.append(t)
    assert all(alloc.refcount(int(b)) == m.n_share for b in prefix[:n_pref])
    # S0's chunk
    t0 = tables[0]
    p0 = m.shared + m.private
    assert alloc.reserve_append(t0, p0, m.chunk) == []
    append(t0, p0, *m.chunk_kv)
    # 64 decode sequences: context, then one appended token each
    dtabs = np.full((len(m.decode_ctx), max_blocks), -1, dtype=np.int32)
    for j, ctx in enumerate(m.decode_ctx):
        ctx = int(ctx)
        alloc.reserve_append(dtabs[j], 0, ctx)
        k, v = m.decode_kv[j]
        append(dtabs[j], 0, k[:ctx], v[:ctx])
        alloc.reserve_append(dtabs[j], ctx, 1)
        append(dtabs[j], ctx, k[ctx:], v[ctx:])
    scale = m.scale
    out_p = pkv.pkv_attn_prefill_chunk(cache, m.chunk_q, torch.tensor([0, m.chunk], dtype=torch.int32, device=dev),
                                       torch.from_numpy(t0[None]).to(dev),
                                       torch.tensor([p0 + m.chunk], dtype=torch.int32, device=dev), m.chunk, scale)
    dl = torch.from_numpy((m.decode_ctx + 1).astype(np.int32)).to(dev)
    out_d = pkv.pkv_attn_decode(cache, m.decode_q, torch.from_numpy(dtabs).to(dev), dl, max_blocks * bs, scale)
    torch.cuda.synchronize()
    # oracle over contiguous K/V
    k0 = np.concatenate([_f64(m.prefix_kv[0]), _f64(m.private_kv[0][0]), _f64(m.chunk_kv[0])])
    v0 = np.concatenate([_f64(m.prefix_kv[1]), _f64(m.private_kv[0][1]), _f64(m.chunk_kv[1])])
    ref_p = attention.prefill_chunk(_f64(m.chunk_q), k0.transpose(1, 0, 2), v0.transpose(1, 0, 2), scale)
    parity(f"cfg4 chunk via prefill {prefill_kernel}", out_p.cpu().double().numpy(), ref_p, 2e-3, 1e-4)
    qd = _f64(m.decode_q)
    gd = out_d.cpu().double().numpy()
    refs = {}
    for j in range(len(m.decode_ctx)):
        k, v = m.decode_kv[j]
        refs[j] = attention.decode(qd[j:j + 1], [_f64(k).transpose(1, 0, 2)], [_f64(v).transpose(1, 0, 2)], scale)[0]
    parity("cfg4 64 decodes (matrix)", {j: gd[j] for j in refs}, refs, 2e-3, 1e-4)
    # another sharer's view of the prefix is untouched by S0's appends
    k1 = torch.from_numpy(tables[1][:n_pref].copy()).to(dev)
    gk, _ = pkv.pkv_debug_gather(cache, k1, m.shared)
    torch.cuda.synchronize()
    assert torch.equal(gk.cpu(), m.prefix_kv[0].cpu().permute(1, 0, 2))


def test_copy_on_write_of_shared_partial_tail():
    """Two sequences share a half-filled tail; the writer gets a private copy
    (allocator + copy_blocks) and the other sequence still reads its own data."""
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(9)
    alloc = pkv.BlockAllocator(16, 16)
    kp, vp = new_pools(16, 2, 128, "bf16", dev)
    cache = pkv.Cache(kp, vp)
    ta = np.full(4, -1, dtype=np.int32)
    alloc.reserve_append(ta, 0, 24)
    k = _bf16((26, 2, 128), gen, dev)
    v = _bf16((26, 2, 128), gen, dev)
    pkv.pkv_kv_append(cache, k[:24], v[:24], torch.from_numpy(pkv.pkv_slot_mapping(ta, 16, 0, 24)).to(dev))
    alloc.incref(ta[:2])
    tb = ta.copy()
    cow = alloc.reserve_append(ta, 24, 2)
    assert len(cow) == 1
    src, dst = cow[0]
    pkv.pkv_copy_blocks(cache, torch.tensor([src], dtype=torch.int32, device=dev),
                        torch.tensor([dst], dtype=torch.int32, device=dev))
    kb_new = _bf16((1, 2, 128), gen, dev)
    pkv.pkv_kv_append(cache, k[24:], v[24:], torch.from_numpy(pkv.pkv_slot_mapping(ta, 16, 24, 2)).to(dev))
    gk_a, _ = pkv.pkv_debug_gather(cache, torch.from_numpy(ta[:2].copy()).to(dev), 26)
    gk_b, _ = pkv.pkv_debug_gather(cache, torch.from_numpy(tb[:2].copy()).to(dev), 24)
    torch.cuda.synchronize()
    assert torch.equal(gk_a.cpu(), k.cpu().permute(1, 0, 2))
    assert torch.equal(gk_b.cpu(), k[:24].cpu().permute(1, 0, 2))
    # B's tail slots 24, 25 were never written in its (original) block
    assert torch.isnan(kp[int(tb[1]), :, 8:].float()).all()
    del kb_new


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_blocks_missing_from_the_table_contribute_nothing(bs, prefill_kernel):
    """A table entry of −1, or an id outside the pool, inside a sequence: the
    tokens of that block are not attended to (the library's reading of an id
    that names no pool block), by either prefill kernel. The oracle attends
    over the remaining keys only, in their logical order. With 8-token blocks
    the missing entries are the second half of a 16-row unit (block 1, 5) and
    the first half of one (block 2)."""
    dev = device()
    gen = torch.Generator(device=dev).manual_seed(21 + bs)
    hq, hkv, dh = 32, 8, 128
    seqs = [(100, 40), (300, 64), (0, 90)]
    nb_pool = 64 if bs >= 16 else 96
    kp, vp = new_pools(nb_pool, hkv, dh, "bf16", dev, block_size=bs)
    cache = pkv.Cache(kp, vp)
    max_blocks = max(-(-(p + c) // bs) for p, c in seqs)
    bt = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
    perm = np.random.default_rng(bs).permutation(nb_pool).astype(np.int32)
    missing = {0: {1: -1}, 1: {2: nb_pool + 7, 5: -1}, 2: {}}       # sequence -> {logical block: bad id}
    pos, qs, refs = 0, [], {}
    for i, (p, c) in enumerate(seqs):
        t = p + c
        nb = -(-t // bs)
        bt[i, :nb] = perm[pos:pos + nb]
        pos += nb
        k = _bf16((t, hkv, dh), gen, dev)
        v = _bf16((t, hkv, dh), gen, dev)
        pkv.pkv_kv_append(cache, k, v, torch.from_numpy(pkv.pkv_slot_mapping(bt[i], bs, 0, t)).to(dev))
        for lb, bad in missing[i].items():
            bt[i, lb] = bad
        keep = np.array([j // bs not in missing[i] for j in range(t)])
        q = _bf16((c, hq, dh), gen, dev)
        qs.append(q)
        # query at position p + r sees the kept keys j <= p + r: in the kept
        # keys' own order those are the first (#kept up to p + r) of them
        q_pos = np.cumsum(keep)[p:] - 1
        kk = np.transpose(_f64(k)[keep], (1, 0, 2))
        vv = np.transpose(_f64(v)[keep], (1, 0, 2))
        refs[i] = np.transpose(attention.causal_attention(np.transpose(_f64(q), (1, 0, 2)), kk, vv, q_pos,
                                                          1.0 / np.sqrt(dh)), (1, 0, 2))
    q_start = np.concatenate([[0], np.cumsum([c for _, c in seqs])]).astype(np.int32)
    out = pkv.pkv_attn_prefill_chunk(cache, torch.cat(qs).contiguous(), torch.from_numpy(q_start).to(dev),
                                     torch.from_numpy(bt).to(dev),
                                     torch.tensor([p + c for p, c in seqs], dtype=torch.int32, device=dev),
                                     max(c for _, c in seqs), 1.0 / np.sqrt(dh))
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    parity(f"prefill {prefill_kernel} missing blocks bs{bs}", {i: got[q_start[i]:q_start[i + 1]] for i in refs},
           refs, 2e-3)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_scores_far_above_the_running_base(sign, prefill_kernel):
    """Queries equal to ±40× one key in a late tile: that key's score exceeds
    every earlier one by hundreds of powers of two (the kernel keeps a running
    base per row and must rescale, not overflow), or falls far below all
    others (its weight underflows to zero). Rows are spread over the chunk and
    over the query heads of each KV head."""
    dev = device()
    hq, hkv, dh = 32, 8, 128
    group = hq // hkv

    def shape_q(i, q, k):
        rng = np.random.default_rng(77 + i)
        c = q.shape[0]
        p = k.shape[0] - c
        for r in range(0, c, 29):
            h = int(rng.integers(hq))
            t = int(rng.integers(min(p + r, 100), p + r + 1))   # a key the row sees
            q[r, h] = (sign * 40.0 * k[t, h // group].float()).to(torch.bfloat16)

    _prefill_case(dev, [(2048, 512), (700, 300)], hq, hkv, dh, seed=41, shape_q=shape_q)
