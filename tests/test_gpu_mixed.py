"""GPU: one mixed continuous-batching step (pkv_attn_mixed_step) against the
separate calls — pkv_kv_append_paged for every new token, then
pkv_attn_prefill_chunk and pkv_attn_decode — with the pool bytes and both
outputs bit-identical, and against the oracle within 2e-3. The new tokens'
slots hold NaN before the step."""

import numpy as np
import pytest
import torch

import paged_kv_cache_430_amd as pkv
from oracle import attention

from gpu_helpers import device, new_pools

pytestmark = pytest.mark.gpu

# PKV_MIXED: "one" runs the appends, the decodes and the prefill in one
# launch (when the prefill takes the key-stream kernel); "pair" the same with
# four-wave workgroups, a prefill tile and a decode unit sharing each CU;
# "two", the default, the decode launch with the appends followed by the
# prefill launch
LAUNCHES = ["one", "pair", "two"]


def _same(launches, got, ref):
    """Outputs of the mixed step against the separate calls': bit-identical,
    except in the paired form, whose prefill runs two key streams instead of
    four and whose decodes run four waves instead of eight (other summation
    orders of the same sums)."""
    if launches == "pair":
        assert got.shape == ref.shape
        assert got.numel() == 0 or (got - ref).abs().max().item() <= 1e-4
    else:
        assert torch.equal(got, ref)


def _bf16(shape, gen, dev):
    return torch.randn(*shape, generator=gen, device=dev).to(torch.bfloat16)


def _f64(t):
    return t.float().cpu().double().numpy()


def _case(dev, chunks, dec_ctx, hq, hkv, dh, seed, bs=16):
    """chunks: (prefix P, chunk C) per prefill sequence; dec_ctx: cached tokens
    of each decode sequence before its new one. Prefixes and contexts are in
    the pool; the step's tokens are not."""
    gen = torch.Generator(device=dev).manual_seed(seed)
    rng = np.random.default_rng(seed)
    lens = [p + c for p, c in chunks] + [t + 1 for t in dec_ctx]
    nblk = [-(-t // bs) for t in lens]
    max_blocks = max(nblk)
    num_blocks = sum(nblk) + 7
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    pos = 0
    for i, n in enumerate(nblk):
        bt[i, :n] = perm[pos:pos + n]
        pos += n
    kp, vp = new_pools(num_blocks, hkv, dh, "bf16", dev, block_size=bs)
    cache = pkv.Cache(kp, vp)
    ks = [_bf16((t, hkv, dh), gen, dev) for t in lens]
    vs = [_bf16((t, hkv, dh), gen, dev) for t in lens]
    first = [p for p, _ in chunks] + list(dec_ctx)          # first position appended by the step
    for i in range(len(lens)):
        if first[i] > 0:
            s = pkv.pkv_slot_mapping(bt[i], bs, 0, first[i])
            pkv.pkv_kv_append(cache, ks[i][:first[i]].contiguous(), vs[i][:first[i]].contiguous(),
                              torch.from_numpy(s).to(dev))
    n_ch = len(chunks)
    qc = _bf16((sum(c for _, c in chunks), hq, dh), gen, dev)
    qd = _bf16((len(dec_ctx), hq, dh), gen, dev)
    new_k = torch.cat([ks[i][first[i]:] for i in range(len(lens))]).contiguous()
    new_v = torch.cat([vs[i][first[i]:] for i in range(len(lens))]).contiguous()
    n_new = [lens[i] - first[i] for i in range(len(lens))]
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    return dict(cache=cache, ks=ks, vs=vs, lens=lens, n_ch=n_ch, qc=qc, qd=qd, new_k=new_k, new_v=new_v,
                cu=t(cu), first=t(np.array(first, dtype=np.int32)), max_new=max(n_new), bt=bt, t=t,
                q_start=t(cu[:n_ch + 1]), chunk_tables=t(bt[:n_ch]), dec_tables=t(bt[n_ch:]),
                chunk_lens=t(np.array(lens[:n_ch], dtype=np.int32)),
                dec_lens=t(np.array(lens[n_ch:], dtype=np.int32)),
                max_q=max([c for _, c in chunks] or [0]), msl=max(lens[n_ch:] or [1]),
                scale=1.0 / np.sqrt(dh), n_chunk_rows=int(cu[n_ch]))


def _clone(cache):
    return pkv.Cache(cache.k.clone(), cache.v.clone())


def _separate(c, cache, pt):
    t = c["t"]
    pkv.pkv_kv_append_paged(cache, c["new_k"], c["new_v"], t(c["bt"]), c["cu"], c["first"], c["max_new"])
    out_p = out_d = None
    if c["n_ch"]:
        out_p = pkv.pkv_attn_prefill_chunk(cache, c["qc"], c["q_start"], c["chunk_tables"], c["chunk_lens"],
                                           c["max_q"], c["scale"])
    if len(c["lens"]) > c["n_ch"]:
        out_d = pkv.pkv_attn_decode(cache, c["qd"], c["dec_tables"], c["dec_lens"], c["msl"], c["scale"],
                                    partition_tokens=pt)
    return out_p, out_d


def _mixed(c, cache, pt):
    r = c["n_chunk_rows"]
    return pkv.pkv_attn_mixed_step(cache, c["scale"], c["qc"], c["new_k"][:r], c["new_v"][:r], c["q_start"],
                                   c["chunk_tables"], c["chunk_lens"], c["max_q"], c["qd"], c["new_k"][r:],
                                   c["new_v"][r:], c["dec_tables"], c["dec_lens"], c["msl"], partition_tokens=pt)


def _oracle_check(c, out_p, out_d):
    n_ch, scale = c["n_ch"], c["scale"]
    qs = c["q_start"].cpu().numpy()
    if n_ch:
        got = out_p.cpu().double().numpy()
        qc = _f64(c["qc"])
        for i in range(n_ch):
            ref = attention.prefill_chunk(qc[qs[i]:qs[i + 1]], np.transpose(_f64(c["ks"][i]), (1, 0, 2)),
                                          np.transpose(_f64(c["vs"][i]), (1, 0, 2)), scale)
            assert np.abs(got[qs[i]:qs[i + 1]] - ref).max() <= 2e-3, f"chunk {i}"
    got = out_d.cpu().double().numpy() if out_d is not None else None
    qd = _f64(c["qd"])
    for j in range(len(c["lens"]) - n_ch):
        i = n_ch + j
        ref = attention.decode(qd[j:j + 1], [np.transpose(_f64(c["ks"][i]), (1, 0, 2))],
                               [np.transpose(_f64(c["vs"][i]), (1, 0, 2))], scale)[0]
        assert np.abs(got[j] - ref).max() <= 2e-3, f"decode {j}"


@pytest.mark.parametrize("hq,hkv,dh,pt", [(32, 8, 128, 0), (32, 8, 128, 64), (16, 2, 64, 0), (8, 8, 128, 32),
                                          (32, 1, 64, 48)])
@pytest.mark.parametrize("prefill_kernel", ["tiles", "columns"])
@pytest.mark.parametrize("launches", LAUNCHES)
def test_mixed_step_matches_separate_calls(hq, hkv, dh, pt, prefill_kernel, launches, monkeypatch):
    monkeypatch.setenv("PKV_PREFILL_KERNEL", prefill_kernel)
    monkeypatch.setenv("PKV_MIXED", launches)
    dev = device()
    chunks = [(0, 1), (5, 17), (100, 64), (1000, 130), (31, 33)]
    dec_ctx = [0, 1, 15, 16, 200, 1023, 77]
    c = _case(dev, chunks, dec_ctx, hq, hkv, dh, seed=hq + 3 * hkv + dh + pt)
    ref = _clone(c["cache"])
    mix = _clone(c["cache"])
    rp, rd = _separate(c, ref, pt)
    mp, md = _mixed(c, mix, pt)
    torch.cuda.synchronize()
    assert torch.equal(mix.k.view(torch.int16), ref.k.view(torch.int16))
    assert torch.equal(mix.v.view(torch.int16), ref.v.view(torch.int16))
    _same(launches, mp, rp)
    _same(launches, md, rd)
    _oracle_check(c, mp, md)


@pytest.mark.parametrize("bs", [8, 32, 64])
@pytest.mark.parametrize("prefill_kernel", ["tiles", "columns"])
@pytest.mark.parametrize("launches", LAUNCHES)
def test_mixed_step_at_block_sizes_8_32_and_64(bs, prefill_kernel, launches, monkeypatch):
    """The mixed step on pools of 8-, 32- and 64-token blocks: chunk and
    decode tokens land inside larger blocks, or a 16-row unit spans two
    blocks; bit-identical to the separate calls. (With 8-token blocks the
    prefill takes the key-stream kernel whatever PKV_PREFILL_KERNEL says, and
    the step takes two launches.)"""
    monkeypatch.setenv("PKV_PREFILL_KERNEL", prefill_kernel)
    monkeypatch.setenv("PKV_MIXED", launches)
    dev = device()
    c = _case(dev, [(0, 1), (5, 17), (100, 64), (1000, 130), (31, 33)], [0, 1, 15, 16, 200, 1023, 77],
              32, 8, 128, seed=90 + bs, bs=bs)
    ref, mix = _clone(c["cache"]), _clone(c["cache"])
    rp, rd = _separate(c, ref, 48)
    mp, md = _mixed(c, mix, 48)
    torch.cuda.synchronize()
    assert torch.equal(mix.k.view(torch.int16), ref.k.view(torch.int16))
    assert torch.equal(mix.v.view(torch.int16), ref.v.view(torch.int16))
    _same(launches, mp, rp)
    _same(launches, md, rd)
    _oracle_check(c, mp, md)


@pytest.mark.parametrize("launches", LAUNCHES)
def test_mixed_step_chunks_only_and_decodes_only(launches, monkeypatch):
    monkeypatch.setenv("PKV_MIXED", launches)
    monkeypatch.setenv("PKV_PREFILL_KERNEL", "tiles")
    dev = device()
    # chunks only: the decode launch carries just the appending workgroups
    c = _case(dev, [(40, 100), (0, 16)], [], 32, 8, 128, seed=5)
    ref, mix = _clone(c["cache"]), _clone(c["cache"])
    rp, _ = _separate(c, ref, 0)
    mp, md = _mixed(c, mix, 0)
    torch.cuda.synchronize()
    assert md.numel() == 0
    assert torch.equal(mix.k.view(torch.int16), ref.k.view(torch.int16))
    assert torch.equal(mix.v.view(torch.int16), ref.v.view(torch.int16))
    _same(launches, mp, rp)
    _oracle_check(c, mp, None)
    # decodes only
    c = _case(dev, [], [3, 300, 4095], 32, 8, 128, seed=6)
    ref, mix = _clone(c["cache"]), _clone(c["cache"])
    _, rd = _separate(c, ref, 0)
    mp, md = _mixed(c, mix, 0)
    torch.cuda.synchronize()
    assert mp.numel() == 0
    assert torch.equal(mix.k.view(torch.int16), ref.k.view(torch.int16))
    assert torch.equal(mix.v.view(torch.int16), ref.v.view(torch.int16))
    _same(launches, md, rd)
    _oracle_check(c, None, md)


@pytest.mark.parametrize("seed", range(10))
def test_mixed_step_seeded_shapes(seed, monkeypatch):
    """Random mixed steps (head layout, head dim, block size, 1-3 chunks on
    prefixes of 0-1500 tokens, 0-12 decodes of 0-2000 cached tokens, the
    partition size) with the key-stream prefill, in the paired one launch
    (PKV_MIXED=pair, wherever it applies), the default and two launches:
    pool bytes bit-identical to the separate calls', outputs within 1e-4 of
    theirs and within 2e-3 of the oracle; two launches bit-identical."""
    monkeypatch.setenv("PKV_PREFILL_KERNEL", "tiles")
    rng = np.random.default_rng(9100 + seed)
    hq, hkv = [(32, 8), (16, 2), (8, 8), (32, 1), (64, 8), (48, 4)][int(rng.integers(6))]
    dh = [64, 128][int(rng.integers(2))]
    bs = [16, 32, 64, 8][seed % 4]
    chunks = [(int(rng.integers(0, 1501)), int(rng.integers(1, 301))) for _ in range(int(rng.integers(1, 4)))]
    dec_ctx = [int(t) for t in rng.integers(0, 2001, int(rng.integers(0, 13)))]
    pt = [0, 48, 256][int(rng.integers(3))]
    print(f"seed {seed}: {hq}/{hkv} dh{dh} bs{bs} chunks {chunks} decodes {dec_ctx} pt {pt}", flush=True)
    dev = device()
    c = _case(dev, chunks, dec_ctx, hq, hkv, dh, seed=9100 + seed, bs=bs)
    ref = _clone(c["cache"])
    rp, rd = _separate(c, ref, pt)
    for launches in ("pair", "default", "two"):
        if launches == "default":
            monkeypatch.delenv("PKV_MIXED", raising=False)
        else:
            monkeypatch.setenv("PKV_MIXED", launches)
        mix = _clone(c["cache"])
        mp, md = _mixed(c, mix, pt)
        torch.cuda.synchronize()
        assert torch.equal(mix.k.view(torch.int16), ref.k.view(torch.int16)), launches
        assert torch.equal(mix.v.view(torch.int16), ref.v.view(torch.int16)), launches
        form = "pair" if launches == "default" else launches
        _same(form, mp, rp)
        if rd is not None:
            _same(form, md, rd)
        _oracle_check(c, mp, md if rd is not None else None)


@pytest.mark.parametrize("hq,hkv,dh,pt", [(32, 8, 128, 0), (16, 2, 64, 48), (8, 8, 128, 0), (32, 1, 64, 256)])
def test_small_chunk_step_in_one_launch(hq, hkv, dh, pt, monkeypatch):
    """Chunks small enough for the prefill's column form, with fewer query
    blocks than compute units: by default appends, decodes and the query
    blocks run as one launch of the decode body, bit-identical to the
    separate calls and to the two-launch form."""
    monkeypatch.delenv("PKV_PREFILL_KERNEL", raising=False)
    dev = device()
    c = _case(dev, [(100, 20), (0, 9), (37, 3)], [0, 5, 300, 1023, 16], hq, hkv, dh, seed=hq + dh + pt)
    ref = _clone(c["cache"])
    rp, rd = _separate(c, ref, pt)
    for launches in ("default", "two"):
        if launches == "default":
            monkeypatch.delenv("PKV_MIXED", raising=False)
        else:
            monkeypatch.setenv("PKV_MIXED", launches)
        mix = _clone(c["cache"])
        mp, md = _mixed(c, mix, pt)
        torch.cuda.synchronize()
        assert torch.equal(mix.k.view(torch.int16), ref.k.view(torch.int16)), launches
        assert torch.equal(mix.v.view(torch.int16), ref.v.view(torch.int16)), launches
        assert torch.equal(mp, rp), launches
        assert torch.equal(md, rd), launches
    _oracle_check(c, mp, md)


@pytest.mark.parametrize("hq,hkv,dh", [(32, 8, 128), (16, 2, 64)])
def test_small_chunks_with_many_query_blocks_take_the_paired_launch(hq, hkv, dh, monkeypatch):
    """Chunks whose prefill alone takes the column form, with 128 query blocks
    or more: the paired launch (PKV_MIXED=pair; the default beside enough
    decode work) runs their prefill on the key-stream tiles (pool bytes
    bit-identical to the separate calls, outputs within 1e-4 of theirs and
    2e-3 of the oracle); PKV_PREFILL_KERNEL=columns keeps the column form
    (two launches, bit-identical)."""
    monkeypatch.delenv("PKV_PREFILL_KERNEL", raising=False)
    monkeypatch.setenv("PKV_MIXED", "pair")
    dev = device()
    c = _case(dev, [(200, 70), (0, 60), (513, 21)], [0, 7, 900, 2000], hq, hkv, dh, seed=hq * 5 + dh)
    ref = _clone(c["cache"])
    rp, rd = _separate(c, ref, 0)
    mix = _clone(c["cache"])
    mp, md = _mixed(c, mix, 0)
    torch.cuda.synchronize()
    assert torch.equal(mix.k.view(torch.int16), ref.k.view(torch.int16))
    assert torch.equal(mix.v.view(torch.int16), ref.v.view(torch.int16))
    _same("pair", mp, rp)
    _same("pair", md, rd)
    _oracle_check(c, mp, md)
    monkeypatch.setenv("PKV_PREFILL_KERNEL", "columns")
    mix = _clone(c["cache"])
    mp, md = _mixed(c, mix, 0)
    torch.cuda.synchronize()
    assert torch.equal(mix.k.view(torch.int16), ref.k.view(torch.int16))
    assert torch.equal(mp, rp)
    assert torch.equal(md, rd)


def test_paired_step_with_long_decode_partitions_falls_back(monkeypatch):
    """PKV_MIXED=pair with decodes whose partitions exceed the four-wave
    workgroup's 4096 tokens: the step takes two launches, bit-identical to
    the separate calls."""
    monkeypatch.setenv("PKV_MIXED", "pair")
    monkeypatch.setenv("PKV_PREFILL_KERNEL", "tiles")
    dev = device()
    c = _case(dev, [(40, 100)], [8000, 20], 32, 8, 128, seed=8)
    ref, mix = _clone(c["cache"]), _clone(c["cache"])
    rp, rd = _separate(c, ref, 8192)
    mp, md = _mixed(c, mix, 8192)
    torch.cuda.synchronize()
    assert torch.equal(mix.k.view(torch.int16), ref.k.view(torch.int16))
    assert torch.equal(mp, rp)
    assert torch.equal(md, rd)
    _oracle_check(c, mp, md)


def test_shared_prefix_step_with_sharers_decoding():
    """The shared-prefix workload with its idle sharers decoding too: S0 runs
    its 512-token chunk on 2048 cached tokens; 64 separate sequences and the 15
    other sharers (1024 shared + 1024 private tokens each) append one token and
    decode, all in one pkv_attn_mixed_step. Blocks come from the library's
    allocator: each sharer's token opens a private block (2048 is
    block-aligned, so nothing is copied), and the prefix blocks keep their 16
    references. Outputs against the oracle within 2e-3."""
    import workloads

    dev = device()
    m = workloads.shared_prefix_mixed(device=dev, sharers_decode=True)
    bs, hkv, hq, dh = 16, m.hkv, m.hq, m.head_dim
    alloc = pkv.BlockAllocator(m.num_blocks, bs, free_order=m.free_order)
    kp, vp = new_pools(m.num_blocks, hkv, dh, "bf16", dev)
    cache = pkv.Cache(kp, vp)
    max_blocks = (m.shared + m.private + m.chunk) // bs + 1

    def append(table, first, k, v):
        s = pkv.pkv_slot_mapping(table, bs, first, k.shape[0])
        pkv.pkv_kv_append(cache, k.contiguous(), v.contiguous(), torch.from_numpy(s).to(dev))

    prefix = np.full(max_blocks, -1, dtype=np.int32)
    assert alloc.reserve_append(prefix, 0, m.shared) == []
    append(prefix, 0, *m.prefix_kv)
    n_pref = m.shared // bs
    tables = []
    for i in range(m.n_share):
        t = prefix.copy()
        if i > 0:
            alloc.incref(prefix[:n_pref])
        assert alloc.reserve_append(t, m.shared, m.private) == []
        append(t, m.shared, *m.private_kv[i])
        tables.append(t)
    p0 = m.shared + m.private
    t0 = tables[0]
    assert alloc.reserve_append(t0, p0, m.chunk) == []
    n_dec = len(m.decode_ctx)
    dtabs = np.full((n_dec + m.n_share - 1, max_blocks), -1, dtype=np.int32)
    for j, ctx in enumerate(m.decode_ctx):
        ctx = int(ctx)
        alloc.reserve_append(dtabs[j], 0, ctx + 1)
        k, v = m.decode_kv[j]
        append(dtabs[j], 0, k[:ctx], v[:ctx])
    free_before = alloc.num_free()
    for i in range(1, m.n_share):
        assert alloc.reserve_append(tables[i], p0, 1) == []      # a new private block, no copy
        dtabs[n_dec + i - 1] = tables[i]
    assert alloc.num_free() == free_before - (m.n_share - 1)
    assert all(alloc.refcount(int(b)) == m.n_share for b in prefix[:n_pref])
    assert all(alloc.refcount(int(tables[i][p0 // bs])) == 1 for i in range(1, m.n_share))

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    dec_ctx = np.concatenate([m.decode_ctx, np.full(m.n_share - 1, p0)]).astype(np.int32)
    dec_q = torch.cat([m.decode_q, m.sharer_q]).contiguous()
    dec_k = torch.cat([m.decode_kv[j][0][-1:] for j in range(n_dec)] + [m.sharer_new_kv[0]]).contiguous()
    dec_v = torch.cat([m.decode_kv[j][1][-1:] for j in range(n_dec)] + [m.sharer_new_kv[1]]).contiguous()
    out_p, out_d = pkv.pkv_attn_mixed_step(
        cache, m.scale, m.chunk_q, m.chunk_kv[0].contiguous(), m.chunk_kv[1].contiguous(),
        torch.tensor([0, m.chunk], dtype=torch.int32, device=dev), t(t0[None]),
        torch.tensor([p0 + m.chunk], dtype=torch.int32, device=dev), m.chunk,
        dec_q, dec_k, dec_v, t(dtabs), t(dec_ctx + 1), max_blocks * bs)
    torch.cuda.synchronize()

    k0 = np.concatenate([_f64(m.prefix_kv[0]), _f64(m.private_kv[0][0]), _f64(m.chunk_kv[0])])
    v0 = np.concatenate([_f64(m.prefix_kv[1]), _f64(m.private_kv[0][1]), _f64(m.chunk_kv[1])])
    ref_p = attention.prefill_chunk(_f64(m.chunk_q), k0.transpose(1, 0, 2), v0.transpose(1, 0, 2), m.scale)
    assert np.abs(out_p.cpu().double().numpy() - ref_p).max() <= 2e-3
    qd = _f64(dec_q)
    gd = out_d.cpu().double().numpy()
    for j in range(n_dec):
        k, v = m.decode_kv[j]
        ref = attention.decode(qd[j:j + 1], [_f64(k).transpose(1, 0, 2)], [_f64(v).transpose(1, 0, 2)], m.scale)[0]
        assert np.abs(gd[j] - ref).max() <= 2e-3, j
    for i in range(1, m.n_share):
        j = n_dec + i - 1
        k = np.concatenate([_f64(m.prefix_kv[0]), _f64(m.private_kv[i][0]), _f64(m.sharer_new_kv[0][i - 1:i])])
        v = np.concatenate([_f64(m.prefix_kv[1]), _f64(m.private_kv[i][1]), _f64(m.sharer_new_kv[1][i - 1:i])])
        ref = attention.decode(qd[j:j + 1], [k.transpose(1, 0, 2)], [v.transpose(1, 0, 2)], m.scale)[0]
        assert np.abs(gd[j] - ref).max() <= 2e-3, i
    # the prefix blocks are unchanged by every append of the step
    gk, gv = pkv.pkv_debug_gather(cache, t(prefix[:n_pref]), m.shared)
    torch.cuda.synchronize()
    assert torch.equal(gk.cpu(), m.prefix_kv[0].cpu().permute(1, 0, 2))
    assert torch.equal(gv.cpu(), m.prefix_kv[1].cpu().permute(1, 0, 2))
