"""Seeded synthetic inputs for the paged-attention workloads.

This module only draws numbers: query/key/value tensors, sequence lengths,
block tables and allocator free orders, from fixed seeds. It contains none of
the attention, paging or quantisation arithmetic; both the CPU oracle side of a
test and the GPU library side consume what it returns.

Recipe (one per named workload):
* values are N(0, 1), drawn in fp32 with `torch.randn` from a seeded
  `torch.Generator` on the requested device, then rounded to bf16 (RNE) when
  the workload is bf16 or fp8;
* lengths, block tables and free orders come from
  `numpy.random.default_rng(seed)`; a block table is a random permutation of a
  pool sized to the total number of blocks, handed out to sequences in order;
* fp8 workloads also carry per-KV-head calibration scales amax/448 (one for K,
  one for V) and their fp32 reciprocals — static inputs to both sides.

Token tensors are packed varlen, token-major: [ΣT, Hkv, Dh], with
`cu_seqlens` giving each sequence's slice, the layout a projection produces and
the append step consumes.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

SEEDS = {"single_seq_f32": 4301, "gqa_b32": 4302, "long_context": 4303, "shared_prefix_mixed": 4304,
         "head_layouts_t8192": 4305}
BLOCK_SIZE = 16


def _ceil_div(a, b):
    return -(-int(a) // int(b))


def _randn(shape, gen, device, dtype):
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if dtype in ("bf16", "fp8"):
        x = x.to(torch.bfloat16)
    return x


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


@dataclass
class DecodeInputs:
    name: str
    seed: int
    batch: int
    hq: int
    hkv: int
    head_dim: int
    block_size: int
    cache_dtype: str                 # "f32", "bf16" or "fp8" (stored dtype)
    seq_lens: np.ndarray             # int32 [B], tokens visible to the decode step
    cu_seqlens: np.ndarray           # int64 [B+1]
    block_tables: np.ndarray         # int32 [copies, B, max_blocks], -1 unused
    num_blocks: int                  # pool size (all copies)
    q: torch.Tensor                  # [B, Hq, Dh] (fp32 or bf16)
    k: torch.Tensor                  # [ΣT, Hkv, Dh] (fp32 or bf16)
    v: torch.Tensor
    scale: float
    k_scale: Optional[np.ndarray] = None     # fp32 [Hkv], fp8 only
    v_scale: Optional[np.ndarray] = None
    k_inv_scale: Optional[np.ndarray] = None
    v_inv_scale: Optional[np.ndarray] = None

    @property
    def max_blocks(self):
        return self.block_tables.shape[2]

    @property
    def copies(self):
        return self.block_tables.shape[0]

    def seq_k(self, b):
        return self.k[int(self.cu_seqlens[b]):int(self.cu_seqlens[b + 1])]

    def seq_v(self, b):
        return self.v[int(self.cu_seqlens[b]):int(self.cu_seqlens[b + 1])]


def _fp8_scales(x, hkv):
    """Per-head amax/448 calibration scales and their fp32 reciprocals."""
    amax = x.float().abs().amax(dim=(0, 2)).cpu().numpy().astype(np.float32)
    amax = np.maximum(amax, np.float32(1e-12))
    scale = (amax / np.float32(448.0)).astype(np.float32)
    inv = (np.float32(1.0) / scale).astype(np.float32)
    assert scale.shape == (hkv,)
    return scale, inv


def decode_inputs(name, seed, seq_lens, hq, hkv, head_dim, cache_dtype, device,
                  block_size=BLOCK_SIZE, copies=1, rng=None, extra_blocks=0):
    """Generic decode batch: values on `device`, tables from numpy."""
    rng = np.random.default_rng(seed) if rng is None else rng
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    b = len(seq_lens)
    nblk = [_ceil_div(t, block_size) for t in seq_lens]
    per_copy = int(sum(nblk))
    max_blocks = max(1, max(nblk) if b else 1)
    num_blocks = per_copy * copies + extra_blocks
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((copies, b, max_blocks), -1, dtype=np.int32)
    pos = 0
    for c in range(copies):
        for i in range(b):
            tables[c, i, :nblk[i]] = perm[pos:pos + nblk[i]]
            pos += nblk[i]
    cu = np.zeros(b + 1, dtype=np.int64)
    cu[1:] = np.cumsum(seq_lens.astype(np.int64))
    gen = _gen(seed, device)
    qd = "f32" if cache_dtype == "f32" else "bf16"
    q = _randn((b, hq, head_dim), gen, device, qd)
    k = _randn((int(cu[-1]), hkv, head_dim), gen, device, qd)
    v = _randn((int(cu[-1]), hkv, head_dim), gen, device, qd)
    out = DecodeInputs(name, seed, b, hq, hkv, head_dim, block_size, cache_dtype,
                       seq_lens, cu, tables, num_blocks, q, k, v,
                       scale=float(1.0 / np.sqrt(head_dim)))
    if cache_dtype == "fp8":
        out.k_scale, out.k_inv_scale = _fp8_scales(k, hkv)
        out.v_scale, out.v_inv_scale = _fp8_scales(v, hkv)
    return out


# ---- named workloads -------------------------------------------------------

def single_seq_f32(device="cpu"):
    """Single sequence, fp32: B=1, Hq=4, Hkv=1, Dh=64, 35 cached tokens + the
    36th appended; 3 blocks at random ids from a pool of 8."""
    seed = SEEDS["single_seq_f32"]
    rng = np.random.default_rng(seed)
    ids = rng.choice(8, 3, replace=False).astype(np.int32)
    gen = _gen(seed, device)
    q = _randn((1, 4, 64), gen, device, "f32")
    k = _randn((36, 1, 64), gen, device, "f32")
    v = _randn((36, 1, 64), gen, device, "f32")
    tables = np.full((1, 1, 3), -1, dtype=np.int32)
    tables[0, 0, :] = ids
    return DecodeInputs("single-seq-f32-t35", seed, 1, 4, 1, 64, BLOCK_SIZE, "f32",
                        np.array([36], dtype=np.int32), np.array([0, 36], dtype=np.int64),
                        tables, 8, q, k, v, scale=1.0 / 8.0)


def gqa_b32(variant="all4096", device="cpu", copies=1, batch=32, max_len=4096, block_size=BLOCK_SIZE):
    """GQA decode, bf16: B=32, Hq=32, Hkv=8, Dh=128; lengths all 4096 or
    uniform in [1, 4096]."""
    seed = SEEDS["gqa_b32"]
    rng = np.random.default_rng(seed)
    if variant == "all4096":
        lens = np.full(batch, max_len, dtype=np.int32)
    elif variant == "uniform":
        lens = rng.integers(1, max_len + 1, batch).astype(np.int32)
    else:
        raise ValueError(variant)
    name = {"all4096": f"gqa-b{batch}-t{max_len}", "uniform": f"gqa-b{batch}-ragged"}[variant]
    return decode_inputs(name, seed, lens, 32, 8, 128, "bf16", device,
                         block_size=block_size, copies=copies, rng=rng)


def long_context(batch=1, device="cpu", tokens=32768, layers=32):
    """Long context, bf16: B ∈ {1, 4}, T=32768, Hq=32, Hkv=8, Dh=128, one
    table per sequence shared by `layers` independent caches (one pool per
    layer, each drawn from its own stream)."""
    seed = SEEDS["long_context"]
    rng = np.random.default_rng(seed)
    lens = np.full(batch, tokens, dtype=np.int32)
    base = decode_inputs(f"long-b{batch}-t{tokens}", seed, lens, 32, 8, 128, "bf16", device, rng=rng)
    out = [base]
    for layer in range(1, layers):
        gen = _gen(seed * 1000 + layer, device)
        li = DecodeInputs(**{f: getattr(base, f) for f in base.__dataclass_fields__})
        li.q = _randn(tuple(base.q.shape), gen, device, "bf16")
        li.k = _randn(tuple(base.k.shape), gen, device, "bf16")
        li.v = _randn(tuple(base.v.shape), gen, device, "bf16")
        out.append(li)
    return out


def head_layouts_t8192(kind, device="cpu", batch=8, tokens=8192, copies=1, block_size=BLOCK_SIZE):
    """Head-layout / KV-dtype sweep at T=8192, B=8, Dh=128: "mha" 32/32,
    "gqa" 32/8, "mqa" 32/1 in bf16, "gqa-fp8" 32/8 with e4m3 storage."""
    seed = SEEDS["head_layouts_t8192"]
    hkv, dt = {"mha": (32, "bf16"), "gqa": (8, "bf16"), "mqa": (1, "bf16"),
               "gqa-fp8": (8, "fp8")}[kind]
    rng = np.random.default_rng(seed)
    lens = np.full(batch, tokens, dtype=np.int32)
    return decode_inputs(f"{kind}-b{batch}-t{tokens}", seed, lens, 32, hkv, 128, dt, device,
                         block_size=block_size, copies=copies, rng=rng)


@dataclass
class MixedInputs:
    """Shared-prefix mixed step: 16 sequences share `shared` tokens' blocks and
    hold `private` more each; sequence 0 runs a causal chunk of `chunk` tokens;
    `n_decode` other sequences with cached lengths `decode_ctx` decode one
    token each."""
    seed: int
    hq: int
    hkv: int
    head_dim: int
    block_size: int
    n_share: int
    shared: int
    private: int
    chunk: int
    decode_ctx: np.ndarray          # int32 [n_decode], cached tokens before the step
    free_order: np.ndarray          # int32 permutation of the pool
    num_blocks: int
    prefix_kv: List[torch.Tensor]   # k, v [shared, Hkv, Dh]
    private_kv: List[List[torch.Tensor]] = field(default_factory=list)  # per seq [k, v] [private, Hkv, Dh]
    chunk_kv: List[torch.Tensor] = field(default_factory=list)          # k, v [chunk, Hkv, Dh]
    chunk_q: Optional[torch.Tensor] = None                              # [chunk, Hq, Dh]
    decode_kv: List[List[torch.Tensor]] = field(default_factory=list)   # per seq [k, v] [ctx+1, Hkv, Dh]
    decode_q: Optional[torch.Tensor] = None                             # [n_decode, Hq, Dh]
    scale: float = 1.0
    # sharers_decode variant: sequences 1 … n_share−1 also decode one token
    # (position shared + private), drawn after everything above
    sharer_new_kv: Optional[List[torch.Tensor]] = None                  # k, v [n_share−1, Hkv, Dh]
    sharer_q: Optional[torch.Tensor] = None                             # [n_share−1, Hq, Dh]


def shared_prefix_mixed(device="cpu", n_share=16, shared=1024, private=1024, chunk=512, n_decode=64,
         ctx_lo=256, ctx_hi=2048, hq=32, hkv=8, head_dim=128, sharers_decode=False):
    """Mixed chunked prefill + decode with a shared prefix (bf16). With
    sharers_decode the n_share − 1 sequences that share S0's prefix decode one
    token each as well (their draws come last, so the rest is unchanged)."""
    seed = SEEDS["shared_prefix_mixed"]
    bs = BLOCK_SIZE
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, n_decode).astype(np.int32)
    blocks = (_ceil_div(shared, bs) + n_share * _ceil_div(private, bs)
              + _ceil_div(chunk, bs) + sum(_ceil_div(int(t) + 1, bs) for t in ctx) + 64)
    free_order = rng.permutation(blocks).astype(np.int32)
    gen = _gen(seed, device)
    r = lambda n, h: _randn((n, h, head_dim), gen, device, "bf16")  # noqa: E731
    m = MixedInputs(seed, hq, hkv, head_dim, bs, n_share, shared, private, chunk, ctx,
                    free_order, blocks, [r(shared, hkv), r(shared, hkv)])
    m.private_kv = [[r(private, hkv), r(private, hkv)] for _ in range(n_share)]
    m.chunk_kv = [r(chunk, hkv), r(chunk, hkv)]
    m.chunk_q = r(chunk, hq)
    m.decode_kv = [[r(int(t) + 1, hkv), r(int(t) + 1, hkv)] for t in ctx]
    m.decode_q = _randn((n_decode, hq, head_dim), gen, device, "bf16")
    m.scale = float(1.0 / np.sqrt(head_dim))
    if sharers_decode:
        m.sharer_new_kv = [r(n_share - 1, hkv), r(n_share - 1, hkv)]
        m.sharer_q = _randn((n_share - 1, hq, head_dim), gen, device, "bf16")
    return m
