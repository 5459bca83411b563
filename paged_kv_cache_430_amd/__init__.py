"""Python binding for libpkv.so, the gfx950 paged KV-cache attention library.

Argument marshalling only: every function here forwards torch tensors'
device pointers and the current HIP stream to the C entry point of the same
name (declared in include/pkv.h) and raises PKVError on a non-zero status.
All computation happens in the library's HIP kernels; there is no fallback —
if libpkv.so is missing or fails to load, importing the binding's functions
raises.
"""

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "PKVError", "Cache", "BlockAllocator", "PrefixIndex", "load",
    "pkv_version", "pkv_slot_mapping", "pkv_slot_mapping_device", "pkv_kv_append", "pkv_kv_append_paged",
    "pkv_attn_decode_workspace_bytes", "pkv_attn_decode_auto_partition", "pkv_attn_decode",
    "pkv_attn_decode_append", "pkv_attn_decode_noalloc",
    "pkv_attn_prefill_chunk", "pkv_attn_mixed_step", "pkv_copy_blocks", "pkv_swap_out", "pkv_swap_in", "pkv_debug_gather",
    "pkv_debug_stream_read", "pkv_debug_mfma_rate", "pkv_debug_prefill_mix",
    "PKV_F32", "PKV_BF16", "PKV_FP8_E4M3",
]

# PKV_LIB names another build of the same library (the AddressSanitizer one
# from `python -m paged_kv_cache_430_amd._build --asan`)
LIB_PATH = os.environ.get("PKV_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_ENOBLOCKS, PKV_EDTYPE, PKV_EREF, PKV_EWORKSPACE, PKV_EHIP = 0, -1, -2, -3, -4, -5, -6
PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
STATUS_NAMES = {0: "PKV_OK", -1: "PKV_EINVAL", -2: "PKV_ENOBLOCKS", -3: "PKV_EDTYPE",
                -4: "PKV_EREF", -5: "PKV_EWORKSPACE", -6: "PKV_EHIP"}


class PKVError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class _CacheStruct(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


_I32P = ctypes.POINTER(ctypes.c_int32)
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
class _ChunkBatch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("q", ctypes.c_void_p), ("q_start", ctypes.c_void_p),
                ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("block_tables", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("seq_lens", ctypes.c_void_p), ("max_q_len", ctypes.c_int32),
                ("out", ctypes.c_void_p)]


class _DecodeBatch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q", ctypes.c_void_p), ("k_new", ctypes.c_void_p),
                ("v_new", ctypes.c_void_p), ("block_tables", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("max_seq_len", ctypes.c_int32),
                ("partition_tokens", ctypes.c_int32), ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


_SIGS = {
    "pkv_version": (_I32, []),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_slot_mapping": (ctypes.c_int, [_VP, _I32, _I32, _I32, _I32, _VP]),
    "pkv_slot_mapping_device": (ctypes.c_int, [_VP, _I32, _I32, _I32, _VP, _VP, _I32, _VP, _VP]),
    "pkv_kv_append": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, _VP, _I32, _I32, _VP, _VP, _VP, _VP]),
    "pkv_kv_append_paged": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, _VP, _I32, _I32, _VP, _VP, _I32, _VP,
                                           _I32, _VP, _VP, _VP, _VP]),
    "pkv_attn_decode_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_attn_decode_auto_partition": (_I32, [_I32, _I32, _I32, _I32, _I32]),
    "pkv_attn_decode": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, _I32, _I32, _I32, _VP, _I32, _VP,
                                       _I32, ctypes.c_float, _I32, _VP, _VP, ctypes.c_size_t, _VP]),
    "pkv_attn_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, _I32, _I32, _I32, _VP, _I32,
                                               _VP, _I32, ctypes.c_float, _I32, _VP, _VP]),
    "pkv_attn_decode_append": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, _VP, _I32, _VP, _VP, _VP, _I32,
                                              _I32, _I32, _VP, _I32, _VP, _I32, ctypes.c_float, _I32, _VP, _VP,
                                              ctypes.c_size_t, _VP]),
    "pkv_attn_prefill_chunk": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, _I32, _I32, _I32, _VP, _VP,
                                              _I32, _VP, _I32, ctypes.c_float, _VP, _VP]),
    "pkv_attn_mixed_step": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _I32, ctypes.c_float,
                                           ctypes.POINTER(_ChunkBatch), ctypes.POINTER(_DecodeBatch), _VP]),
    "pkv_copy_blocks": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, _VP, _I32, _VP]),
    "pkv_debug_gather": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, _I32, _VP, _VP, _VP]),
    "pkv_debug_stream_read": (ctypes.c_int, [_VP, ctypes.c_int64, _VP, _I32, _I32, _VP, _VP]),
    "pkv_debug_mfma_rate": (ctypes.c_int, [_VP, _I32, _I32, _VP, _VP]),
    "pkv_debug_prefill_mix": (ctypes.c_int, [_VP, _VP, ctypes.c_int64, _I32, _I32, _I32, _VP, _VP]),
    "pkv_swap_out": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, _I32, _VP, ctypes.c_size_t, _VP]),
    "pkv_swap_in": (ctypes.c_int, [ctypes.POINTER(_CacheStruct), _VP, ctypes.c_size_t, _VP, _I32, _VP]),
    "pkv_alloc_create": (ctypes.c_int, [_I32, _I32, _VP, ctypes.POINTER(_VP)]),
    "pkv_alloc_destroy": (None, [_VP]),
    "pkv_alloc_allocate": (ctypes.c_int, [_VP, _I32, _VP]),
    "pkv_alloc_incref": (ctypes.c_int, [_VP, _VP, _I32]),
    "pkv_alloc_decref": (ctypes.c_int, [_VP, _VP, _I32]),
    "pkv_alloc_refcount": (ctypes.c_int, [_VP, _I32]),
    "pkv_alloc_num_free": (_I32, [_VP]),
    "pkv_alloc_reserve_append": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _VP, _VP, _VP]),
    "pkv_prefix_create": (ctypes.c_int, [_I32, ctypes.POINTER(_VP)]),
    "pkv_prefix_destroy": (None, [_VP]),
    "pkv_prefix_insert": (ctypes.c_int, [_VP, _VP, _VP, _I32, ctypes.c_uint64, _VP, _I32, _VP]),
    "pkv_prefix_match": (ctypes.c_int, [_VP, _VP, _VP, _I32, ctypes.c_uint64, _VP, _I32, _VP]),
    "pkv_prefix_stats": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP]),
    "pkv_prefix_clear": (ctypes.c_int, [_VP, _VP]),
}

_lib = None


def load():
    """Load libpkv.so (built in-tree by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python __graft_entry__.py` "
                               "(or paged_kv_cache_430_amd/_build.py) first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status):
    if status != PKV_OK:
        raise PKVError(status, load().pkv_last_error().decode())
    return status


def _dtype_code(t):
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PKV_FP8_E4M3
    raise PKVError(PKV_EDTYPE, f"unsupported tensor dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if not t.is_contiguous():
            raise PKVError(PKV_EINVAL, "tensors passed to the library must be contiguous")
        return t.data_ptr()
    return t


def _stream(stream, device):
    if stream is not None:
        return stream
    return torch.cuda.current_stream(device).cuda_stream


def _i32_host(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Cache:
    """One layer's paged cache: K and V pools [num_blocks, Hkv, block_size, Dh]
    (block_size 8, 16, 32 or 64) in f32, bf16 or e4m3 bytes (uint8), plus
    per-KV-head fp32 scales for e4m3."""

    def __init__(self, k_cache, v_cache, k_scale=None, v_scale=None):
        if k_cache.shape != v_cache.shape or k_cache.dim() != 4:
            raise PKVError(PKV_EINVAL, "k_cache and v_cache must both be [num_blocks, Hkv, block_size, Dh]")
        self.k, self.v, self.k_scale, self.v_scale = k_cache, v_cache, k_scale, v_scale
        nb, hkv, bs, dh = k_cache.shape
        self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim = nb, hkv, bs, dh
        self.dtype = _dtype_code(k_cache)
        self._s = _CacheStruct(nb, bs, hkv, dh, self.dtype, _ptr(k_cache), _ptr(v_cache),
                               _ptr(k_scale), _ptr(v_scale))

    @property
    def device(self):
        return self.k.device

    def ref(self):
        return ctypes.byref(self._s)


def pkv_version():
    return load().pkv_version()


def pkv_slot_mapping(block_table, block_size, first_pos, n):
    """Host slots for n positions from first_pos (numpy int32)."""
    bt = _i32_host(block_table)
    out = np.empty(n, dtype=np.int32)
    _check(load().pkv_slot_mapping(bt.ctypes.data, len(bt), block_size, first_pos, n, out.ctypes.data))
    return out


def pkv_slot_mapping_device(block_tables, cu_new, first_pos, n_tokens, block_size=16, out=None, stream=None):
    dev = block_tables.device
    if out is None:
        out = torch.empty(n_tokens, dtype=torch.int32, device=dev)
    _check(load().pkv_slot_mapping_device(_ptr(block_tables), block_tables.shape[1], block_size,
                                          len(first_pos), _ptr(cu_new), _ptr(first_pos), n_tokens,
                                          _ptr(out), _stream(stream, dev)))
    return out


def pkv_kv_append(cache, k_new, v_new, slot_mapping, k_inv_scale=None, v_inv_scale=None, stream=None):
    _check(load().pkv_kv_append(cache.ref(), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), k_new.shape[0],
                                _ptr(slot_mapping), _ptr(k_inv_scale), _ptr(v_inv_scale),
                                _stream(stream, cache.device)))


def pkv_kv_append_paged(cache, k_new, v_new, block_tables, cu_new, first_pos, max_new, k_inv_scale=None,
                        v_inv_scale=None, out_slots=None, stream=None):
    """Slot mapping and append in one launch; returns out_slots (may be None)."""
    _check(load().pkv_kv_append_paged(cache.ref(), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), len(first_pos),
                                      _ptr(cu_new), _ptr(first_pos), int(max_new), _ptr(block_tables),
                                      block_tables.shape[1], _ptr(k_inv_scale), _ptr(v_inv_scale), _ptr(out_slots),
                                      _stream(stream, cache.device)))
    return out_slots


def pkv_attn_decode_workspace_bytes(cache_dtype, batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                    partition_tokens=0):
    return load().pkv_attn_decode_workspace_bytes(cache_dtype, batch, num_q_heads, num_kv_heads, head_dim,
                                                  max_seq_len, partition_tokens)


def pkv_attn_decode_auto_partition(cache_dtype, batch, num_q_heads, num_kv_heads, max_seq_len):
    return load().pkv_attn_decode_auto_partition(cache_dtype, batch, num_q_heads, num_kv_heads, max_seq_len)


def decode_workspace(cache_dtype, batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_tokens,
                     device):
    """A workspace of the size pkv_attn_decode needs (or None); its contents
    need no initialisation."""
    n = pkv_attn_decode_workspace_bytes(cache_dtype, batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                        partition_tokens)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def pkv_attn_decode(cache, q, block_tables, seq_lens, max_seq_len, scale, partition_tokens=0,
                    out=None, workspace=None, stream=None):
    b, hq, dh = q.shape
    dev = q.device
    if out is None:
        out = torch.empty(b, hq, dh, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = decode_workspace(cache.dtype, b, hq, cache.num_kv_heads, dh, max_seq_len, partition_tokens, dev)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pkv_attn_decode(cache.ref(), _ptr(q), _dtype_code(q), b, hq, _ptr(block_tables),
                                  block_tables.shape[1], _ptr(seq_lens), max_seq_len, float(scale),
                                  partition_tokens, _ptr(out), _ptr(workspace), wbytes, _stream(stream, dev)))
    return out


def pkv_attn_decode_noalloc(cache, q, block_tables, seq_lens, max_seq_len, scale, out, partition_tokens=0,
                            stream=None):
    """pkv_attn_decode with the library's static split-KV scratch: no workspace,
    and nothing allocated (out is the caller's [B, Hq, Dh] fp32 tensor)."""
    b, hq, dh = q.shape
    _check(load().pkv_attn_decode_noalloc(cache.ref(), _ptr(q), _dtype_code(q), b, hq, _ptr(block_tables),
                                          block_tables.shape[1], _ptr(seq_lens), max_seq_len, float(scale),
                                          partition_tokens, _ptr(out), _stream(stream, q.device)))
    return out


def pkv_attn_decode_append(cache, k_new, v_new, q, block_tables, seq_lens, max_seq_len, scale, partition_tokens=0,
                           k_inv_scale=None, v_inv_scale=None, out=None, workspace=None, stream=None):
    """Append each sequence's new token (k_new, v_new: [B, Hkv, Dh]) at position
    seq_lens[b] - 1 and decode, in one launch for bf16/fp8 caches."""
    b, hq, dh = q.shape
    dev = q.device
    if out is None:
        out = torch.empty(b, hq, dh, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = decode_workspace(cache.dtype, b, hq, cache.num_kv_heads, dh, max_seq_len, partition_tokens, dev)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pkv_attn_decode_append(cache.ref(), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(k_inv_scale),
                                         _ptr(v_inv_scale), _ptr(q), _dtype_code(q), b, hq, _ptr(block_tables),
                                         block_tables.shape[1], _ptr(seq_lens), max_seq_len, float(scale),
                                         partition_tokens, _ptr(out), _ptr(workspace), wbytes, _stream(stream, dev)))
    return out


def pkv_attn_mixed_step(cache, scale, chunk_q, chunk_k_new, chunk_v_new, q_start, chunk_tables, chunk_lens, max_q_len,
                        dec_q, dec_k_new, dec_v_new, dec_tables, dec_lens, max_seq_len, partition_tokens=0,
                        chunk_out=None, dec_out=None, workspace=None, stream=None):
    """One mixed continuous-batching step (bf16 cache): the chunks' tokens are
    appended and their chunks attend causally; each decode sequence appends its
    token and attends. Returns (chunk_out, dec_out)."""
    dev = dec_q.device
    b, hq, dh = dec_q.shape
    n_chunks = len(chunk_lens)
    if chunk_out is None:
        chunk_out = torch.empty(chunk_q.shape[0], hq, dh, dtype=torch.float32, device=dev)
    if dec_out is None:
        dec_out = torch.empty(b, hq, dh, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = decode_workspace(cache.dtype, b, hq, cache.num_kv_heads, dh, max_seq_len, partition_tokens, dev)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ch = _ChunkBatch(n_chunks, _ptr(chunk_q), _ptr(q_start), _ptr(chunk_k_new), _ptr(chunk_v_new), _ptr(chunk_tables),
                     chunk_tables.shape[1], _ptr(chunk_lens), max_q_len, _ptr(chunk_out))
    de = _DecodeBatch(b, _ptr(dec_q), _ptr(dec_k_new), _ptr(dec_v_new), _ptr(dec_tables), dec_tables.shape[1],
                      _ptr(dec_lens), max_seq_len, partition_tokens, _ptr(dec_out), _ptr(workspace), wbytes)
    _check(load().pkv_attn_mixed_step(cache.ref(), hq, float(scale), ctypes.byref(ch), ctypes.byref(de),
                                      _stream(stream, dev)))
    return chunk_out, dec_out


def pkv_attn_prefill_chunk(cache, q, q_start, block_tables, seq_lens, max_q_len, scale, out=None, stream=None):
    n, hq, dh = q.shape
    dev = q.device
    if out is None:
        out = torch.empty(n, hq, dh, dtype=torch.float32, device=dev)
    _check(load().pkv_attn_prefill_chunk(cache.ref(), _ptr(q), _dtype_code(q), len(seq_lens), hq, _ptr(q_start),
                                         _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), max_q_len,
                                         float(scale), _ptr(out), _stream(stream, dev)))
    return out


def pkv_copy_blocks(cache, src, dst, stream=None):
    _check(load().pkv_copy_blocks(cache.ref(), _ptr(src), _ptr(dst), src.numel(), _stream(stream, cache.device)))


def pkv_swap_out(cache, ids, host, stream=None):
    """Blocks ids (device int32) → host (a pinned uint8 tensor of n·2·block bytes)."""
    _check(load().pkv_swap_out(cache.ref(), _ptr(ids), ids.numel(), _ptr(host), host.numel() * host.element_size(),
                               _stream(stream, cache.device)))
    return host


def pkv_swap_in(cache, host, ids, stream=None):
    """host (pinned, as written by pkv_swap_out) → blocks ids (device int32)."""
    _check(load().pkv_swap_in(cache.ref(), _ptr(host), host.numel() * host.element_size(), _ptr(ids), ids.numel(),
                              _stream(stream, cache.device)))


def pkv_debug_stream_read(buf, tile_ids, num_workgroups, sink=None, stream=None):
    """Read the 4 KiB tiles of `buf` (a 16-byte aligned device tensor) listed in
    `tile_ids` (device int32) in that order; returns the per-workgroup XOR of
    what was read (device uint32 [num_workgroups])."""
    dev = buf.device
    if sink is None:
        sink = torch.empty(num_workgroups, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * buf.element_size()
    _check(load().pkv_debug_stream_read(_ptr(buf), nbytes // 4096, _ptr(tile_ids), tile_ids.numel(), num_workgroups,
                                        _ptr(sink), _stream(stream, dev)))
    return sink


def pkv_debug_mfma_rate(operands, iterations, num_workgroups, sink=None, stream=None):
    """Run the prefill's steady-iteration products `iterations` times in
    `num_workgroups` 8-wave workgroups on `operands` (device bf16, at least
    664 values); returns the per-lane accumulator sums (device float32
    [num_workgroups * 512])."""
    dev = operands.device
    if operands.dtype != torch.bfloat16 or operands.numel() < 664:
        raise PKVError(PKV_EINVAL, "operands: bf16, at least 664 values")
    if sink is None:
        sink = torch.empty(num_workgroups * 512, dtype=torch.float32, device=dev)
    _check(load().pkv_debug_mfma_rate(_ptr(operands), iterations, num_workgroups, _ptr(sink), _stream(stream, dev)))
    return sink


def pkv_debug_prefill_mix(operands, tiles, mode, iterations, num_workgroups, sink=None, stream=None):
    """Run the prefill's steady-iteration mix (products and vector work; mode
    1 adds its LDS operand reads, mode 2 also its LDS-direct tile loads and a
    barrier) `iterations` times in `num_workgroups` 8-wave workgroups;
    `operands` device bf16 (at least 664 values), `tiles` a device tensor of
    at least 1 MiB. Returns the per-lane sums (device float32
    [num_workgroups * 512])."""
    dev = operands.device
    if operands.dtype != torch.bfloat16 or operands.numel() < 664:
        raise PKVError(PKV_EINVAL, "operands: bf16, at least 664 values")
    if sink is None:
        sink = torch.empty(num_workgroups * 512, dtype=torch.float32, device=dev)
    nbytes = tiles.numel() * tiles.element_size()
    _check(load().pkv_debug_prefill_mix(_ptr(operands), _ptr(tiles), nbytes, mode, iterations, num_workgroups,
                                        _ptr(sink), _stream(stream, dev)))
    return sink


def pkv_debug_gather(cache, block_table, seq_len, stream=None):
    shape = (cache.num_kv_heads, seq_len, cache.head_dim)
    k_out = torch.empty(shape, dtype=cache.k.dtype, device=cache.device)
    v_out = torch.empty(shape, dtype=cache.k.dtype, device=cache.device)
    _check(load().pkv_debug_gather(cache.ref(), _ptr(block_table), seq_len, _ptr(k_out), _ptr(v_out),
                                   _stream(stream, cache.device)))
    return k_out, v_out


class BlockAllocator:
    """Host ref-counted block allocator (pkv_alloc_*)."""

    def __init__(self, num_blocks, block_size=16, free_order=None):
        lib = load()
        self._h = ctypes.c_void_p()
        fo = None if free_order is None else _i32_host(free_order)
        self._keep = fo
        _check(lib.pkv_alloc_create(num_blocks, block_size, None if fo is None else fo.ctypes.data,
                                    ctypes.byref(self._h)))
        self.num_blocks, self.block_size = num_blocks, block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.pkv_alloc_destroy(h)
            self._h = None

    def allocate(self, n):
        out = np.empty(n, dtype=np.int32)
        _check(load().pkv_alloc_allocate(self._h, n, out.ctypes.data))
        return out

    def incref(self, ids):
        ids = _i32_host(ids)
        _check(load().pkv_alloc_incref(self._h, ids.ctypes.data, len(ids)))

    def decref(self, ids):
        ids = _i32_host(ids)
        _check(load().pkv_alloc_decref(self._h, ids.ctypes.data, len(ids)))

    def refcount(self, bid):
        return _check_nonneg(load().pkv_alloc_refcount(self._h, bid))

    def num_free(self):
        return load().pkv_alloc_num_free(self._h)

    def reserve_append(self, table, seq_len, n_new):
        """Grow a host int32 table in place; returns the (src, dst) copies needed."""
        if not (isinstance(table, np.ndarray) and table.dtype == np.int32 and table.flags.c_contiguous):
            raise PKVError(PKV_EINVAL, "table must be a contiguous numpy int32 array")
        src = np.zeros(1, dtype=np.int32)
        dst = np.zeros(1, dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(load().pkv_alloc_reserve_append(self._h, table.ctypes.data, len(table), seq_len, n_new,
                                               src.ctypes.data, dst.ctypes.data, ctypes.addressof(n)))
        return [(int(src[0]), int(dst[0]))] if n.value else []


class PrefixIndex:
    """Host prefix-cache index over full blocks (pkv_prefix_*). `alloc` (a
    BlockAllocator or None) is passed to every call that can take or give
    references."""

    def __init__(self, block_size=16, alloc=None):
        lib = load()
        self._h = ctypes.c_void_p()
        _check(lib.pkv_prefix_create(block_size, ctypes.byref(self._h)))
        self.block_size, self.alloc = block_size, alloc

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.pkv_prefix_destroy(h)
            self._h = None

    def _a(self):
        return None if self.alloc is None else self.alloc._h

    def insert(self, tokens, block_ids, identity=0):
        tok, ids = _i32_host(tokens), _i32_host(block_ids)
        n = ctypes.c_int32(0)
        _check(load().pkv_prefix_insert(self._h, self._a(), tok.ctypes.data, len(tok), identity, ids.ctypes.data,
                                        len(ids), ctypes.addressof(n)))
        return n.value

    def match(self, tokens, identity=0, max_ids=None):
        tok = _i32_host(tokens)
        cap = len(tok) // self.block_size if max_ids is None else max_ids
        out = np.empty(max(cap, 1), dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(load().pkv_prefix_match(self._h, self._a(), tok.ctypes.data, len(tok), identity, out.ctypes.data,
                                       cap, ctypes.addressof(n)))
        return out[:n.value].copy()

    def stats(self):
        v = [ctypes.c_int64(0) for _ in range(4)]
        e = ctypes.c_int32(0)
        _check(load().pkv_prefix_stats(self._h, *[ctypes.addressof(x) for x in v], ctypes.addressof(e)))
        return {"hit_tokens": v[0].value, "compared_tokens": v[1].value, "requests": v[2].value,
                "hit_requests": v[3].value, "entries": e.value}

    def clear(self):
        _check(load().pkv_prefix_clear(self._h, self._a()))


def _check_nonneg(v):
    if v < 0:
        raise PKVError(v, load().pkv_last_error().decode())
    return v
