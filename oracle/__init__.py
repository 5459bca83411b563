"""CPU oracle for paged KV-cache attention — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct statement of what the GPU
library computes. It exists so that tests, the smoke check and the bench's CPU
baseline have something independent to compare against. It shares no code,
constants or helpers with the HIP library and never imports it; the product
path never imports this package.

Everything here is float64 numpy (or plain Python integers), written to be read
against the pages, not to be fast.

Pages cited (by title, section and table; the addresses are where they live):

* "04. 注意力与 KV 缓存" (Attention and the KV cache),
  niuwancheng.cn/blog/docs/ai/inference-series/04-cache-attention.html
* "07｜KV Cache、FlashAttention与PagedAttention的内部过程" (inner workings of
  the KV cache, FlashAttention and PagedAttention),
  ai-engineering-handbook.eonloom.com/chapters/07.html — questions Q025–Q028
* "06 KV Cache、Prefix Cache、PagedAttention 与 vLLM", sections 6.1–6.7,
  sta324-midterm-2026-5n0wme17.flowershow.me/06-kv-cache
* "03. KV Cache：用显存换计算" (trading memory for compute),
  niuwancheng.cn/blog/docs/ai/llm-inference/03-kv-cache.html

Modules:
  attention  — the materialised causal softmax(QKᵀ·scale + mask)·V definition
  online     — the online-softmax state (m, l, u), block update and merge
  paging     — block counts, position → (block, offset) → slot, pool scatter/gather
  fp8        — OCP e4m3fn decode and round-to-nearest-even saturating encode
  allocator  — a pure-Python model of the ref-counted block allocator
  sizing     — KV-cache byte arithmetic; K/V positions built per generation step
  prefix     — full-block prefix reuse with a chained block hash

Every function is pinned by a CPU test against values the pages print, closed
forms, library routines or brute force; none is "parity unpinned".
"""

from . import attention, online, paging, fp8, allocator, sizing, prefix  # noqa: F401
