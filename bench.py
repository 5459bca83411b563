#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X.

Default workload (the headline metric, `gqa-b32-t4096`): GQA paged decode,
B=32 sequences, Hq=32, Hkv=8, Dh=128, every sequence 4096 tokens, bf16
cache, block size 16. One step is the whole decode hot path for the batch —
slot mapping and KV append of the 32 new tokens (position 4095) through the
block tables, and split-KV paged decode attention over all 4096 tokens — in
one launch (pkv_attn_decode_append); `--unfused` runs the append as its own
launch (pkv_kv_append_paged) before pkv_attn_decode.
Inputs are resident in HBM before timing. Copies of the pool behind separate
block-table sets (at least 2 GiB in total) are used in rotation so that the
256 MB Infinity Cache cannot serve a step from the previous one.

Prints one JSON line. `value` is algorithmic HBM bytes per step (KV read +
q + out + tables + lengths + append traffic) divided by the step time;
`roofline` reports the decode call alone, timed with HIP events on the
stream it runs on in a second pass over the same steps (so the K timed steps
carry no per-call events); `cpu_baseline` times the float64 CPU oracle on a
sample of the same batch on this host.

--workload selects other decode workloads (same kind of line);
`shared-prefix-mixed`: one mixed step of the shared-prefix workload — a causal
512-token prefill chunk on a 2048-token cache plus 64 single-token decodes,
run as pkv_attn_mixed_step (ms_per_step; PKV_MIXED picks its form) — whose
line also reports the chunk and the decodes, each timed as its own call,
against the bf16 MFMA peak and HBM; `prefill-chunk`: one chunk alone
(--chunk queries on --prefix tokens); `swap`: blocks to pinned host memory
and back; `prefix-index`: the host prefix-cache index; `read-ceiling`: the GPU's
streaming-read rate for the decode's 4 KiB tiles, in order and scattered;
`mfma-ceiling`: the bf16 matrix-core rate sustained with every CU running the
prefill's steady-iteration products (the chip's clock drops under that load),
and beside it the rate of the same products with the iteration's vector work,
LDS operand reads and tile loads added in turn.
`append`: slot mapping and KV append in one launch, at the mixed step's size and in bulk.
`allocator`: the host block allocator on the shared-prefix workload's bookkeeping.

Counter summaries: `--calib-copy` adds, after the timed steps, one
pkv_copy_blocks launch over a 256 MiB scratch cache (a plain copy of known
size). Run the bench under `rocprofv3 --pmc FETCH_SIZE` and again under
`--pmc WRITE_SIZE` with that flag, then `python bench.py --counters
FETCH_CSV WRITE_CSV --workload W [--chunk C]` (no GPU needed) scales each
counter by what it read for the copy and writes
profiles/<kernel>_<workload>_traffic.json (picked up by later runs as
roofline.traffic while the decode, or prefill, sources are unchanged) plus a
text summary.

Trace summaries: `python bench.py --trace-summary KERNEL_STATS_CSV --workload W
[--chunk C]` (no GPU needed) records the mean duration of the workload's main
kernel from a `rocprofv3 --kernel-trace --stats` run of this bench as
profiles/<kernel>_<workload>_trace.json; while the kernel's sources are
unchanged, later runs report it as roofline.trace (achieved and frac from the
kernel's own duration) beside the event-timed roofline, which includes the
launch. The prefill line also reports roofline.pipelined: K back-to-back
calls between two events.
"""

import argparse
import csv
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV HBM GB/s (% of peak), B=32 Hkv=8 Dh=128 T=4096 bf16"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PCIE5_X16_GBS = 32.0 * 16 * 128 / 130 / 8   # 63.0 GB/s per direction
MALL_BYTES = 2 * 2 ** 30          # rotate through at least this much pool memory
CALIB_BYTES = 256 * 2 ** 20       # K+V bytes moved by the calibration copy
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SOURCES = ["paged_kv_cache_430_amd/csrc/decode.hip", "paged_kv_cache_430_amd/csrc/device_common.h",
                  "paged_kv_cache_430_amd/csrc/append_common.h"]
APPEND_SOURCES = ["paged_kv_cache_430_amd/csrc/kv_append.hip", "paged_kv_cache_430_amd/csrc/append_common.h"]
PREFILL_SOURCES = ["paged_kv_cache_430_amd/csrc/prefill.hip", "paged_kv_cache_430_amd/csrc/prefill_stream.h",
                   "paged_kv_cache_430_amd/csrc/device_common.h"]
# decode workloads: name → (generator, its arguments)
DECODE_WORKLOADS = {
    "gqa-b32-t4096": ("gqa_b32", "all4096"),        # the headline: B=32 Hq=32 Hkv=8 Dh=128 T=4096 bf16
    "gqa-b32-ragged": ("gqa_b32", "uniform"),       # the same with lengths uniform in [1, 4096]
    "mha-b8-t8192": ("head_layouts_t8192", "mha"),
    "gqa-b8-t8192": ("head_layouts_t8192", "gqa"),
    "mqa-b8-t8192": ("head_layouts_t8192", "mqa"),
    "gqa-fp8-b8-t8192": ("head_layouts_t8192", "gqa-fp8"),
    "long-b1-t32768": ("long_context", 1),          # 32 layers' caches, one table
    "long-b4-t32768": ("long_context", 4),
}
MIXED_WORKLOAD = "shared-prefix-mixed"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="gqa-b32-t4096",
                   choices=list(DECODE_WORKLOADS) + [MIXED_WORKLOAD, "prefill-chunk", "prefix-index", "swap",
                            "read-ceiling", "mfma-ceiling", "append", "allocator"])
    p.add_argument("--prefix", type=int, default=2048, help="prefill-chunk: cached tokens before the chunk")
    p.add_argument("--chunk", type=int, default=128, help="prefill-chunk: queries in the chunk")
    p.add_argument("--mixed-decodes", type=int, default=64,
                   help="shared-prefix-mixed: decode sequences beside the chunk (64 is the workload)")
    p.add_argument("--mixed-chunk", type=int, default=512,
                   help="shared-prefix-mixed: tokens of S0's chunk (512 is the workload; smaller chunks take "
                        "the prefill's column form)")
    p.add_argument("--partition", type=int, default=0, help="partition_tokens (0 = library default)")
    p.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32, 64],
                   help="tokens per pool block for the B=32 and T=8192 decode workloads and prefill-chunk")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--sharers-decode", action="store_true",
                   help="shared-prefix-mixed: the 15 idle sharers (2048 tokens each) decode one token too")
    p.add_argument("--unfused", action="store_true",
                   help="decode workloads: append in its own launch before the decode (default: one launch); "
                        "shared-prefix-mixed: append, prefill and decode as three calls (default: pkv_attn_mixed_step)")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time for the oracle baseline")
    p.add_argument("--calib-copy", action="store_true",
                   help="after timing, copy a 256 MiB scratch cache with pkv_copy_blocks (counter calibration)")
    p.add_argument("--counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="summarise rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this bench; no GPU needed")
    p.add_argument("--trace-summary", metavar="KERNEL_STATS_CSV",
                   help="record the kernel durations of a rocprofv3 --kernel-trace --stats run of this bench "
                        "(--workload, --chunk as in that run) under profiles/; no GPU needed")
    return p.parse_args()


def source_hash(paths):
    """Hash of the decode sources' code: comments and blank space are left
    out, so that only a change to what compiles marks the counters stale."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)      # block comments
        text = re.sub(r"//[^\n]*", " ", text)                    # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def decode_bytes(seq_lens, hq, hkv, dh, kv_elt, q_elt, fp8, block_size=16):
    """Algorithmic bytes of one decode call: every visible K and V element
    once, q, the fp32 output, the block-table entries and lengths read."""
    kv = sum(int(t) for t in seq_lens) * hkv * dh * 2 * kv_elt
    b = len(seq_lens)
    extra = (b * hq * dh * q_elt + b * hq * dh * 4 + sum(-(-int(t) // block_size) for t in seq_lens) * 4
             + 4 * b)
    if fp8:
        extra += 2 * hkv * 4
    return kv + extra


def tail_waste(seq_lens, block_size):
    """Slots allocated but empty: Σ ⌈T/bs⌉·bs − T, and its share of the slots."""
    slots = sum(-(-int(t) // block_size) * block_size for t in seq_lens)
    waste = slots - sum(int(t) for t in seq_lens)
    return {"slots": waste, "frac": round(waste / slots, 5) if slots else 0.0}


def append_bytes(n_tokens, hkv, dh, in_elt, cache_elt):
    return n_tokens * hkv * dh * 2 * (in_elt + cache_elt) + n_tokens * 4


def prefill_flops(prefix, chunk, hq, dh):
    """4·Dh·Hq·Σ_i (P + i + 1): QKᵀ and PV over every visible (query, key) pair."""
    pairs = chunk * prefix + chunk * (chunk + 1) // 2
    return 4 * dh * hq * pairs


class Timer:
    """HIP events recorded on the stream the library launches on."""

    def __init__(self, stream, n):
        import torch
        self.stream = stream
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        self.k = 0

    def start(self):
        self.ev[self.k][0].record(self.stream)

    def stop(self):
        self.ev[self.k][1].record(self.stream)
        self.k += 1

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.ev[:self.k]]


def stats_us(ms):
    s = sorted(ms)
    n = len(s)
    return {"mean": round(sum(s) / n * 1e3, 2), "p10": round(s[n // 10] * 1e3, 2),
            "p50": round(s[n // 2] * 1e3, 2), "p90": round(s[(9 * n) // 10] * 1e3, 2)}


def calib_copy(dev):
    """pkv_copy_blocks over a scratch cache: reads and writes CALIB_BYTES."""
    import torch

    import paged_kv_cache_430_amd as pkv
    nb = CALIB_BYTES // (2 * 8 * 16 * 128 * 2)           # K and V blocks of [8, 16, 128] bf16
    k = torch.zeros(2 * nb, 8, 16, 128, dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    cache = pkv.Cache(k, v)
    src = torch.arange(nb, dtype=torch.int32, device=dev)
    dst = src + nb
    torch.cuda.synchronize()
    pkv.pkv_copy_blocks(cache, src, dst)
    torch.cuda.synchronize()


def decode_kernel_base(cache_dtype):
    """The split kernel the library runs for a cache dtype: the matrix-core
    form for bf16 and fp8 caches (unless PKV_DECODE_KERNEL=vector), the vector
    form for fp32 caches."""
    if cache_dtype == "f32" or os.environ.get("PKV_DECODE_KERNEL") == "vector":
        return "decode_split"
    return "decode_mfma"


def load_traffic(kernel, workload, sources=DECODE_SOURCES):
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("source_hash") != source_hash(sources):
        return None
    return tr.get("bytes_per_launch")


def trace_key(workload, chunk):
    return f"{workload}-c{chunk}" if workload == "prefill-chunk" else workload


def load_trace(kernel, key, sources, flops_or_bytes, peak, unit, name_has=None):
    """The kernel's mean duration from a committed rocprofv3 kernel-trace
    summary of this workload (profiles/<kernel>_<key>_trace.json), if it was
    taken on the current sources (and of a kernel whose name holds
    `name_has`), as a roofline entry; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{key}_trace.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("source_hash") != source_hash(sources):
        return None
    if name_has and name_has not in tr.get("kernel", ""):
        return None
    ns = tr["mean_ns"]
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    achieved = flops_or_bytes / (ns * 1e-9) / scale
    return {"timing": "rocprofv3 kernel trace, mean over the run's dispatches", "mean_us": round(ns / 1e3, 3),
            "achieved": round(achieved, 2), "frac": round(achieved / peak, 4),
            "summary": os.path.relpath(path, ROOT)}


def summarize_trace(stats_csv, workload, chunk):
    """Mean duration of the workload's main kernel in a rocprofv3
    --kernel-trace --stats kernel_stats.csv, recorded with the hash of the
    sources that build it."""
    if workload == "prefill-chunk":
        key, kernel, sources = "prefill_stream_kernel", "prefill_stream", PREFILL_SOURCES
    else:
        key, kernel, sources = "decode_mfma_kernel", "decode_mfma", DECODE_SOURCES
    with open(stats_csv) as f:
        rows = [r for r in csv.DictReader(f) if key in r["Name"]]
    if not rows:
        raise SystemExit(f"no {key} in {stats_csv}")
    r = rows[0]
    out = {"workload": trace_key(workload, chunk), "kernel": r["Name"], "calls": int(r["Calls"]),
           "mean_ns": float(r["AverageNs"]), "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
           "source_hash": source_hash(sources)}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"{kernel}_{trace_key(workload, chunk)}_trace.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return out


# ---------------------------------------------------------------------------
# decode workloads
# ---------------------------------------------------------------------------

def make_decode_setup(name, dev, block_size=16):
    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv
    import workloads

    gen_name, arg = DECODE_WORKLOADS[name]
    if gen_name == "long_context":
        make = None
    else:
        gen = getattr(workloads, gen_name)
        make = lambda copies: gen(arg, device=dev, copies=copies, block_size=block_size)  # noqa: E731
    if make is not None:
        probe = make(1)
        elt = 1 if probe.cache_dtype == "fp8" else 2
        pool_bytes = probe.num_blocks * probe.hkv * probe.block_size * probe.head_dim * elt * 2
        copies = max(1, min(64, math.ceil(MALL_BYTES / pool_bytes)))
        del probe
        ws = [make(copies)]
    else:
        if block_size != 16:
            raise SystemExit("bench.py: the long-context workloads use 16-token blocks")
        ws = workloads.long_context(batch=arg, device=dev, layers=32)
        copies = 1
    layers = []
    for w in ws:
        shape = (w.num_blocks, w.hkv, w.block_size, w.head_dim)
        if w.cache_dtype == "fp8":
            kp = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
            ks = torch.from_numpy(w.k_scale).to(dev)
            vs = torch.from_numpy(w.v_scale).to(dev)
            kinv = torch.from_numpy(w.k_inv_scale).to(dev)
            vinv = torch.from_numpy(w.v_inv_scale).to(dev)
        else:
            kp = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
            ks = vs = kinv = vinv = None
        vp = kp.clone()
        cache = pkv.Cache(kp, vp, ks, vs)
        for c in range(w.copies):
            slots = np.concatenate([pkv.pkv_slot_mapping(w.block_tables[c, i], w.block_size, 0, int(w.seq_lens[i]))
                                    for i in range(w.batch)])
            pkv.pkv_kv_append(cache, w.k, w.v, torch.from_numpy(slots).to(dev), kinv, vinv)
        # the step's new tokens: each sequence's last position
        last = torch.from_numpy(w.cu_seqlens[1:] - 1).to(dev)
        layers.append(dict(w=w, cache=cache, kinv=kinv, vinv=vinv,
                           k_new=w.k.index_select(0, last).contiguous(),
                           v_new=w.v.index_select(0, last).contiguous(),
                           tables=[torch.from_numpy(np.ascontiguousarray(w.block_tables[c])).to(dev)
                                   for c in range(w.copies)]))
    torch.cuda.synchronize()
    return layers, copies


def run_decode(args, dev):
    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv

    layers, copies = make_decode_setup(args.workload, dev, args.block_size)
    w0 = layers[0]["w"]
    B, hq, hkv, dh = w0.batch, w0.hq, w0.hkv, w0.head_dim
    T = int(w0.seq_lens.max())
    fp8 = w0.cache_dtype == "fp8"
    kv_elt = 1 if fp8 else 2
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    lib = pkv.load()
    lens = torch.from_numpy(w0.seq_lens.astype(np.int32)).to(dev)
    cu_new = torch.arange(B + 1, dtype=torch.int32, device=dev)
    first_pos = (lens - 1).contiguous()
    out = torch.empty(B, hq, dh, dtype=torch.float32, device=dev)
    pt = args.partition
    cache_code = {"f32": pkv.PKV_F32, "bf16": pkv.PKV_BF16, "fp8": pkv.PKV_FP8_E4M3}[w0.cache_dtype]
    ws = pkv.decode_workspace(cache_code, B, hq, hkv, dh, T, pt, dev)
    wsp = ws.data_ptr() if ws is not None else None
    wsb = ws.numel() if ws is not None else 0

    def step(i, timer=None):
        c = i % copies
        for L in layers:
            tb = L["tables"][c]
            kinv = L["kinv"].data_ptr() if fp8 else None
            vinv = L["vinv"].data_ptr() if fp8 else None
            if args.unfused:
                # slot mapping and append of the step's tokens in one launch, then the decode
                pkv._check(lib.pkv_kv_append_paged(L["cache"].ref(), L["k_new"].data_ptr(), L["v_new"].data_ptr(),
                                                   pkv.PKV_BF16, B, cu_new.data_ptr(), first_pos.data_ptr(), 1,
                                                   tb.data_ptr(), tb.shape[1], kinv, vinv, None, sh))
                if timer is not None:
                    timer.start()
                pkv._check(lib.pkv_attn_decode(L["cache"].ref(), L["w"].q.data_ptr(), pkv.PKV_BF16, B, hq,
                                               tb.data_ptr(), tb.shape[1], lens.data_ptr(), T, L["w"].scale, pt,
                                               out.data_ptr(), wsp, wsb, sh))
            else:
                # slot mapping, append and decode in one launch
                if timer is not None:
                    timer.start()
                pkv._check(lib.pkv_attn_decode_append(L["cache"].ref(), L["k_new"].data_ptr(), L["v_new"].data_ptr(),
                                                      pkv.PKV_BF16, kinv, vinv, L["w"].q.data_ptr(), pkv.PKV_BF16, B,
                                                      hq, tb.data_ptr(), tb.shape[1], lens.data_ptr(), T,
                                                      L["w"].scale, pt, out.data_ptr(), wsp, wsb, sh))
            if timer is not None:
                timer.stop()

    for i in range(args.warmup):
        step(i)
    # the K timed steps: events only around the whole run
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    # then the same steps again with events around each decode call (roofline)
    timer = Timer(stream, args.steps * len(layers))
    for i in range(args.steps):
        step(i, timer)
    torch.cuda.synchronize()
    dec_ms = timer.ms()
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    if args.calib_copy:
        calib_copy(dev)

    d_bytes = decode_bytes(w0.seq_lens, hq, hkv, dh, kv_elt, 2, fp8, w0.block_size)
    a_bytes = append_bytes(B, hkv, dh, 2, kv_elt) + B * 4 * 2    # + table entry and first_pos per token
    step_bytes = (d_bytes + a_bytes) * len(layers)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    call_bytes = d_bytes if args.unfused else d_bytes + a_bytes   # the fused call also appends
    achieved = call_bytes / (dec_avg_ms * 1e-3) / 1e9
    partition = pt or pkv.pkv_attn_decode_auto_partition(cache_code, B, hq, hkv, T)
    line = {
        "metric": (METRIC if args.workload == "gqa-b32-t4096" and w0.block_size == 16 else
                   f"decode-attn KV HBM GB/s ({args.workload}, {w0.block_size}-token blocks)"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_heads": hq, "kv_heads": hkv, "head_dim": dh,
                   "seq_len": T, "block_size": w0.block_size, "layers": len(layers), "pool_copies": copies,
                   "partition_tokens": partition, "partitions": -(-T // partition),
                   "step": "append launch + decode" if args.unfused else "append and decode in one launch"},
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "tail_waste": tail_waste(w0.seq_lens, w0.block_size),
        "new_tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "kv_tokens_per_s": round(float(w0.seq_lens.sum()) * len(layers) / (ms_step * 1e-3), 1),
        "decode_call_us": stats_us(dec_ms),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic(decode_kernel_base(w0.cache_dtype), args.workload),
                     "kernel": decode_kernel_base(w0.cache_dtype) + "_kernel" +
                               ("" if args.unfused else " (append fused)") +
                               (" + decode_merge_kernel" if partition < T else ""),
                     "bytes_per_launch": call_bytes,
                     "timing": "HIP events around each decode call on its stream (launch included)",
                     "trace": (load_trace("decode_mfma", args.workload, DECODE_SOURCES, call_bytes, PEAK_HBM_GBS,
                                          "GB/s")
                               if partition >= T and decode_kernel_base(w0.cache_dtype) == "decode_mfma" else None)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(w0, args.cpu_seconds, d_bytes)
    return line


def cpu_baseline_decode(w, target_s, d_bytes):
    """The float64 oracle on this host's cores over the first layer's batch:
    whole sequences are attended until target_s of compute has elapsed."""
    import numpy as np
    import torch

    import oracle
    from oracle import fp8 as ofp8
    threads = _blas_threads()
    q = w.q.float().cpu().double().numpy()
    per_seq_bytes = [d_bytes * int(t) / float(sum(int(x) for x in w.seq_lens)) for t in w.seq_lens]
    done_bytes, seqs, el = 0.0, 0, 0.0
    cache = {}
    b = 0
    while el < target_s:
        if b not in cache:
            k = w.seq_k(b).float().cpu().double().numpy().transpose(1, 0, 2).copy()
            v = w.seq_v(b).float().cpu().double().numpy().transpose(1, 0, 2).copy()
            if w.cache_dtype == "fp8":
                kb = w.seq_k(b).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                vb = w.seq_v(b).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                k = np.stack([ofp8.dequantize(ofp8.quantize_bf16_bits(kb[:, h], w.k_inv_scale[h]), w.k_scale[h])
                              for h in range(w.hkv)])
                v = np.stack([ofp8.dequantize(ofp8.quantize_bf16_bits(vb[:, h], w.v_inv_scale[h]), w.v_scale[h])
                              for h in range(w.hkv)])
            cache[b] = (k, v)
        k, v = cache[b]
        t0 = time.perf_counter()
        oracle.attention.decode(q[b:b + 1], [k], [v], w.scale)
        el += time.perf_counter() - t0
        done_bytes += per_seq_bytes[b]
        seqs += 1
        b = (b + 1) % w.batch
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "cores_available": len(os.sched_getaffinity(0)), "kind": "oracle", "host": _host_libs(),
            "sample": f"{seqs} sequences of the batch (float64 numpy, materialised softmax over contiguous K/V), "
                      f"{el:.1f} s of oracle compute; GB/s on the same algorithmic bytes"}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return 1


def _host_libs():
    """numpy's version and the BLAS it calls (library, version, threads)."""
    import numpy as np
    libs = {"numpy": np.__version__}
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            libs["blas"] = {"library": blas[0].get("internal_api"), "version": blas[0].get("version"),
                            "threads": blas[0].get("num_threads")}
    except Exception:  # noqa: BLE001
        pass
    return libs


# ---------------------------------------------------------------------------
# mixed chunked prefill + decode with a shared prefix
# ---------------------------------------------------------------------------

def make_mixed_setup(dev, sharers_decode=False, chunk=512, n_decode=64):
    """Blocks come from the library's allocator with the workload's seeded free
    order: 16 sequences share the prefix blocks (refcount 16) and own their
    private blocks; S0 reserves its chunk (512 tokens unless asked otherwise); 64 decode sequences hold
    their context plus the step's token. With sharers_decode the other 15
    sharers also decode: each reserves a private block for its token at
    position 2048 and joins the decode batch after the 64."""
    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv
    import workloads

    m = workloads.shared_prefix_mixed(device=dev, sharers_decode=sharers_decode, chunk=chunk, n_decode=n_decode)
    bs, hkv, dh = 16, m.hkv, m.head_dim
    alloc = pkv.BlockAllocator(m.num_blocks, bs, free_order=m.free_order)
    kp = torch.full((m.num_blocks, hkv, bs, dh), float("nan"), dtype=torch.bfloat16, device=dev)
    cache = pkv.Cache(kp, kp.clone())
    max_blocks = (m.shared + m.private + m.chunk) // bs + 1

    def append(table, first, k, v):
        s = pkv.pkv_slot_mapping(table, bs, first, k.shape[0])
        pkv.pkv_kv_append(cache, k.contiguous(), v.contiguous(), torch.from_numpy(s).to(dev))

    prefix = np.full(max_blocks, -1, dtype=np.int32)
    alloc.reserve_append(prefix, 0, m.shared)
    append(prefix, 0, *m.prefix_kv)
    n_pref = m.shared // bs
    tables = []
    for i in range(m.n_share):
        t = prefix.copy()
        if i > 0:
            alloc.incref(prefix[:n_pref])
        alloc.reserve_append(t, m.shared, m.private)
        append(t, m.shared, *m.private_kv[i])
        tables.append(t)
    t0 = tables[0]
    p0 = m.shared + m.private
    alloc.reserve_append(t0, p0, m.chunk)
    dtabs = np.full((len(m.decode_ctx), max_blocks), -1, dtype=np.int32)
    for j, ctx in enumerate(m.decode_ctx):
        ctx = int(ctx)
        alloc.reserve_append(dtabs[j], 0, ctx + 1)
        k, v = m.decode_kv[j]
        append(dtabs[j], 0, k[:ctx], v[:ctx])
    dec_ctx = m.decode_ctx.astype(np.int32)
    dec_q = m.decode_q
    dec_new_k = [kv[0][-1:] for kv in m.decode_kv]
    dec_new_v = [kv[1][-1:] for kv in m.decode_kv]
    if sharers_decode:
        for i in range(1, m.n_share):
            alloc.reserve_append(tables[i], p0, 1)      # a new private block (2048 is block-aligned)
        dtabs = np.concatenate([dtabs, np.stack(tables[1:])])
        dec_ctx = np.concatenate([dec_ctx, np.full(m.n_share - 1, p0, dtype=np.int32)])
        dec_q = torch.cat([dec_q, m.sharer_q]).contiguous()
        dec_new_k.append(m.sharer_new_kv[0])
        dec_new_v.append(m.sharer_new_kv[1])
    # the step's appends: the chunk's 512 tokens (S0) and one token per decode sequence
    new_k = torch.cat([m.chunk_kv[0]] + dec_new_k).contiguous()
    new_v = torch.cat([m.chunk_kv[1]] + dec_new_v).contiguous()
    all_tables = torch.from_numpy(np.concatenate([t0[None], dtabs])).to(dev)
    n_dec = len(dec_ctx)
    cu_new = torch.tensor([0, m.chunk] + list(range(m.chunk + 1, m.chunk + n_dec + 1)), dtype=torch.int32,
                          device=dev)
    first_pos = torch.tensor([p0] + [int(c) for c in dec_ctx], dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    return dict(m=m, cache=cache, p0=p0, max_blocks=max_blocks, all_tables=all_tables,
                new_k=new_k, new_v=new_v, cu_new=cu_new, first_pos=first_pos, dec_q=dec_q, dec_ctx=dec_ctx,
                dec_tables=all_tables[1:].contiguous(), chunk_table=all_tables[:1].contiguous(),
                dec_lens=torch.from_numpy((dec_ctx + 1).astype(np.int32)).to(dev),
                chunk_lens=torch.tensor([p0 + m.chunk], dtype=torch.int32, device=dev),
                q_start=torch.tensor([0, m.chunk], dtype=torch.int32, device=dev))


def run_mixed(args, dev):
    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv

    S = make_mixed_setup(dev, args.sharers_decode, getattr(args, "mixed_chunk", 512), getattr(args, "mixed_decodes", 64))
    m = S["m"]
    hq, hkv, dh = m.hq, m.hkv, m.head_dim
    n_dec = len(S["dec_ctx"])
    n_new = m.chunk + n_dec
    stream = torch.cuda.current_stream(dev)
    lib = pkv.load()
    sh = stream.cuda_stream
    out_p = torch.empty(m.chunk, hq, dh, dtype=torch.float32, device=dev)
    out_d = torch.empty(n_dec, hq, dh, dtype=torch.float32, device=dev)
    msl = S["max_blocks"] * 16
    ws = pkv.decode_workspace(pkv.PKV_BF16, n_dec, hq, hkv, dh, msl, args.partition, dev)
    wsp = ws.data_ptr() if ws is not None else None
    wsb = ws.numel() if ws is not None else 0
    at = S["all_tables"]

    # the mixed step: one decode launch whose last workgroups append the
    # chunk's 512 tokens (each decode appends its own), then the prefill
    r = m.chunk
    k_ch, v_ch = S["new_k"][:r], S["new_v"][:r]
    k_dec, v_dec = S["new_k"][r:], S["new_v"][r:]
    chunk_b = pkv._ChunkBatch(1, m.chunk_q.data_ptr(), S["q_start"].data_ptr(), k_ch.data_ptr(), v_ch.data_ptr(),
                              S["chunk_table"].data_ptr(), S["max_blocks"], S["chunk_lens"].data_ptr(), m.chunk,
                              out_p.data_ptr())
    dec_b = pkv._DecodeBatch(n_dec, S["dec_q"].data_ptr(), k_dec.data_ptr(), v_dec.data_ptr(),
                             S["dec_tables"].data_ptr(), S["max_blocks"], S["dec_lens"].data_ptr(), msl,
                             args.partition, out_d.data_ptr(), wsp, wsb)

    def mixed_step():
        pkv._check(lib.pkv_attn_mixed_step(S["cache"].ref(), hq, m.scale, ctypes.byref(chunk_b),
                                           ctypes.byref(dec_b), sh))

    def step(tp=None, td=None):
        pkv._check(lib.pkv_kv_append_paged(S["cache"].ref(), S["new_k"].data_ptr(), S["new_v"].data_ptr(),
                                           pkv.PKV_BF16, at.shape[0], S["cu_new"].data_ptr(), S["first_pos"].data_ptr(),
                                           m.chunk, at.data_ptr(), at.shape[1], None, None, None, sh))
        if tp is not None:
            tp.start()
        pkv._check(lib.pkv_attn_prefill_chunk(S["cache"].ref(), m.chunk_q.data_ptr(), pkv.PKV_BF16, 1, hq,
                                              S["q_start"].data_ptr(), S["chunk_table"].data_ptr(),
                                              S["max_blocks"], S["chunk_lens"].data_ptr(), m.chunk, m.scale,
                                              out_p.data_ptr(), sh))
        if tp is not None:
            tp.stop()
            td.start()
        pkv._check(lib.pkv_attn_decode(S["cache"].ref(), S["dec_q"].data_ptr(), pkv.PKV_BF16, n_dec, hq,
                                       S["dec_tables"].data_ptr(), S["max_blocks"], S["dec_lens"].data_ptr(), msl,
                                       m.scale, args.partition, out_d.data_ptr(), wsp, wsb, sh))
        if td is not None:
            td.stop()

    timed_step = step if args.unfused else mixed_step
    for _ in range(args.warmup):
        timed_step()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        timed_step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    # the kernels one by one (separate calls) with events around each
    tp, td = Timer(stream, args.steps), Timer(stream, args.steps)
    for _ in range(args.steps):
        step(tp, td)
    torch.cuda.synchronize()
    p_ms, d_ms = tp.ms(), td.ms()
    p_avg, d_avg = sum(p_ms) / len(p_ms), sum(d_ms) / len(d_ms)
    if args.calib_copy:
        calib_copy(dev)
    flops = prefill_flops(S["p0"], m.chunk, hq, dh)
    d_bytes = decode_bytes(S["dec_ctx"] + 1, hq, hkv, dh, 2, 2, False)
    p_tflops = flops / (p_avg * 1e-3) / 1e12
    line = {
        "metric": f"mixed step: causal {m.chunk}-token prefill chunk TFLOP/s (bf16 MFMA) + {n_dec} decodes, shared prefix",
        "value": round(p_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": MIXED_WORKLOAD, "q_heads": hq, "kv_heads": hkv, "head_dim": dh, "block_size": 16,
                   "prefix_tokens": S["p0"], "chunk": m.chunk, "shared_prefix_tokens": m.shared,
                   "sharers": m.n_share, "decodes": n_dec,
                   "sharers_decoding": m.n_share - 1 if args.sharers_decode else 0,
                   "decode_ctx_mean": float(np.mean(S["dec_ctx"])) + 1.0,
                   "step": ("append launch + prefill + decode" if args.unfused else {
                       "two": "pkv_attn_mixed_step: decode launch that also appends the chunk, then the prefill",
                       "one": "pkv_attn_mixed_step: one launch of eight-wave workgroups (appends, decodes, prefill)",
                   }.get(os.environ.get("PKV_MIXED"), "pkv_attn_mixed_step: one launch, a prefill tile beside a "
                                                       "decode workgroup on every CU (four-wave workgroups)"))},
        "prefill_us": stats_us(p_ms),
        "prefill_flops": flops,
        "decode_us": stats_us(d_ms),
        "decode_gbs": round(d_bytes / (d_avg * 1e-3) / 1e9, 2),
        "decode_bytes": d_bytes,
        "roofline": {"bound": "mfma", "achieved": round(p_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(p_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_stream_kernel (the chunk as its own call)", "flops_per_launch": flops},
        "decode_roofline": {"bound": "hbm", "achieved": round(d_bytes / (d_avg * 1e-3) / 1e9, 2),
                            "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(d_bytes / (d_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(m, S["p0"], flops)
    return line


def cpu_baseline_prefill(m, p0, flops):
    """The float64 oracle's prefill chunk (materialised causal attention over
    the contiguous 2560-token cache), once."""
    import numpy as np

    import oracle
    f = lambda t: t.float().cpu().double().numpy()  # noqa: E731
    k = np.concatenate([f(m.prefix_kv[0]), f(m.private_kv[0][0]), f(m.chunk_kv[0])]).transpose(1, 0, 2).copy()
    v = np.concatenate([f(m.prefix_kv[1]), f(m.private_kv[0][1]), f(m.chunk_kv[1])]).transpose(1, 0, 2).copy()
    q = f(m.chunk_q)
    t0 = time.perf_counter()
    oracle.attention.prefill_chunk(q, k, v, m.scale)
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(_blas_threads()),
            "cores_available": len(os.sched_getaffinity(0)), "kind": "oracle", "host": _host_libs(),
            "sample": f"the whole 512-query chunk on {p0 + m.chunk} cached tokens, once "
                      f"(float64 numpy, materialised causal softmax), {el:.2f} s"}


# ---------------------------------------------------------------------------
# one prefill chunk alone (the mixed step's head layout, any prefix and chunk length)
# ---------------------------------------------------------------------------

def run_prefill_chunk(args, dev):
    """One sequence: a causal chunk of --chunk queries over --prefix cached
    tokens plus the chunk's own (Hq=32, Hkv=8, Dh=128, bf16 N(0,1), blocks of
    --block-size tokens at a seeded random permutation). A step is one
    pkv_attn_prefill_chunk call; the kernel is the library's choice unless
    PKV_PREFILL_KERNEL names one."""
    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv

    hq, hkv, dh = 32, 8, 128
    P, C = args.prefix, args.chunk
    T = P + C
    bsz = args.block_size
    nb = -(-T // bsz)
    rng = np.random.default_rng(4306)
    gen = torch.Generator(device=dev).manual_seed(4306)
    kp = torch.randn(nb + 8, hkv, bsz, dh, generator=gen, device=dev).to(torch.bfloat16)
    vp = torch.randn(nb + 8, hkv, bsz, dh, generator=gen, device=dev).to(torch.bfloat16)
    cache = pkv.Cache(kp, vp)
    table = torch.from_numpy(rng.permutation(nb + 8)[:nb].astype(np.int32)[None]).to(dev)
    q = torch.randn(C, hq, dh, generator=gen, device=dev).to(torch.bfloat16)
    q_start = torch.tensor([0, C], dtype=torch.int32, device=dev)
    lens = torch.tensor([T], dtype=torch.int32, device=dev)
    out = torch.empty(C, hq, dh, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(dh)
    stream = torch.cuda.current_stream(dev)
    lib = pkv.load()

    def step():
        pkv._check(lib.pkv_attn_prefill_chunk(cache.ref(), q.data_ptr(), pkv.PKV_BF16, 1, hq, q_start.data_ptr(),
                                              table.data_ptr(), nb, lens.data_ptr(), C, scale, out.data_ptr(),
                                              stream.cuda_stream))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    timer = Timer(stream, args.steps)
    for _ in range(args.steps):
        timer.start()
        step()
        timer.stop()
    torch.cuda.synchronize()
    call = timer.ms()
    avg = sum(call) / len(call)
    if getattr(args, "calib_copy", False):
        calib_copy(dev)
    flops = prefill_flops(P, C, hq, dh)
    env = os.environ.get("PKV_PREFILL_KERNEL")
    kernel = env if env in ("tiles", "tiles128", "tiles256", "tiles16", "columns") else (
        "columns" if C * hq < 128 * 64 and nb * bsz <= 8192 and bsz >= 16 else "tiles256" if C * hq >= 2 * 256 * 256
        else "tiles128" if C * hq >= 128 * 256 else "tiles")
    names = {"tiles": "prefill_stream_kernel", "tiles128": "prefill_stream_kernel (128 rows)",
             "tiles256": "prefill_stream_kernel (256 rows)",
             "tiles16": "prefill_kernel",
             "columns": "decode_mfma_kernel (prefill columns)"}
    tf = flops / (avg * 1e-3) / 1e12
    pipelined = flops / (ms * 1e-3) / 1e12
    if kernel in ("tiles16", "columns") and bsz < 16:
        kernel = "tiles"                   # 8-token blocks: the key-stream kernel whatever is asked
    rg = {"tiles128": 4, "tiles256": 8 if dh == 128 else 4}.get(kernel, 2)   # row groups per key stream
    # the key-stream kernel's name: prefill_stream_kernel<Dh, row groups, 8-token blocks>
    stream_name = f"prefill_stream_kernel<{dh}, {rg}, {'true' if bsz == 8 else 'false'}>"
    line = {
        "metric": f"prefill chunk TFLOP/s (bf16 MFMA), C={C} on P={P}",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill-chunk", "q_heads": hq, "kv_heads": hkv, "head_dim": dh, "block_size": bsz,
                   "prefix_tokens": P, "chunk": C,
                   "kernel": names[kernel]},
        "call_us": stats_us(call),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": (load_prefill_traffic(C, stream_name)
                                 if kernel in ("tiles", "tiles128", "tiles256") else None),
                     "flops_per_launch": flops,
                     "timing": "HIP events around each call on its stream (launch included)",
                     "pipelined": {"timing": "K back-to-back calls between two events", "achieved": round(pipelined, 2),
                                   "frac": round(pipelined / PEAK_BF16_TFLOPS, 4)},
                     "trace": (load_trace("prefill_stream", trace_key("prefill-chunk", C), PREFILL_SOURCES, flops,
                                          PEAK_BF16_TFLOPS, "TFLOP/s",
                                          name_has=stream_name)
                               if kernel in ("tiles", "tiles128", "tiles256") else None)},
    }
    return line


# ---------------------------------------------------------------------------
# counter summaries
# ---------------------------------------------------------------------------

def summarize_counters(fetch_csv, write_csv, workload, chunk=None):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the decode kernels (or,
    for prefill-chunk, of the key-stream prefill kernel; for append, of the
    bulk append's dispatches, the second half of the run's append dispatches),
    each scaled by the factor that maps the calibration copy's reading onto
    the bytes it is known to move."""
    def load(path, counter):
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                per.setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0)
        return per

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")

    def pick(per, key):
        names = [n for n in per if key in n]
        if not names:
            raise SystemExit(f"no dispatch of {key} in the counter file")
        return names[0], per[names[0]]

    _, cf = pick(fetch, "copy_blocks_kernel")
    _, cw = pick(write, "copy_blocks_kernel")
    f_scale = CALIB_BYTES / cf[-1]
    w_scale = CALIB_BYTES / cw[-1]
    prefill = workload == "prefill-chunk"
    append = workload == "append"
    sources = PREFILL_SOURCES if prefill else APPEND_SOURCES if append else DECODE_SOURCES
    out = {"workload": trace_key(workload, chunk) if prefill else workload,
           "source_hash": source_hash(sources),
           "calibration": {"kernel": "copy_blocks_kernel", "bytes": CALIB_BYTES,
                           "fetch_bytes_read": cf[-1], "write_bytes_read": cw[-1],
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": {}}
    total = 0.0
    if prefill:
        base, keys = "prefill_stream", ("prefill_stream_kernel",)
    elif append:
        base, keys = "kv_append_paged", ("kv_append_paged_kernel",)
        # the step shape is timed first, then the bulk shape, with the same
        # number of dispatches each: keep the bulk half
        for per in (fetch, write):
            for n in [n for n in per if keys[0] in n]:
                per[n] = per[n][len(per[n]) // 2:]
    else:
        base = "decode_mfma" if any("decode_mfma_kernel" in n for n in fetch) else "decode_split"
        keys = (base + "_kernel", "decode_merge_kernel")
    for key in keys:
        names = [n for n in fetch if key in n]
        if not names:
            continue
        fv = fetch[names[0]]
        wv = write[[n for n in write if key in n][0]]
        fb = sum(fv) / len(fv) * f_scale
        wb = sum(wv) / len(wv) * w_scale
        out["kernels"][key] = {"name": names[0], "dispatches": len(fv), "fetch_bytes": fb, "write_bytes": wb}
        total += fb + wb
    out["bytes_per_launch"] = round(total)
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"{base}_{out['workload']}_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return out


def load_prefill_traffic(chunk, kernel_name_has):
    """HBM bytes per launch of the key-stream prefill from a committed counter
    summary of this chunk size, if taken on the current sources and of the
    same kernel form; else None."""
    path = os.path.join(PROFILES, f"prefill_stream_{trace_key('prefill-chunk', chunk)}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("source_hash") != source_hash(PREFILL_SOURCES):
        return None
    k = tr.get("kernels", {}).get("prefill_stream_kernel", {})
    if kernel_name_has not in k.get("name", ""):
        return None
    return tr["bytes_per_launch"]


# ---------------------------------------------------------------------------
# prefix-cache index (host)
# ---------------------------------------------------------------------------

def run_prefix_index(args):
    """Host workload for the prefix-cache index: 16 system prompts of 2048
    tokens shared by 512 requests that each add 512 private tokens (16-token
    blocks). All requests are indexed, then 512 new requests of the same mix
    are matched; a step is matching those 512 prompts. Reported as blocks
    looked up per second (each request walks its matched blocks plus the
    first miss); the oracle's Python index is timed on the same lookups."""
    import numpy as np

    import paged_kv_cache_430_amd as pkv
    from oracle import prefix as oprefix

    page, n_sys, sys_len, n_req, priv = 16, 16, 2048, 512, 512
    rng = np.random.default_rng(4306)
    systems = [rng.integers(0, 32000, sys_len).astype(np.int32) for _ in range(n_sys)]

    def prompts(n):
        return [np.concatenate([systems[int(rng.integers(0, n_sys))],
                                rng.integers(0, 32000, priv).astype(np.int32)]) for _ in range(n)]

    cached, queries = prompts(n_req), prompts(n_req)
    idx = pkv.PrefixIndex(page)
    nid = 0
    for t in cached:
        nb = len(t) // page
        idx.insert(t, np.arange(nid, nid + nb, dtype=np.int32))
        nid += nb
    lib = pkv.load()
    qbufs = [np.ascontiguousarray(q) for q in queries]
    out = np.empty((sys_len + priv) // page, dtype=np.int32)
    n = pkv.ctypes.c_int32(0)
    lookups = 0
    for q in qbufs:
        pkv._check(lib.pkv_prefix_match(idx._h, None, q.ctypes.data, len(q), 0, out.ctypes.data, len(out),
                                        pkv.ctypes.addressof(n)))
        lookups += n.value + (1 if n.value < len(q) // page else 0)
    for _ in range(args.warmup):
        for q in qbufs:
            lib.pkv_prefix_match(idx._h, None, q.ctypes.data, len(q), 0, out.ctypes.data, len(out),
                                 pkv.ctypes.addressof(n))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for q in qbufs:
            lib.pkv_prefix_match(idx._h, None, q.ctypes.data, len(q), 0, out.ctypes.data, len(out),
                                 pkv.ctypes.addressof(n))
    el = time.perf_counter() - t0
    value = lookups * args.steps / el
    line = {
        "metric": "prefix-index match, blocks looked up per second (host)",
        "value": round(value, 1), "unit": "blocks/s", "n_gpus": 0, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(el / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": "prefix-index", "block_size": page, "system_prompts": n_sys,
                   "system_tokens": sys_len, "requests": n_req, "private_tokens": priv,
                   "indexed_blocks": idx.stats()["entries"]},
        "us_per_request": round(el / args.steps / n_req * 1e6, 3),
        "roofline": None,
    }
    if not args.no_cpu_baseline:
        ref = oprefix.PrefixIndex(page)
        nid = 0
        for t in cached:
            nb = len(t) // page
            ref.insert(list(map(int, t)), list(range(nid, nid + nb)))
            nid += nb
        ql = [list(map(int, q)) for q in queries]
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            for q in ql:
                ref.match(q)
            reps += 1
        el_o = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(lookups * reps / el_o, 1), "unit": "blocks/s", "cores": 1,
                                "kind": "oracle", "host": _host_libs(), "sample": f"{reps} passes over the 512 prompts (Python dict of "
                                                            f"nested-tuple keys), {el_o:.2f} s"}
    return line


# ---------------------------------------------------------------------------
# swap-out / swap-in (pool <-> pinned host memory)
# ---------------------------------------------------------------------------

def run_swap(args, dev):
    """4096 scattered blocks of a pool shaped like the headline's (Hkv=8, Dh=128, bf16: 64 KiB
    of K+V per block, 256 MiB per call) out to pinned host memory and back in.
    `value` is the swap-out rate; the line also carries the swap-in rate.
    Both directions are bound by the host link, not by HBM."""
    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv

    nb, hkv, dh, n = 8192, 8, 128, 4096
    k = torch.randn(nb, hkv, 16, dh, device=dev).to(torch.bfloat16)
    v = torch.randn(nb, hkv, 16, dh, device=dev).to(torch.bfloat16)
    cache = pkv.Cache(k, v)
    ids = torch.from_numpy(np.random.default_rng(4307).permutation(nb)[:n].astype(np.int32)).to(dev)
    bb = hkv * 16 * dh * 2
    host = torch.empty(n * 2 * bb, dtype=torch.uint8).pin_memory()
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_out = timed(lambda: pkv.pkv_swap_out(cache, ids, host))
    ms_in = timed(lambda: pkv.pkv_swap_in(cache, host, ids))
    moved = n * 2 * bb
    return {
        "metric": "swap-out of 4096 KV blocks to pinned host memory, GB/s",
        "value": round(moved / (ms_out * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_out, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap", "blocks": n, "pool_blocks": nb, "kv_heads": hkv, "head_dim": dh,
                   "block_size": 16, "bytes_per_call": moved},
        "swap_in_gbs": round(moved / (ms_in * 1e-3) / 1e9, 2), "swap_in_ms": round(ms_in, 4),
        # the host link: PCIe 5.0 x16, 32 GT/s per lane with 128b/130b coding, per direction
        "roofline": {"bound": "host-link", "achieved": round(moved / (ms_out * 1e-3) / 1e9, 2),
                     "peak": PCIE5_X16_GBS, "unit": "GB/s",
                     "frac": round(moved / (ms_out * 1e-3) / 1e9 / PCIE5_X16_GBS, 4), "traffic": None,
                     "kernel": "swap_out_kernel", "bytes_per_launch": moved},
    }


# ---------------------------------------------------------------------------
# the box's read-bandwidth ceiling for the decode's access pattern
# ---------------------------------------------------------------------------

def run_mfma_ceiling(args, dev):
    """pkv_debug_mfma_rate: the prefill steady iteration's 24 bf16 products
    per wave, from one 8-wave workgroup per CU (two waves per SIMD, as the
    prefill runs) on N(0,1) operands, timed with events over K launches.
    Beside it, pkv_debug_prefill_mix: the same products with the iteration's
    vector work, then also its LDS operand reads (mode 1), then also its
    LDS-direct tile loads and barrier (mode 2), per iteration as many as the
    prefill moves."""
    import torch

    import paged_kv_cache_430_amd as pkv

    gen = torch.Generator(device=dev).manual_seed(4307)
    ops = torch.randn(1024, generator=gen, device=dev).to(torch.bfloat16)
    tiles = torch.randn((1 << 20) // 2, generator=gen, device=dev).to(torch.bfloat16)
    nwg = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4096
    sink = torch.empty(nwg * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    flops = nwg * 8 * iters * 24 * 2 * 32 * 32 * 16

    def timed(call):
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        timer = Timer(stream, args.steps)
        for _ in range(args.steps):
            timer.start()
            call()
            timer.stop()
        torch.cuda.synchronize()
        ms = timer.ms()
        return ms, sum(ms) / len(ms)

    ms, avg = timed(lambda: pkv.pkv_debug_mfma_rate(ops, iters, nwg, sink))
    tf = flops / (avg * 1e-3) / 1e12
    mix = {}
    for mode, name in ((0, "products+vector"), (1, "+lds_reads"), (2, "+lds_reads+tile_loads+barrier")):
        _, a = timed(lambda: pkv.pkv_debug_prefill_mix(ops, tiles, mode, iters, nwg, sink))
        mix[name] = {"call_us": round(a * 1e3, 2), "tflops": round(flops / (a * 1e-3) / 1e12, 1),
                     "us_per_iteration": round(a * 1e3 / iters, 4)}
    return {
        "metric": "sustained bf16 MFMA TFLOP/s, prefill steady-iteration products, every CU busy",
        "value": round(tf, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(avg, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mfma-ceiling", "workgroups": nwg, "waves_per_workgroup": 8, "iterations": iters,
                   "mfma": "v_mfma_f32_32x32x16_bf16 x 24 per wave-iteration"},
        "call_us": stats_us(ms),
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": "mfma_rate_kernel",
                     "flops_per_launch": flops},
        "prefill_mix": mix,
    }


def run_read_ceiling(args, dev):
    """pkv_debug_stream_read over a 2 GiB buffer of 4 KiB tiles (the decode's
    (block, head) tile at bf16, Dh=128, 16-token blocks), with the decode's
    non-temporal buffer loads and no arithmetic: tiles in order, and tiles in a
    seeded random order (a paged pool read through its tables), each with one
    8-wave workgroup per CU (the decode's shape) and with four per CU. `value`
    is the scattered order at one workgroup per CU."""
    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv

    n_tiles = MALL_BYTES // 4096
    buf = torch.empty(n_tiles * 1024, dtype=torch.int32, device=dev)
    buf.random_(generator=torch.Generator(device=dev).manual_seed(4307))
    rng = np.random.default_rng(4307)
    orders = {"in order": torch.arange(n_tiles, dtype=torch.int32, device=dev),
              "random order": torch.from_numpy(rng.permutation(n_tiles).astype(np.int32)).to(dev)}
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, ids in orders.items():
        for nwg in (256, 1024):
            sink = torch.empty(nwg, dtype=torch.int32, device=dev)
            for _ in range(args.warmup):
                pkv.pkv_debug_stream_read(buf, ids, nwg, sink)
            timer = Timer(stream, args.steps)
            for _ in range(args.steps):
                timer.start()
                pkv.pkv_debug_stream_read(buf, ids, nwg, sink)
                timer.stop()
            torch.cuda.synchronize()
            ms = timer.ms()
            avg = sum(ms) / len(ms)
            res[f"{name}, {nwg} workgroups"] = {"GB/s": round(n_tiles * 4096 / (avg * 1e-3) / 1e9, 1),
                                                "call_us": stats_us(ms)}
    key = "random order, 256 workgroups"
    gbs = res[key]["GB/s"]
    return {
        "metric": "HBM streaming-read ceiling: 2 GiB of 4 KiB tiles in random order, GB/s",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res[key]["call_us"]["mean"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": "read-ceiling", "bytes_per_call": n_tiles * 4096, "tile_bytes": 4096,
                   "waves_per_workgroup": 8},
        "results": res,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "stream_read_kernel",
                     "bytes_per_launch": n_tiles * 4096},
    }


# ---------------------------------------------------------------------------
# slot mapping + KV append alone
# ---------------------------------------------------------------------------

def run_append(args, dev):
    """pkv_kv_append_paged (slot mapping and append in one launch), bf16 pool,
    Hkv=8, Dh=128, 16-token blocks at a seeded random permutation. Two shapes:
    the shared-prefix mixed step's appends (a 512-token chunk on a 2048-token
    cache plus 64 sequences appending one token: 576 tokens) and a bulk append
    of 16 sequences x 2048 tokens (32768 tokens), whose rate is `value`.
    Algorithmic bytes per token: K and V read from the input and written to
    the pool (2 x Hkv x Dh x 2 bytes each way) plus one table entry and one
    slot computation's inputs (8 bytes). Each shape rotates through copies of
    its pool and inputs (at least 2 GiB together), so that no call finds the
    previous call's lines in the caches."""
    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv

    hkv, dh, bs = 8, 128, 16
    per_token = 2 * hkv * dh * 2 * 2 + 8
    rng = np.random.default_rng(4308)
    gen = torch.Generator(device=dev).manual_seed(4308)
    stream = torch.cuda.current_stream(dev)

    def setup(first, counts):
        total_blocks = sum(-(-(f + c) // bs) for f, c in zip(first, counts))
        perm = rng.permutation(total_blocks).astype(np.int32)
        max_blocks = max(-(-(f + c) // bs) for f, c in zip(first, counts))
        bt = np.full((len(first), max_blocks), -1, dtype=np.int32)
        pos = 0
        for i, (f, c) in enumerate(zip(first, counts)):
            nb = -(-(f + c) // bs)
            bt[i, :nb] = perm[pos:pos + nb]
            pos += nb
        n = sum(counts)
        copy_bytes = (total_blocks * bs + n) * hkv * dh * 2 * 2
        sets = []
        for _ in range(max(1, min(16, math.ceil(MALL_BYTES / copy_bytes)))):
            kp = torch.zeros(total_blocks, hkv, bs, dh, dtype=torch.bfloat16, device=dev)
            k = torch.randn(n, hkv, dh, generator=gen, device=dev).to(torch.bfloat16)
            v = torch.randn(n, hkv, dh, generator=gen, device=dev).to(torch.bfloat16)
            sets.append((pkv.Cache(kp, torch.zeros_like(kp)), k, v))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device=dev)
        fp = torch.tensor(np.array(first, dtype=np.int32), device=dev)
        return sets, torch.from_numpy(bt).to(dev), cu, fp, max(counts), bt, n

    def timed(c):
        sets, btd, cu, fp, mx, _, n = c
        for i in range(args.warmup):
            cache, k, v = sets[i % len(sets)]
            pkv.pkv_kv_append_paged(cache, k, v, btd, cu, fp, mx)
        timer = Timer(stream, args.steps)
        for i in range(args.steps):
            cache, k, v = sets[(args.warmup + i) % len(sets)]
            timer.start()
            pkv.pkv_kv_append_paged(cache, k, v, btd, cu, fp, mx)
            timer.stop()
        torch.cuda.synchronize()
        return timer.ms()

    step = setup([2048] + [int(t) for t in rng.integers(256, 2049, 64)], [512] + [1] * 64)
    bulk = setup([0] * 16, [2048] * 16)
    ms_step, ms_bulk = timed(step), timed(bulk)
    if getattr(args, "calib_copy", False):
        calib_copy(dev)
    avg_bulk = sum(ms_bulk) / len(ms_bulk)
    gbs = bulk[-1] * per_token / (avg_bulk * 1e-3) / 1e9
    traffic = load_traffic("kv_append_paged", "append", APPEND_SOURCES)
    line = {
        "metric": "paged KV append (slot mapping + append, one launch), bulk 32768 tokens, GB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(avg_bulk, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "append", "kv_heads": hkv, "head_dim": dh, "block_size": bs,
                   "bulk_tokens": bulk[-1], "step_tokens": step[-1], "bytes_per_token": per_token,
                   "pool_copies": {"bulk": len(bulk[0]), "step": len(step[0])}},
        "bulk_us": stats_us(ms_bulk),
        "step_576_tokens_us": stats_us(ms_step),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": "kv_append_paged_kernel",
                     "bytes_per_launch": bulk[-1] * per_token},
    }
    if not args.no_cpu_baseline:
        import oracle
        sets, _, _, _, _, bt, _ = bulk
        _, k, v = sets[0]
        kh = k.float().cpu().numpy()
        vh = v.float().cpu().numpy()
        pool_k = np.zeros((int(bt.max()) + 1, hkv, bs, dh), dtype=np.float32)
        pool_v = np.zeros_like(pool_k)
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) and done < bulk[-1]:
            seq, off = divmod(done, 2048)
            slots = oracle.paging.slot_mapping(bt[seq], off, 256, bs)
            oracle.paging.append(pool_k, kh[done:done + 256], slots, bs)
            oracle.paging.append(pool_v, vh[done:done + 256], slots, bs)
            done += 256
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(done * per_token / el / 1e9, 4), "unit": "GB/s", "cores": 1,
                                "cores_available": len(os.sched_getaffinity(0)), "kind": "oracle",
                                "host": _host_libs(),
                                "sample": f"{done} of the bulk tokens through the oracle's slot mapping and "
                                          f"append (Python loop per token), {el:.2f} s"}
    return line


# ---------------------------------------------------------------------------
# the host block allocator
# ---------------------------------------------------------------------------

def run_allocator(args):
    """Host workload for the block allocator: the shared-prefix workload's
    block bookkeeping, built and torn down once per step. 16 sequences share
    a 1024-token prefix (64 full blocks, one allocation then 15 increfs) and
    grow 1024 private tokens each; sequence 0 reserves a 512-token chunk; 64
    other sequences reserve their contexts (uniform in [257, 2049] tokens);
    then every table is released (decref). Reported as allocator calls per
    second through the Python binding (each call crosses ctypes); the
    oracle's pure-Python model runs the same calls."""
    import numpy as np

    import paged_kv_cache_430_amd as pkv
    from oracle import allocator as oalloc

    bs, shared, private, chunk, n_share = 16, 1024, 1024, 512, 16
    rng = np.random.default_rng(4304)
    ctx = rng.integers(257, 2050, 64)
    max_blocks = (shared + private + chunk) // bs + 1
    num_blocks = shared // bs + n_share * private // bs + chunk // bs + int(sum(-(-int(t) // bs) for t in ctx)) + 64

    def one_step(a, native):
        calls = 0
        def reserve(t, l, n):
            nonlocal calls
            calls += 1
            if native:
                a.reserve_append(t, l, n)
                return t
            st, t2, _ = a.reserve_append(t, l, n)
            assert st == oalloc.OK
            return t2
        def table():
            return np.full(max_blocks, -1, dtype=np.int32) if native else [-1] * max_blocks
        prefix = reserve(table(), 0, shared)
        tables = []
        for i in range(n_share):
            t = prefix.copy() if native else list(prefix)
            if i > 0:
                a.incref(t[:shared // bs])
                calls += 1
            tables.append(reserve(t, shared, private))
        tables[0] = reserve(tables[0], shared + private, chunk)
        for c in ctx:
            tables.append(reserve(table(), 0, int(c)))
        for t in tables:
            a.decref(t[t >= 0] if native else [x for x in t if x >= 0])
            calls += 1
        return calls

    nat = pkv.BlockAllocator(num_blocks, bs)
    for _ in range(args.warmup):
        one_step(nat, True)
    t0 = time.perf_counter()
    calls = 0
    for _ in range(args.steps):
        calls += one_step(nat, True)
    el = time.perf_counter() - t0
    assert nat.num_free() == num_blocks
    line = {
        "metric": "block allocator: shared-prefix set-up and release, allocator calls per second (host)",
        "value": round(calls / el, 1), "unit": "calls/s", "n_gpus": 0, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(el / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": "allocator", "block_size": bs, "num_blocks": num_blocks, "sharers": n_share,
                   "shared_tokens": shared, "private_tokens": private, "chunk": chunk, "decodes": len(ctx),
                   "calls_per_step": calls // args.steps},
        "roofline": None,
    }
    if not args.no_cpu_baseline:
        model = oalloc.ModelAllocator(num_blocks, bs)
        t0 = time.perf_counter()
        reps, mcalls = 0, 0
        while reps < args.steps and time.perf_counter() - t0 < args.cpu_seconds:
            mcalls += one_step(model, False)
            reps += 1
        mel = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(mcalls / mel, 1), "unit": "calls/s", "cores": 1,
                                "cores_available": len(os.sched_getaffinity(0)), "kind": "oracle",
                                "host": _host_libs(),
                                "sample": f"{reps} of the same steps on the oracle's pure-Python allocator model, "
                                          f"{mel:.2f} s"}
    return line


def main():
    args = parse()
    if args.counters:
        summarize_counters(args.counters[0], args.counters[1], args.workload, args.chunk)
        return
    if args.trace_summary:
        summarize_trace(args.trace_summary, args.workload, args.chunk)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(decode shards by sequence or KV head with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    if args.workload == "prefix-index":   # host only
        print(json.dumps(run_prefix_index(args)), flush=True)
        return
    if args.workload == "allocator":      # host only
        print(json.dumps(run_allocator(args)), flush=True)
        return

    import torch

    import paged_kv_cache_430_amd as pkv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    pkv.load()
    if args.workload == "swap":
        line = run_swap(args, dev)
    elif args.workload == MIXED_WORKLOAD:
        line = run_mixed(args, dev)
    elif args.workload == "prefill-chunk":
        line = run_prefill_chunk(args, dev)
    elif args.workload == "read-ceiling":
        line = run_read_ceiling(args, dev)
    elif args.workload == "mfma-ceiling":
        line = run_mfma_ceiling(args, dev)
    elif args.workload == "append":
        line = run_append(args, dev)
    else:
        line = run_decode(args, dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
