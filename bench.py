#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X.

Default workload (the headline metric): GQA paged decode, B=32 sequences,
Hq=32, Hkv=8, Dh=128, every sequence 4096 tokens, bf16 cache, block size 16.
One step is the whole decode hot path for the batch:
  1. slot mapping on the device for the 32 new tokens (position 4095),
  2. KV append of those tokens through the block table,
  3. split-KV paged decode attention over all 4096 tokens (one kernel,
     partitions merged in-kernel).
Inputs are resident in HBM before timing. Four copies of the pool behind
four block-table sets (2 GiB in total) are used in rotation so that the
256 MB Infinity Cache cannot serve a step from the previous one.

Prints one JSON line. `value` is algorithmic HBM bytes per step (KV read +
q + out + tables + lengths + append traffic) divided by the step time;
`roofline` reports the decode kernel alone, timed with HIP events on the
stream it runs on; `cpu_baseline` times the float64 CPU oracle on the same
batch on this host.

Other decode workloads are available with --workload for exploration; they
print the same kind of line.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV HBM GB/s (% of peak), B=32 Hkv=8 Dh=128 T=4096 bf16"
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 2 * 2 ** 30          # rotate through at least this much pool memory
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DECODE_SOURCES = ["paged_kv_cache_430_amd/csrc/decode.hip", "paged_kv_cache_430_amd/csrc/device_common.h"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="cfg2-all4096",
                   choices=["cfg2-all4096", "cfg2-uniform", "cfg5-mha", "cfg5-gqa", "cfg5-mqa", "cfg5-gqa-fp8",
                            "cfg3-b1", "cfg3-b4"])
    p.add_argument("--partition", type=int, default=0, help="partition_tokens (0 = library default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time for the oracle baseline")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after timing, run a plain device copy of this size (for counter calibration)")
    return p.parse_args()


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_bytes(seq_lens, hq, hkv, dh, kv_elt, q_elt, fp8):
    """Algorithmic bytes of one decode call: every visible K and V element
    once, q, the fp32 output, the block-table entries and lengths read."""
    kv = sum(int(t) for t in seq_lens) * hkv * dh * 2 * kv_elt
    b = len(seq_lens)
    extra = b * hq * dh * q_elt + b * hq * dh * 4 + sum(-(-int(t) // 16) for t in seq_lens) * 4 + 4 * b
    if fp8:
        extra += 2 * hkv * 4
    return kv + extra


def append_bytes(n_tokens, hkv, dh, in_elt, cache_elt):
    return n_tokens * hkv * dh * 2 * (in_elt + cache_elt) + n_tokens * 4


def make_decode_setup(name, dev):
    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv
    import workloads

    if name.startswith("cfg2"):
        make = lambda copies: workloads.cfg2(name.split("-", 1)[1], device=dev, copies=copies)  # noqa: E731
        layers = 1
    elif name.startswith("cfg5"):
        make = lambda copies: workloads.cfg5(name.split("-", 1)[1], device=dev, copies=copies)  # noqa: E731
        layers = 1
    else:
        layers = 32
        make = None
    if make is not None:
        probe = make(1)
        elt = 1 if probe.cache_dtype == "fp8" else 2
        pool_bytes = probe.num_blocks * probe.hkv * 16 * probe.head_dim * elt * 2
        copies = max(1, min(64, math.ceil(MALL_BYTES / pool_bytes)))
        del probe
        ws = [make(copies)]
    else:
        b = int(name.split("-b")[1])
        ws = workloads.cfg3(batch=b, device=dev, layers=layers)
        copies = 1
    caches, tables = [], []
    for w in ws:
        shape = (w.num_blocks, w.hkv, 16, w.head_dim)
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
            slots = np.concatenate([pkv.pkv_slot_mapping(w.block_tables[c, i], 16, 0, int(w.seq_lens[i]))
                                    for i in range(w.batch)])
            pkv.pkv_kv_append(cache, w.k, w.v, torch.from_numpy(slots).to(dev), kinv, vinv)
        # the step's new tokens: each sequence's last position
        last = torch.from_numpy(w.cu_seqlens[1:] - 1).to(dev)
        k_new = w.k.index_select(0, last).contiguous()
        v_new = w.v.index_select(0, last).contiguous()
        caches.append(dict(w=w, cache=cache, k_new=k_new, v_new=v_new, kinv=kinv, vinv=vinv,
                           tables=[torch.from_numpy(np.ascontiguousarray(w.block_tables[c])).to(dev)
                                   for c in range(w.copies)]))
        tables.append(None)
    torch.cuda.synchronize()
    return caches, copies


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(decode shards by sequence or KV head with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_430_amd as pkv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    pkv.load()
    layers, copies = make_decode_setup(args.workload, dev)
    w0 = layers[0]["w"]
    B, hq, hkv, dh = w0.batch, w0.hq, w0.hkv, w0.head_dim
    T = int(w0.seq_lens.max())
    fp8 = w0.cache_dtype == "fp8"
    kv_elt = 1 if fp8 else 2
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    lens = torch.from_numpy(w0.seq_lens.astype(np.int32)).to(dev)
    cu_new = torch.arange(B + 1, dtype=torch.int32, device=dev)
    first_pos = (lens - 1).contiguous()
    slots = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty(B, hq, dh, dtype=torch.float32, device=dev)
    pt = args.partition
    ws = pkv.decode_workspace(B, hq, hkv, dh, T, pt, dev)
    lib = pkv.load()
    wsp = ws.data_ptr() if ws is not None else None
    wsb = ws.numel() if ws is not None else 0

    def step(i, ev=None):
        c = i % copies
        for L in layers:
            tb = L["tables"][c]
            pkv._check(lib.pkv_slot_mapping_device(tb.data_ptr(), tb.shape[1], 16, B, cu_new.data_ptr(),
                                                   first_pos.data_ptr(), B, slots.data_ptr(), sh))
            pkv._check(lib.pkv_kv_append(L["cache"].ref(), L["k_new"].data_ptr(), L["v_new"].data_ptr(),
                                         pkv.PKV_BF16, B, slots.data_ptr(),
                                         L["kinv"].data_ptr() if fp8 else None,
                                         L["vinv"].data_ptr() if fp8 else None, sh))
            if ev is not None:
                ev[0].record(stream)
            pkv._check(lib.pkv_attn_decode(L["cache"].ref(), L["w"].q.data_ptr(), pkv.PKV_BF16, B, hq,
                                           tb.data_ptr(), tb.shape[1], lens.data_ptr(), T, L["w"].scale, pt,
                                           out.data_ptr(), wsp, wsb, sh))
            if ev is not None:
                ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n_dec = args.steps * len(layers)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dec)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    k = 0
    for i in range(args.steps):
        c = i % copies
        for L in layers:
            # per-layer events around the decode launch only
            tb = L["tables"][c]
            pkv._check(lib.pkv_slot_mapping_device(tb.data_ptr(), tb.shape[1], 16, B, cu_new.data_ptr(),
                                                   first_pos.data_ptr(), B, slots.data_ptr(), sh))
            pkv._check(lib.pkv_kv_append(L["cache"].ref(), L["k_new"].data_ptr(), L["v_new"].data_ptr(),
                                         pkv.PKV_BF16, B, slots.data_ptr(),
                                         L["kinv"].data_ptr() if fp8 else None,
                                         L["vinv"].data_ptr() if fp8 else None, sh))
            evs[k][0].record(stream)
            pkv._check(lib.pkv_attn_decode(L["cache"].ref(), L["w"].q.data_ptr(), pkv.PKV_BF16, B, hq,
                                           tb.data_ptr(), tb.shape[1], lens.data_ptr(), T, L["w"].scale, pt,
                                           out.data_ptr(), wsp, wsb, sh))
            evs[k][1].record(stream)
            k += 1
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    ms_step = total_ms / args.steps
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    dec_sorted = sorted(dec_ms)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2 ** 20 // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    d_bytes = decode_bytes(w0.seq_lens, hq, hkv, dh, kv_elt, 2, fp8)
    a_bytes = append_bytes(B, hkv, dh, 2, kv_elt) + B * 4 * 3
    step_bytes = (d_bytes + a_bytes) * len(layers)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = d_bytes / (dec_avg_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash(DECODE_SOURCES) and tr.get("workload") == args.workload:
            traffic = tr.get("bytes_per_launch")

    line = {
        "metric": METRIC if args.workload == "cfg2-all4096" else f"decode-attn KV HBM GB/s ({args.workload})",
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
                   "seq_len": T, "block_size": 16, "layers": len(layers), "pool_copies": copies,
                   "partition_tokens": pt or pkv.pkv_attn_decode_auto_partition(B, hq, hkv, T)},
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "new_tokens_per_s": round(B / (ms_step * 1e-3) if len(layers) == 1 else B / (ms_step * 1e-3), 1),
        "kv_tokens_per_s": round(float(w0.seq_lens.sum()) * len(layers) / (ms_step * 1e-3), 1),
        "decode_kernel_us": {"mean": round(dec_avg_ms * 1e3, 2), "p10": round(dec_sorted[len(dec_sorted) // 10] * 1e3, 2),
                             "p50": round(dec_sorted[len(dec_sorted) // 2] * 1e3, 2),
                             "p90": round(dec_sorted[(9 * len(dec_sorted)) // 10] * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "decode_split_kernel", "bytes_per_launch": d_bytes},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w0, args.cpu_seconds, d_bytes)
    print(json.dumps(line), flush=True)


def cpu_baseline(w, target_s, d_bytes):
    """The float64 oracle on this host's cores, over the first layer's batch:
    whole batches are repeated until target_s of compute has elapsed."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    cores = len(os.sched_getaffinity(0))
    q = w.q.float().cpu().double().numpy()
    ks, vs = [], []
    nseq = w.batch
    for b in range(nseq):
        k = w.seq_k(b).float().cpu().double().numpy().transpose(1, 0, 2).copy()
        v = w.seq_v(b).float().cpu().double().numpy().transpose(1, 0, 2).copy()
        if w.cache_dtype == "fp8":
            from oracle import fp8 as ofp8
            kb = w.seq_k(b).contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)
            vb = w.seq_v(b).contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)
            k = np.stack([ofp8.dequantize(ofp8.quantize_bf16_bits(kb[:, h], w.k_inv_scale[h]), w.k_scale[h])
                          for h in range(w.hkv)])
            v = np.stack([ofp8.dequantize(ofp8.quantize_bf16_bits(vb[:, h], w.v_inv_scale[h]), w.v_scale[h])
                          for h in range(w.hkv)])
        ks.append(k)
        vs.append(v)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.attention.decode(q, ks, vs, w.scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    per_batch = el / reps
    return {"value": round(d_bytes / per_batch / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "cores_available": cores, "kind": "oracle",
            "sample": f"whole batch ({nseq} sequences, float64 numpy, materialised softmax), "
                      f"{reps} repetitions in {el:.1f} s; {per_batch * 1e3:.1f} ms per batch"}


if __name__ == "__main__":
    main()
