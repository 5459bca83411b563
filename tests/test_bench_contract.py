"""CPU checks of the bench's contract: one GPU only, and algorithmic bytes that
rest on the oracle's KV-byte arithmetic (itself pinned to the pages' tables)."""

import os
import subprocess
import sys

import bench
from oracle import sizing

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_reason():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_headline_decode_bytes_are_the_kv_bytes_plus_the_small_terms():
    """B=32, Hq=32, Hkv=8, Dh=128, T=4096 bf16: the K/V part is the pages'
    2·L·ΣT·Hkv·Dh·bytes at L=1 (512 MiB); q, the fp32 output, one table
    entry per 16-token block and one length per sequence come on top."""
    lens = [4096] * 32
    kv = sizing.kv_bytes_varlen(1, lens, 8, 128, 2)
    assert kv == 536_870_912
    got = bench.decode_bytes(lens, 32, 8, 128, 2, 2, False)
    assert got == kv + 32 * 32 * 128 * 2 + 32 * 32 * 128 * 4 + 32 * 256 * 4 + 32 * 4
    # fp8: one byte per K/V element, plus the two per-head scale arrays
    got8 = bench.decode_bytes(lens, 32, 8, 128, 1, 2, True)
    assert got8 == sizing.kv_bytes_varlen(1, lens, 8, 128, 1) + 32 * 32 * 128 * 6 + 32 * 256 * 4 + 32 * 4 + 64


def test_prefill_flops_count_every_visible_pair():
    """4·Dh·Hq flops per visible (query, key) pair, causal and inclusive: query
    i of a C-token chunk on P cached tokens sees P + i + 1 keys."""
    P, C, hq, dh = 2048, 512, 32, 128
    pairs = sum(P + i + 1 for i in range(C))
    assert pairs == 1_179_904
    assert bench.prefill_flops(P, C, hq, dh) == 4 * dh * hq * pairs == 19_331_547_136


def test_counter_summary_scales_by_the_copy_and_keeps_the_bulk_append(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE per dispatch (KiB) are scaled by what the same
    counter reads for the calibration copy of known size; for the append
    workload only the bulk half of the run's append dispatches counts (the
    step shape runs first, with as many dispatches)."""
    import csv
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    k = "void pkv::kv_append_paged_kernel<1, 1>(...)"
    cal = "void pkv::(anonymous namespace)::copy_blocks_kernel(...)"
    kib = bench.CALIB_BYTES / 1024

    def write(path, counter, rows):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for name, v in rows:
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})

    # the step shape (10 KiB) twice, the bulk shape (1000 KiB) twice, then the copy
    write(tmp_path / "f.csv", "FETCH_SIZE", [(k, 10), (k, 10), (k, 1000), (k, 1000), (cal, kib / 2)])
    write(tmp_path / "w.csv", "WRITE_SIZE", [(k, 20), (k, 20), (k, 3000), (k, 3000), (cal, kib)])
    out = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "append")
    e = out["kernels"]["kv_append_paged_kernel"]
    assert e["dispatches"] == 2
    assert e["fetch_bytes"] == 1000 * 1024 * 2.0         # the copy's reads count half on this counter
    assert e["write_bytes"] == 3000 * 1024 * 1.0
    assert out["bytes_per_launch"] == round(1000 * 1024 * 2 + 3000 * 1024)
    assert (tmp_path / "kv_append_paged_append_traffic.json").exists()
