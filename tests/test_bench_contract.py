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
