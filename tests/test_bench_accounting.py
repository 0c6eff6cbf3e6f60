"""The benchmark's own arithmetic, on the CPU: the byte and flop counts behind `value` and `roofline`
against brute-force counts on small workloads, and the single-GPU contract of the command line."""
import os
import subprocess
import sys

import numpy as np

import bench
from paged_kv_cache_199_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _brute_kv_bytes(w):
    """K+V bytes with every (physical block, slot) that some sequence attends counted once."""
    e = 1 if w.kv_fp8 else (4 if w.spec.dtype == "f32" else 2)
    seen = set()
    for s in range(w.num_seqs):
        for t in range(int(w.context_lens[s])):
            seen.add((int(w.block_tables[s, t // 16]), t % 16))
    return len(seen) * w.spec.num_kv_heads * w.spec.head_dim * 2 * e


def test_algorithmic_bytes_count_shared_pages_once():
    spec = W.custom("acct", [5, 40, 33, 64], q_len=[1, 2, 1, 3], num_heads=8, num_kv_heads=2, head_dim=64,
                    shared_prefix_blocks=2)
    w = W.build(spec, "cpu")
    B, H, D = 16, 8, 64
    kv = _brute_kv_bytes(w)
    qo = w.total_q * H * D * 2 * 2 + w.total_q * H * 4
    meta = sum((int(c) + B - 1) // B for c in w.context_lens) * 4 + w.num_seqs * 8
    assert bench.algorithmic_bytes(w) == kv + qo + meta
    assert bench.logical_kv_bytes(w) == int(w.context_lens.sum()) * 2 * D * 2 * 2 > kv


def test_write_bytes_and_fp8_element_size():
    w = W.build(W.custom("acct8", [17, 3], num_heads=4, num_kv_heads=2, head_dim=64, kv_fp8=True,
                         write_new_token=True), "cpu")
    # the new rows are read as bf16 (2 bytes) and written as codes (1 byte), plus their slots
    assert bench.write_bytes(w) == 2 * 2 * 64 * (2 + 1) * 2 + 2 * 8
    assert bench.algorithmic_bytes(w) - bench.algorithmic_bytes(W.build(W.custom(
        "acct16", [17, 3], num_heads=4, num_kv_heads=2, head_dim=64), "cpu")) == -_brute_kv_bytes(w)


def test_prefill_flops_is_the_sum_over_visible_pairs():
    spec = W.custom("pf", [7, 40, 300], q_len=[7, 16, 100], num_heads=4, num_kv_heads=2, head_dim=32)
    w = W.build(spec, "cpu")
    pairs = 0
    for s in range(w.num_seqs):
        n, q = int(w.context_lens[s]), int(w.q_lens[s])
        for i in range(q):
            pairs += n - q + i + 1             # keys 0 .. n - q + i
    assert bench.prefill_flops(w) == pairs * 4 * 4 * 32


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_probe_page_lists_cover_every_page_once():
    """The page-stream probe's per-wave lists (the decode schedule's order) hold every (page, kv head,
    row tile) a decode reads exactly once, with and without the per-item start cost and with a cut
    alignment, for batches whose items are longer and shorter than a wave's share."""
    spec = W.custom("order", [1, 17, 300, 1100, 2048, 5, 33], q_len=[1, 2, 5, 1, 3, 1, 1], num_heads=8,
                    num_kv_heads=2, head_dim=64)
    w = W.build(spec, "cpu")
    KVH, G = 2, 4
    for rpt in (16, 32):
        want = []
        for kvh in range(KVH):
            for s in range(w.num_seqs):
                nblk = (int(w.context_lens[s]) + 15) // 16
                rts = -(-int(w.q_lens[s]) * G // rpt)
                want += [int(b) * KVH + kvh for b in w.block_tables[s, :nblk]] * rts
        for waves in (64, 1024):
            for cost in (0, 4):
                for align in (1, 2):
                    lists = bench.decode_order_pages(w, rpt, waves, align, cost)
                    assert len(lists) == waves
                    got = np.sort(np.concatenate(lists))
                    assert np.array_equal(got, np.sort(np.asarray(want, np.int64)))


def test_cpu_baseline_uses_every_core_and_names_the_cpu():
    """The oracle baseline runs one worker process per core of the affinity set and records the CPU
    model; its bytes count the same numerator as the GPU figure."""
    import os

    import bench

    w = W.build(W.custom("cpu_base", [17, 300, 64], num_heads=8, num_kv_heads=2, head_dim=64), "cpu")
    r = bench.cpu_baseline(w, 0.5)
    assert r["cores"] == len(os.sched_getaffinity(0)) and r["kind"] == "oracle"
    assert r["cpu_model"] and r["value"] > 0 and "worker processes" in r["sample"]
