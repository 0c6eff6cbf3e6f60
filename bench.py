"""Benchmark: one step = the whole decode hot path on one batch: the slot-mapped append of each
sequence's new K/V row (when the workload has one) plus paged decode attention with its split-K
combine, all through the C ABI.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--partition-size P]

Prints ONE JSON line.  With no --workload it is the long-context configuration (256 sequences,
lognormal contexts up to 32768 tokens, 64 query / 8 kv heads): the largest that fits one GPU.  Its
fixed 512-key-partition variant rides along under "variants", and the concurrency-32 step (with its
slot_mapping-write variant) under "secondary".  `value` is whole-step throughput in GB/s of algorithmic
bytes (every attended K/V row once, Q, the output, the LSE, the block ids and lengths, plus the
appended rows), with every input resident in HBM before the clock starts.  The K/V pool is cloned into
enough copies (>= 1 GiB in total) that consecutive steps never hit the 256 MB Infinity Cache; step i
uses copy i mod R.  `roofline` reports the partition kernel alone, timed by HIP events the library
records around it on the launch stream.  `cpu_baseline` times the float64 oracle on every host core
on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hip_runtime_api.h
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic_bytes(w) -> int:
    """Bytes the decode must move at least once (split-K partials excluded: they are overhead)."""
    e = 4 if w.spec.dtype == "f32" else 2
    ekv = 1 if w.kv_fp8 else e                       # E4M3 pools: one byte per element
    KVH, D, B = w.spec.num_kv_heads, w.spec.head_dim, w.spec.block_size
    rows_by_block = {}
    for s in range(w.num_seqs):
        n = int(w.context_lens[s])
        for j in range((n + B - 1) // B):
            blk = int(w.block_tables[s, j])
            rows_by_block[blk] = max(rows_by_block.get(blk, 0), min(B, n - j * B))
    kv_tokens = sum(rows_by_block.values())          # shared pages count once
    kv = kv_tokens * KVH * D * 2 * ekv
    qo = w.total_q * w.spec.num_heads * D * e * 2 + w.total_q * w.spec.num_heads * 4
    meta = int(((w.context_lens.astype(np.int64) + B - 1) // B).sum()) * 4 + w.num_seqs * 8
    return int(kv + qo + meta)


def logical_kv_bytes(w) -> int:
    """K/V bytes when every sequence reads its own pages (shared pages counted once per reader)."""
    ekv = 1 if w.kv_fp8 else (4 if w.spec.dtype == "f32" else 2)
    return int(w.context_lens.astype(np.int64).sum()) * w.spec.num_kv_heads * w.spec.head_dim * 2 * ekv


def write_bytes(w) -> int:
    if w.slot_mapping is None:
        return 0
    e = 4 if w.spec.dtype == "f32" else 2
    ekv = 1 if w.kv_fp8 else e
    rows = int(w.slot_mapping.shape[0])
    return rows * w.spec.num_kv_heads * w.spec.head_dim * (e + ekv) * 2 + rows * 8


# the sources the decode partition kernels are built from (the kernel the traffic record measures)
DECODE_SOURCES = ("decode_mfma.hip", "decode_valu.hip", "mfma_wave.h", "decode_args.h", "device_common.h", "e4m3.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_199_amd", "csrc")
    for f in DECODE_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, path: str, schedule: str, part_size: int, depth: int, grid_waves: int):
    """HBM bytes per launch of the partition kernel from committed rocprofv3 counter runs, or None when
    the kernels or the launch configuration changed since they were taken."""
    f = os.path.join(PROFILES, f"traffic_{path}_{schedule}_{workload}.json")
    if not os.path.exists(f):
        return None
    d = json.load(open(f))
    if d.get("source_hash") != kernel_source_hash():
        return None
    if d.get("partition_size") != part_size or d.get("pipeline_depth") != depth:
        return None
    if d.get("grid_waves") != grid_waves:
        return None
    return d.get("bytes_per_launch")


def decode_order_pages(w, rows_per_tile: int, waves: int, cut_align: int, item_cost: int = 0):
    """Per-wave K/V page lists in the order the persistent decode schedule visits them: the stream of
    work items (kv head, sequence, row tile) kv-head-major, each item_cost virtual pages followed by
    its logical pages, cut into NW equal shares (share x * W + wx goes to wave wx of XCD x; workgroup
    i runs on XCD i % 8).  A boundary on an item's virtual pages moves to the item's start; one on its
    real pages moves down to a multiple of cut_align pages from the first of them.  Virtual pages
    are dropped from the lists."""
    KVH, B = w.spec.num_kv_heads, w.spec.block_size
    G = w.spec.num_heads // KVH
    parts, starts = [], []
    pos = 0
    for kvh in range(KVH):
        for s in range(w.num_seqs):
            nblk = (int(w.context_lens[s]) + B - 1) // B
            if nblk == 0:
                continue
            row_ids = w.block_tables[s, :nblk].astype(np.int64) * KVH + kvh
            rts = -(-int(w.q_lens[s]) * G // rows_per_tile)
            for _ in range(rts):
                parts.append(np.full(item_cost, -1, np.int64))
                parts.append(row_ids)
                starts.append(pos)
                pos += item_cost + nblk
    stream = np.concatenate(parts)
    starts = np.asarray(starts, np.int64)
    L = len(stream)
    W = waves // 8

    def raw(o):
        return L * o // (8 * W)

    def cut(b):
        if b >= L:
            return L
        st = starts[np.searchsorted(starts, b, side="right") - 1]
        ro = b - st - item_cost
        rr = ro - ro % cut_align if ro > 0 else 0
        return st + (item_cost + rr if rr > 0 else 0)

    lists = [np.zeros(0, np.int64)] * waves
    for o in range(8 * W):
        a, b = cut(raw(o)), cut(raw(o + 1))
        x, wx = divmod(o, W)
        seg = stream[a:b]
        lists[((wx // 4) * 8 + x) * 4 + wx % 4] = seg[seg >= 0]
    return lists


PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_199_amd", "libpkv_probe.so")
_probe = None


def probe_lib():
    """libpkv_probe.so (include/pkv_probe.h), the page-stream probe built beside libpkv.so."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"{PROBE_LIB} is missing: build it with `python -m paged_kv_cache_199_amd.build`")
        lib = ctypes.CDLL(PROBE_LIB)
        vp = ctypes.c_void_p
        lib.pkv_probe_page_stream.restype = ctypes.c_int
        lib.pkv_probe_page_stream.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int,
                                              vp, vp]
        _probe = lib
    return _probe


def probe_page_stream(k_cache, v_cache, page_index, wave_offsets, sink, stream=None) -> None:
    """Stream the listed K/V pages with the decode kernel's load shapes and no arithmetic.
    page_index / wave_offsets: int32 on the GPU."""
    import torch

    nb, kvh, B, D = k_cache.shape
    if not (page_index.dtype == torch.int32 and wave_offsets.dtype == torch.int32):
        raise ValueError("int32 lists")
    if not (k_cache.dtype in (torch.bfloat16, torch.uint8) and v_cache.dtype == k_cache.dtype
            and v_cache.numel() == k_cache.numel() and B == 16):
        raise ValueError("bf16 or uint8 (E4M3) pools of one shape")
    for t in (k_cache, v_cache, page_index, wave_offsets, sink):
        if not (t.is_cuda and t.device == k_cache.device and t.is_contiguous()):
            raise ValueError("contiguous tensors on the pools' GPU")
    s = torch.cuda.current_stream() if stream is None else stream
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = probe_lib().pkv_probe_page_stream(p(k_cache), p(v_cache), nb * kvh, D, k_cache.element_size(), p(page_index),
                                           p(wave_offsets), wave_offsets.numel() - 1, p(sink),
                                           ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"pkv_probe_page_stream failed (status {rc})")


def pattern_ceiling(w, plan, kcs, vcs, reps: int = 3):
    """Time the page-stream probe (same loads as the decode kernel, no arithmetic) on this workload's
    pages in the decode schedule's order, rotating over the same pool copies as the timed steps.
    Returns (seconds per launch, pages streamed)."""
    import torch

    from paged_kv_cache_199_amd import _lib

    cut_align = plan["pipeline_depth"] if plan["num_partitions"] > 1 else 1
    lists = decode_order_pages(w, plan["rows_per_tile"], plan["grid_waves"], cut_align, plan["item_cost"])
    offs = np.zeros(len(lists) + 1, np.int64)
    offs[1:] = np.cumsum([len(l) for l in lists])
    dev = kcs[0].device
    flat = torch.from_numpy(np.concatenate(lists).astype(np.int32)).to(dev)
    off_t = torch.from_numpy(offs.astype(np.int32)).to(dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    R = len(kcs)
    for r in range(R):
        probe_page_stream(kcs[r], vcs[r], flat, off_t, sink)
    torch.cuda.synchronize()
    n = reps * R
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        probe_page_stream(kcs[i % R], vcs[i % R], flat, off_t, sink)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / n, int(offs[-1])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Host bytes of K/V pages the CPU baseline copies out for its sample of sequences (it cycles over them).
CPU_SAMPLE_BYTES = 1 << 30


def _oracle_worker(job):
    """One host core's share of the CPU baseline (runs in a spawned process): the oracle, unchanged, on
    whole sequences of the sample (cycling from this worker's offset) until the shared deadline, with
    one BLAS thread.  Returns (units, tokens, calls): units are bytes ("bytes") or matrix flops
    ("flops") by the GPU figure's own numerator."""
    root, files, p, start, deadline = job
    if root not in sys.path:
        sys.path.insert(0, root)
    from threadpoolctl import threadpool_limits

    from oracle import fp8 as F8
    from oracle import paged_attention as O

    a = {k: np.load(f, mmap_mode="r") for k, f in files.items()}
    q, kc, vc, table, ctx, ql = a["q"], a["kc"], a["vc"], a["table"], a["ctx"], a["ql"]
    S, B, KVH, H, D = len(ctx), p["block"], p["kvh"], p["heads"], p["dim"]
    units = tokens = calls = 0
    i = start
    with threadpool_limits(limits=1):
        while time.time() < deadline:
            s = i % S
            i += 1
            n, qs = int(ctx[s]), int(ql[s])
            if p["fp8"]:
                ids = np.asarray(table[s, :(n + B - 1) // B], dtype=np.int64)
                kd, vd = F8.dequantize(kc[ids], p["k_scale"]), F8.dequantize(vc[ids], p["v_scale"])
                t1 = np.full_like(np.asarray(table), -1)
                t1[s, :ids.shape[0]] = np.arange(ids.shape[0])
                O.paged_decode_attention(q, kd, vd, t1, ctx, ql, p["scale"], KVH, B, seqs=[s])
            else:
                O.paged_decode_attention(q, kc, vc, table, ctx, ql, p["scale"], KVH, B, seqs=[s])
            if p["count"] == "flops":
                units += (qs * (n - qs) + qs * (qs + 1) // 2) * H * 4 * D
            else:
                units += n * KVH * D * 2 * p["ekv"] + qs * H * (D * p["e"] * 2 + 4) + ((n + B - 1) // B) * 4 + 8
            tokens += n
            calls += 1
    return units, tokens, calls


def oracle_on_all_cores(w, budget_s: float, count: str = "bytes"):
    """The oracle on every core this process may use (os.sched_getaffinity), one spawned worker process
    per core with one BLAS thread each (so BLAS runs as many threads as there are cores), for about
    budget_s of wall time.  The sample: the workload's first sequences whose pages fit CPU_SAMPLE_BYTES
    (all of them when they fit), copied to memory-mapped files the workers share, with the block tables
    renumbered to the copied pages.  Returns (units, tokens, calls, cores, wall seconds, sequences)."""
    import multiprocessing as mp
    import shutil
    import tempfile

    import torch

    def bits(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    B = w.spec.block_size
    nblk = (w.context_lens.astype(np.int64) + B - 1) // B
    page_bytes = w.spec.num_kv_heads * B * w.spec.head_dim * 2 * w.k_cache.element_size()
    n_seq = int(max(1, min(w.num_seqs, np.searchsorted(np.cumsum(nblk) * page_bytes, CPU_SAMPLE_BYTES,
                                                          side="right"))))
    ids = np.concatenate([w.block_tables[s, :nblk[s]] for s in range(n_seq)]).astype(np.int64)
    uniq = np.unique(ids)
    remap = np.full(w.num_blocks, -1, np.int32)
    remap[uniq] = np.arange(uniq.shape[0], dtype=np.int32)
    table = np.where(w.block_tables[:n_seq] >= 0, remap[np.maximum(w.block_tables[:n_seq], 0)], -1).astype(np.int32)
    sel = torch.from_numpy(uniq).to(w.k_cache.device)
    q_rows = int(w.q_lens[:n_seq].sum())
    arrays = {"q": bits(w.q[:q_rows]), "kc": bits(w.k_cache.index_select(0, sel)),
              "vc": bits(w.v_cache.index_select(0, sel)), "table": table,
              "ctx": w.context_lens[:n_seq].copy(), "ql": w.q_lens[:n_seq].copy()}
    need = sum(x.nbytes for x in arrays.values())
    base = "/dev/shm" if os.path.isdir("/dev/shm") and shutil.disk_usage("/dev/shm").free > 2 * need else None
    tmp = tempfile.mkdtemp(prefix="pkv_cpu_", dir=base)
    try:
        files = {}
        for k, x in arrays.items():
            files[k] = os.path.join(tmp, k + ".npy")
            np.save(files[k], x)
        del arrays
        e = 4 if w.spec.dtype == "f32" else 2
        p = {"block": B, "kvh": w.spec.num_kv_heads, "heads": w.spec.num_heads, "dim": w.spec.head_dim,
             "scale": w.scale, "fp8": w.kv_fp8, "k_scale": w.spec.k_scale, "v_scale": w.spec.v_scale,
             "e": e, "ekv": 1 if w.kv_fp8 else e, "count": count}
        cores = len(os.sched_getaffinity(0))
        ctx = mp.get_context("spawn")
        with ctx.Pool(cores) as pool:
            # start every worker and load its imports before the clock starts
            pool.map(_oracle_worker, [(ROOT, files, p, 0, 0.0)] * cores, chunksize=1)
            t0 = time.time()
            jobs = [(ROOT, files, p, k * n_seq // cores, t0 + budget_s) for k in range(cores)]
            parts = pool.map(_oracle_worker, jobs, chunksize=1)
            wall = time.time() - t0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return (sum(x[0] for x in parts), sum(x[1] for x in parts), sum(x[2] for x in parts), cores, wall, n_seq)


def cpu_baseline(w, budget_s: float):
    """The oracle as it is, on whole sequences of the workload (cycling over a sample of them), on every
    core of the host, for about budget_s of wall time.  Same numerator as the GPU figure: each
    sequence's K/V bytes, its q/out/lse rows, page ids and lengths."""
    nbytes, tokens, calls, cores, wall, n_seq = oracle_on_all_cores(w, budget_s)
    return {
        "value": round(nbytes / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{calls} sequence decodes cycling over the first {n_seq} of the workload's {w.num_seqs} "
                  f"sequences ({tokens} context tokens, all heads), numpy float64, {cores} worker processes "
                  f"with one BLAS thread each, {wall:.1f} s wall",
        "attended_tokens_per_s": round(tokens / wall, 1),
    }


def bench_blocks(args, dev):
    """The block manager: copy-on-write block copies on the GPU (GB/s against HBM peak) and the host
    bookkeeping of a decode step (slots for one new token per sequence), with the oracle's model of
    the same bookkeeping as the CPU baseline."""
    import torch

    from paged_kv_cache_199_amd import blocks as BM

    NB, KVH, D, n = 8192, 8, 128, 2048          # bf16 pools of 512 MiB each; 2048 copies per launch
    kc = torch.randn((NB, KVH, 16, D), device=dev).to(torch.bfloat16)
    vc = torch.randn((NB, KVH, D, 16), device=dev).to(torch.bfloat16)
    perm = np.random.default_rng(0).permutation(NB).astype(np.int32)
    src, dst = torch.from_numpy(perm[:n]).to(dev), torch.from_numpy(perm[n:2 * n]).to(dev)
    block_bytes = KVH * 16 * D * 2
    moved = 2 * 2 * n * block_bytes              # both pools, read + write
    for _ in range(args.warmup):
        BM.copy_blocks(kc, vc, src, dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        BM.copy_blocks(kc, vc, src, dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = moved / (ms * 1e-3) / 1e9

    # host: 256 sequences of 1000 tokens, each forked once (shared partial last block), then decode
    # steps of one token per sequence on all 512
    def host_steps(n_steps):
        pool = BM.BlockPool(1 << 16)
        seqs = []
        for _ in range(256):
            s = BM.Sequence(pool)
            s.append(1000)
            seqs += [s, s.fork()]
        t0 = time.perf_counter()
        copies = 0
        for _ in range(n_steps):
            copies += len(BM.append_step(seqs, 1)[1])   # the step's slot_mapping in one call
        dt = time.perf_counter() - t0
        pool.close()
        return len(seqs) * n_steps / dt, copies

    host_rate, copies = host_steps(200)
    res = {
        "metric": "copy-on-write block copies GB/s (% of HBM peak) + host slot allocations/s, 1 GPU",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) pools, permuted block ids)",
        "config": {"workload": "blocks_cow", "num_blocks": NB, "num_kv_heads": KVH, "head_dim": D,
                   "copies_per_launch": n, "host_sequences": 512, "host_context": 1000},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "copy_blocks_kernel",
                     "kernel_ms": round(ms, 5), "algorithmic_bytes_per_launch": moved},
        "host_slot_allocations_per_s": round(host_rate, 1),
        "host_copy_on_write_pairs": copies,
    }
    if args.cpu_budget > 0:
        from oracle.block_manager import BlockModel

        m = BlockModel(1 << 12)
        for k in range(64):                      # sequence k owns blocks k*64 .. k*64+63
            m.new_seq(k)
            m.append(k, 1000, [k * 64 + j for j in range(63)])
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < min(args.cpu_budget, 10.0) and done < 64 * 24:
            k = done % 64
            fresh, _ = m.append_needs(k, 1)
            m.append(k, 1, m.tables[k] + ([k * 64 + 63] if fresh else []))
            done += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(done / dt, 1), "unit": "slot allocations/s", "cores": 1,
                               "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"{done} one-token appends on 64 sequences of 1000+ tokens through the "
                                         f"oracle's reference model of the block manager, {dt:.1f} s"}
    print(json.dumps(res), flush=True)


def prefill_flops(w) -> int:
    """Matrix products of the attention: 2 D flops for q.k and 2 D for p.v per (query row, head,
    visible key); row i of a q-token chunk sees ctx - q + i + 1 keys."""
    ctx = w.context_lens.astype(np.int64)
    q = w.q_lens.astype(np.int64)
    pairs = int((q * (ctx - q) + q * (q + 1) // 2).sum())
    return pairs * w.spec.num_heads * 4 * w.spec.head_dim


def bench_prefill(args, dev, spec):
    """Chunked prefill: pkv_paged_attn_prefill over the workload's chunks, timed as a HIP graph of K
    steps; the roofline is the matrix cores' dense bf16 peak."""
    import torch

    from paged_kv_cache_199_amd import _lib
    from paged_kv_cache_199_amd import workloads as W

    w = W.build(spec, dev)
    meta = w.device_meta(dev)
    H, KVH, D = spec.num_heads, spec.num_kv_heads, spec.head_dim
    out = torch.empty_like(w.q)
    lse = torch.empty((w.total_q, H), dtype=torch.float32, device=dev)
    q_lens = None if w.uniform_q else meta["q_lens"]

    scales = dict(k_scale=spec.k_scale, v_scale=spec.v_scale) if spec.kv_fp8 else {}

    def step():
        _lib.paged_attn_prefill(w.q, w.k_cache, w.v_cache, meta["block_tables"], meta["context_lens"], q_lens, out,
                                lse, H, KVH, D, spec.block_size, w.scale, w.max_context_len, w.max_q_len, **scales)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(args.steps):
            step()
    g.replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / args.steps
    flops = prefill_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    kv = algorithmic_bytes(w)
    res = {
        "metric": "paged prefill attention TFLOP/s (% of bf16 MFMA peak) + new tokens/s, 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) Q/K/V, shuffled 16-token pages)",
        "config": {"workload": spec.name, "num_seqs": w.num_seqs, "num_heads": H, "num_kv_heads": KVH,
                   "head_dim": D, "block_size": spec.block_size, "kv_cache": "e4m3" if spec.kv_fp8 else "bf16",
                   "new_tokens": int(w.q_lens.sum()),
                   "context_tokens": int(w.context_lens.astype(np.int64).sum()),
                   "max_context_len": w.max_context_len},
        "new_tokens_per_s": round(int(w.q_lens.sum()) / (ms * 1e-3), 1),
        "kv_bytes_per_step": kv,
        "eager_ms_per_step": round(eager_ms, 5),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_mfma_kernel", "kernel_ms": round(ms, 5), "flops_per_launch": flops},
    }
    if args.cpu_budget > 0:
        done, _, n, cores, wall, n_seq = oracle_on_all_cores(w, min(args.cpu_budget, 20.0), count="flops")
        res["cpu_baseline"] = {"value": round(done / wall / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
                               "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"{n} whole sequences cycling over the first {n_seq} of the workload "
                                         f"(all heads), numpy float64, {cores} worker processes with one BLAS "
                                         f"thread each, {wall:.1f} s wall"}
    print(json.dumps(res), flush=True)


def measure_decode(args, dev, spec, w=None, **override):
    """One decode workload timed as the bench line describes (graph replay of K steps, HIP events around
    the partition kernel, pattern ceiling).  `override` replaces command-line options for this run (e.g.
    partition_size, append, no_ceiling).  The built workload comes back under "_workload"."""
    import torch

    from paged_kv_cache_199_amd import _lib
    from paged_kv_cache_199_amd import workloads as W

    args = argparse.Namespace(**{**vars(args), **override})
    P = spec.partition_size if args.partition_size < 0 else args.partition_size
    path = {"auto": _lib.PATH_AUTO, "valu": _lib.PATH_VALU, "mfma": _lib.PATH_MFMA}[args.path]
    if w is None:
        w = W.build(spec, dev)
    meta = w.device_meta(dev)
    H, KVH, D = spec.num_heads, spec.num_kv_heads, spec.head_dim
    pool_bytes = w.k_cache.numel() * w.k_cache.element_size() * 2
    R = max(1, math.ceil(args.min_pool_bytes / pool_bytes))
    kcs = [w.k_cache] + [w.k_cache.clone() for _ in range(R - 1)]
    vcs = [w.v_cache] + [w.v_cache.clone() for _ in range(R - 1)]
    out = torch.empty_like(w.q)
    lse = torch.empty((w.total_q, H), dtype=torch.float32, device=dev)
    code = (_lib.PKV_BF16_FP8KV if spec.kv_fp8 else _lib.PKV_BF16) if spec.dtype == "bf16" else _lib.PKV_F32
    sched = {"auto": 0, "grid": 1, "persistent": 2}[args.schedule]
    plan = _lib.decode_plan(w.num_seqs, w.total_q, w.max_q_len, w.max_context_len, H, KVH, D, code, P, path,
                            args.depth, sched, args.wgs_per_cu)
    P_used = plan["partition_size"]
    kernel = "decode_valu_kernel"
    if plan["path"] == _lib.PATH_MFMA:
        kernel = "decode_mfma_persistent_kernel" if plan["schedule"] == 2 else "decode_mfma_kernel"
    ws_bytes = plan["workspace_bytes"]
    ws = _lib.new_workspace(ws_bytes, dev)
    q_lens = None if w.uniform_q else meta["q_lens"]
    stream = torch.cuda.current_stream()
    total = args.warmup + args.steps
    # Timing events around the partition kernel, recorded by the library on its stream.  They skip
    # the system-scope cache writeback / invalidate a default event performs when it is recorded,
    # which would otherwise add several microseconds of idle GPU next to the kernel being timed.
    hip = ctypes.CDLL("libamdhip64.so.7")     # the HIP runtime torch already loaded

    def new_event():
        e = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def elapsed_ms(a, b):
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    ev = [(new_event(), new_event()) for _ in range(args.steps)]

    append_mode = args.append
    dstep = _lib.DecodeStep(w.q, kcs[0], vcs[0], meta["block_tables"], meta["context_lens"], q_lens, out, lse,
                            H, KVH, D, spec.block_size, w.scale, w.max_context_len, max_q_len=w.max_q_len,
                            partition_size=P, path=path, depth=args.depth, schedule=sched, workspace=ws,
                            new_k=w.new_k, new_v=w.new_v,
                            slot_mapping=meta["slot_mapping"] if w.slot_mapping is not None and append_mode == "slots"
                            else None, wgs_per_cu=args.wgs_per_cu,
                            k_scale=spec.k_scale if spec.kv_fp8 else 0.0, v_scale=spec.v_scale if spec.kv_fp8 else 0.0)

    def step(i, events=None):
        r = i % R
        dstep(kcs[r], vcs[r], events=events)

    prefix_call = spec.shared_prefix_blocks > 0 and args.prefix_mode != "off"
    prefix_mode = {"auto": _lib.PREFIX_AUTO, "once": _lib.PREFIX_READ_ONCE,
                   "per-seq": _lib.PREFIX_PER_SEQUENCE, "off": None}[args.prefix_mode]
    if prefix_call:
        # shared-prefix decode: all sequences form one group over their shared prefix blocks
        if w.slot_mapping is not None:
            raise SystemExit("shared-prefix workloads append nothing")
        pre_tokens = spec.shared_prefix_blocks * spec.block_size
        gs, pl, pb = W.share_prefixes(w, [(0, w.num_seqs, pre_tokens)])
        meta = w.device_meta(dev)
        gdev = [torch.from_numpy(a).to(dev) for a in (gs, pl, pb)]
        pws = _lib.new_workspace(_lib.shared_prefix_workspace_bytes(
            w.num_seqs, w.total_q, w.max_q_len, w.max_context_len, H, KVH, D, code, 1, w.num_seqs, pre_tokens,
            partition_size=P, depth=args.depth, schedule=sched, wgs_per_cu=args.wgs_per_cu), dev)

        def step(i, events=None):
            r = i % R
            _lib.paged_attn_decode_shared_prefix(
                w.q, kcs[r], vcs[r], meta["block_tables"], meta["context_lens"], q_lens, out, lse, H, KVH, D,
                spec.block_size, w.scale, w.max_context_len, gdev[0], gdev[1], gdev[2], w.num_seqs, pre_tokens,
                max_q_len=w.max_q_len, partition_size=P, workspace=pws, events=None, depth=args.depth,
                schedule=sched, wgs_per_cu=args.wgs_per_cu, mode=prefix_mode)

    # eager: every step is two C calls from Python; HIP events around the partition kernel
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, ev[i])
    t_end.record(stream)
    host_enqueue = time.perf_counter() - wall0
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    eager_ms_step = t_start.elapsed_time(t_end) / args.steps
    k_ms = None if prefix_call else float(np.mean([elapsed_ms(b, e) for b, e in ev]))
    for b, e in ev:
        hip.hipEventDestroy(b)
        hip.hipEventDestroy(e)
    ms_step = eager_ms_step
    timing = "eager"
    graph_ok = None
    if not args.no_graph:
        # the same K steps captured into one HIP graph and replayed: no host work between steps
        ref_out = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(args.warmup + i)
        graph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        wallg = time.perf_counter()
        g0.record(stream)
        graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        wall += time.perf_counter() - wallg
        ms_step = g0.elapsed_time(g1) / args.steps
        timing = "hip graph replay of the K steps"
        graph_ok = bool(torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                                    ref_out.view(torch.int16) if out.dtype == torch.bfloat16 else ref_out))
        del graph

    dec_bytes = algorithmic_bytes(w)
    step_bytes = dec_bytes + write_bytes(w)
    tokens = int(w.context_lens.astype(np.int64).sum())
    value = step_bytes / (ms_step * 1e-3) / 1e9
    if prefix_call:
        # several kernels share the step (prep, shared-prefix pass, suffix decode and its combine,
        # merge): the roofline line covers the whole step
        kernel, k_ms = "shared-prefix step (pkv_paged_attn_decode_shared_prefix, all kernels)", ms_step
    achieved = dec_bytes / (k_ms * 1e-3) / 1e9
    sched_name = ["", "grid", "persistent"][plan["schedule"]]
    traffic = None if prefix_call else measured_traffic(spec.name, kernel.split("_")[1], sched_name, P_used,
                                                       plan["pipeline_depth"], plan["grid_waves"])
    res = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) + attended tokens/s, 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, shuffled 16-token pages)",
        "config": {
            "workload": spec.name, "num_seqs": w.num_seqs, "num_heads": H, "num_kv_heads": KVH,
            "head_dim": D, "block_size": spec.block_size, "q_len": w.max_q_len,
            "context_tokens": tokens, "max_context_len": w.max_context_len, "partition_size": P_used,
            "path": kernel.split("_")[1], "schedule": sched_name,
            "pipeline_depth": plan["pipeline_depth"], "grid_waves": plan["grid_waves"], "pool_copies": R,
            "appends_new_token": w.slot_mapping is not None,
            "append": (append_mode if w.slot_mapping is not None else None),
            "kv_cache": "e4m3" if spec.kv_fp8 else spec.dtype,
            "shared_prefix_call": prefix_call,
            "prefix_mode": args.prefix_mode if prefix_call else None,
        },
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "attended_tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "algorithmic_bytes_per_step": step_bytes,
        "logical_kv_bytes_per_step": logical_kv_bytes(w),
        "step_timing": timing,
        "eager_ms_per_step": round(eager_ms_step, 5),
        "eager_host_us_per_step": round(host_enqueue / args.steps * 1e6, 2),
        "graph_matches_eager": graph_ok,
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "kernel_ms": round(k_ms, 5),
            "algorithmic_bytes_per_launch": dec_bytes,
        },
    }
    if plan["schedule"] == 2 and not args.no_ceiling and not prefix_call:
        t_probe, pages = pattern_ceiling(w, plan, kcs, vcs)
        ceil = dec_bytes / t_probe / 1e9
        res["roofline"]["pattern_ceiling"] = {
            "value": round(ceil, 2), "unit": "GB/s",
            "what": "this workload's algorithmic bytes over the time the page-stream probe takes to read "
                    f"the same {pages} K+V pages in the decode schedule's order with the decode loads "
                    "and no arithmetic",
        }
        res["roofline"]["frac_of_pattern_ceiling"] = round(achieved / ceil, 4)
    res["_workload"] = w
    return res


# The default line: the largest configuration that fits one GPU (256 sequences, 64 query / 8 kv heads,
# lognormal contexts up to 32768 tokens), with the concurrency-32 step nested beside it.
DEFAULT_WORKLOAD = "long_ctx_splitk_bf16"
SECONDARY_WORKLOAD = "conc32_bf16"


def _summary(r):
    """The figures of one measured run that a variant or nested line carries."""
    ro = r["roofline"]
    out = {"ms_per_step": r["ms_per_step"], "value": r["value"], "unit": r["unit"],
           "frac_of_hbm_peak": r["frac_of_hbm_peak"], "attended_tokens_per_s": r["attended_tokens_per_s"],
           "algorithmic_bytes_per_step": r["algorithmic_bytes_per_step"],
           "partition_size": r["config"]["partition_size"], "append": r["config"]["append"],
           "eager_ms_per_step": r["eager_ms_per_step"],
           "roofline": {k: ro[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                           "kernel_ms", "algorithmic_bytes_per_launch")}}
    for k in ("pattern_ceiling", "frac_of_pattern_ceiling"):
        if k in ro:
            out["roofline"][k] = ro[k]
    return out


def default_line(args, dev):
    """The long-context step (library policy: the balanced split), its variant with fixed 512-key
    partitions (the configuration's own wording), the oracle on the host's cores, and the
    concurrency-32 step (fused append, and the slot_mapping write + decode variant) nested under
    "secondary"."""
    from paged_kv_cache_199_amd import workloads as W

    res = measure_decode(args, dev, W.named(DEFAULT_WORKLOAD))
    w = res.pop("_workload")
    v512 = measure_decode(args, dev, w.spec, w=w, partition_size=512, no_ceiling=True)
    v512.pop("_workload")
    res["variants"] = {"partition_512": {
        "what": "the same step with fixed 512-key partitions merged through their LSE; the default line lets "
                "the balanced persistent schedule cut each sequence where its wave shares end",
        **_summary(v512)}}
    if args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    del w
    conc = measure_decode(args, dev, W.named(SECONDARY_WORKLOAD))
    cw = conc.pop("_workload")
    slots = measure_decode(args, dev, cw.spec, w=cw, append="slots", no_ceiling=True)
    slots.pop("_workload")
    nested = {"workload": SECONDARY_WORKLOAD, "config": conc["config"], **_summary(conc)}
    nested["variants"] = {"slot_mapping_write": {
        "what": "pkv_kv_cache_write of the 32 new tokens through slot_mapping, then pkv_paged_attn_decode "
                "(two calls); the nested line appends inside the decode call (bit-identical result)",
        **_summary(slots)}}
    res["secondary"] = {SECONDARY_WORKLOAD: nested}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="one workload by name; default: the long-context line with conc32 nested")
    ap.add_argument("--partition-size", type=int, default=-1, help="-1: the workload's own, 0: policy")
    ap.add_argument("--path", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--depth", type=int, default=0, help="MFMA register ring depth (0: policy)")
    ap.add_argument("--schedule", default="auto", choices=["auto", "grid", "persistent"])
    ap.add_argument("--wgs-per-cu", type=int, default=0, help="persistent grid: workgroups per CU (0: policy)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work; 0 skips")
    ap.add_argument("--min-pool-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-ceiling", action="store_true", help="skip the page-stream ceiling probe")
    ap.add_argument("--no-graph", action="store_true", help="time the eager step only")
    ap.add_argument("--append", default="fused", choices=["fused", "slots"],
                    help="appending workloads: write the new tokens inside the decode call (fused) or "
                         "with pkv_kv_cache_write through slot_mapping first (slots)")
    ap.add_argument("--prefix-mode", default="auto", choices=["auto", "once", "per-seq", "off"],
                    help="shared-prefix workloads: pkv_paged_attn_decode_shared_prefix with the library's "
                         "policy (auto), forced read-once (once) or per-sequence (per-seq); off: plain "
                         "pkv_paged_attn_decode")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_cache_199_amd import _lib
    from paged_kv_cache_199_amd import workloads as W

    _lib.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        n = 1 << 28
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_each_way": n * 4, "launches": 5}))
        return

    if args.workload == "blocks_cow":
        bench_blocks(args, dev)
        return

    if args.workload is None:
        print(json.dumps(default_line(args, dev)), flush=True)
        return
    spec = W.named(args.workload)
    if spec.prefill:
        bench_prefill(args, dev, spec)
        return
    res = measure_decode(args, dev, spec)
    if args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(res.pop("_workload"), args.cpu_budget)
    res.pop("_workload", None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
