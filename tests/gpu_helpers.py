"""Shared plumbing for the GPU parity tests and the benchmark: run the library on a workload and run
the oracle on the same tensors (copied to the host).  No attention arithmetic lives here."""
from __future__ import annotations

import numpy as np
import torch

from oracle import fp8 as F8
from oracle import paged_attention as O
from paged_kv_cache_199_amd import _lib
from paged_kv_cache_199_amd.workloads import Workload

BF16_TOL = 1.5e-2
F32_TOL = 2e-3
LSE_TOL = 2e-3


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor: bf16 as uint16 bit patterns, fp32 as float32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def nan_like(t: torch.Tensor) -> torch.Tensor:
    """An output buffer filled with NaN, so a row a kernel fails to write cannot pass as a result left
    there by an earlier call (the caching allocator hands freed blocks back)."""
    return torch.full_like(t, float("nan"))


def nan_empty(shape, device, dtype=torch.float32) -> torch.Tensor:
    return torch.full(shape, float("nan"), dtype=dtype, device=device)


def poisoned_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace whose every byte is 0xFF (each fp32 word a NaN): the ABI says its contents on entry do
    not matter, so a kernel that reads a slot before writing it shows up as NaN in the output."""
    return torch.full((max(int(nbytes), 1),), 0xFF, dtype=torch.uint8, device=device)


def run_library(w: Workload, device, partition_size=0, path=_lib.PATH_AUTO, with_lse=True,
                ragged=None, k_cache=None, v_cache=None, schedule=0, depth=0):
    meta = w.device_meta(device)
    out = nan_like(w.q)
    lse = nan_empty((w.total_q, w.spec.num_heads), device) if with_lse else None
    use_qlens = (not w.uniform_q) if ragged is None else ragged
    code = ((_lib.PKV_BF16_FP8KV if w.kv_fp8 else _lib.PKV_BF16) if w.spec.dtype == "bf16" else _lib.PKV_F32)
    ws = poisoned_workspace(_lib.decode_workspace_bytes(
        w.num_seqs, w.total_q, w.max_q_len, w.max_context_len, w.spec.num_heads, w.spec.num_kv_heads,
        w.spec.head_dim, code, partition_size, path, depth, schedule), device)
    _lib.paged_attn_decode(w.q, w.k_cache if k_cache is None else k_cache,
                           w.v_cache if v_cache is None else v_cache,
                           meta["block_tables"], meta["context_lens"], meta["q_lens"] if use_qlens else None,
                           out, lse, w.spec.num_heads, w.spec.num_kv_heads, w.spec.head_dim,
                           w.spec.block_size, w.scale, w.max_context_len, max_q_len=w.max_q_len,
                           partition_size=partition_size, path=path, schedule=schedule, depth=depth,
                           k_scale=w.spec.k_scale if w.kv_fp8 else 0.0, v_scale=w.spec.v_scale if w.kv_fp8 else 0.0,
                           workspace=ws)
    torch.cuda.synchronize()
    return out, lse


def widen_out(out: torch.Tensor) -> np.ndarray:
    return O.widen(host_bits(out))


def _pools(w: Workload, kc, vc):
    """Host pools for the oracle: bit patterns, or for E4M3 pools the values their codes stand for."""
    if w.kv_fp8:
        return F8.dequantize(kc, w.spec.k_scale), F8.dequantize(vc, w.spec.v_scale)
    return kc, vc


def oracle_full(w: Workload, k_cache=None, v_cache=None):
    kc = host_bits(w.k_cache if k_cache is None else k_cache)
    vc = host_bits(w.v_cache if v_cache is None else v_cache)
    kc, vc = _pools(w, kc, vc)
    return O.paged_decode_attention(host_bits(w.q), kc, vc, w.block_tables, w.context_lens, w.q_lens,
                                    w.scale, w.spec.num_kv_heads, w.spec.block_size)


def host_threads() -> int:
    """Worker threads for host-side oracle runs: the cores this process may use, at most 16 (the host
    share of one GPU on the test machines)."""
    import os

    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_all(w: Workload, k_cache=None, v_cache=None, seqs=None, threads=None):
    """The oracle on every sequence of a workload (or on `seqs`), for workloads too large for one
    oracle_full call: each sequence is its own single-sequence oracle call over a host copy of just
    its pages (E4M3 pages decoded per sequence), and the calls are spread over host threads (numpy
    releases the GIL in its array work; BLAS runs one thread per call).  Rows of sequences not listed
    stay NaN.  Returns (out [total_q, H, D], lse [total_q, H]) in float64, like oracle_full."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    kc_d = w.k_cache if k_cache is None else k_cache
    vc_d = w.v_cache if v_cache is None else v_cache
    B = w.spec.block_size
    H, D = w.spec.num_heads, w.spec.head_dim
    seqs = list(range(w.num_seqs)) if seqs is None else [int(s) for s in seqs]
    nblk = (w.context_lens.astype(np.int64) + B - 1) // B
    ids = np.concatenate([w.block_tables[s, :nblk[s]].astype(np.int64) for s in seqs])
    uniq = np.unique(ids)
    idx = torch.from_numpy(uniq).to(kc_d.device)
    kc_h = host_bits(kc_d.index_select(0, idx))           # only the pages some listed sequence reads
    vc_h = host_bits(vc_d.index_select(0, idx))
    remap = np.full(max(int(w.num_blocks), int(uniq.max()) + 1), -1, np.int64)
    remap[uniq] = np.arange(uniq.shape[0])
    q_h = host_bits(w.q)
    starts = np.concatenate([[0], np.cumsum(w.q_lens.astype(np.int64))])
    out = np.full((w.total_q, H, D), np.nan)
    lse = np.full((w.total_q, H), np.nan)

    def one(s):
        n, qs, b = int(w.context_lens[s]), int(w.q_lens[s]), int(starts[s])
        loc = remap[w.block_tables[s, :nblk[s]].astype(np.int64)]
        kc, vc = _pools(w, kc_h[loc], vc_h[loc])
        table = np.arange(nblk[s], dtype=np.int32)[None, :]
        o, l = O.paged_decode_attention(q_h[b:b + qs], kc, vc, table, np.array([n], np.int32),
                                        np.array([qs], np.int32), w.scale, w.spec.num_kv_heads, B)
        out[b:b + qs] = o
        lse[b:b + qs] = l

    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(threads or host_threads()) as ex:
            list(ex.map(one, sorted(seqs, key=lambda s: -int(w.context_lens[s]) * int(w.q_lens[s]))))
    return out, lse


def tolerance(w: Workload) -> float:
    return F32_TOL if w.spec.dtype == "f32" else BF16_TOL


# Diagnostic gate for bf16 outputs, far tighter than the 1.5e-2 bar: an output element may differ from
# the oracle by its own bf16 rounding (at most |ref| 2^-9) plus the same again, plus 2e-3 for the
# probabilities the value product multiplies in bf16.  A dropped key, a wrong scale or a misplaced
# partial moves elements by much more at small |ref| long before the absolute bar trips.
BF16_DIAG_REL = 2.0 ** -8
BF16_DIAG_ABS = 2e-3


def compare(w: Workload, out, lse, ref_out, ref_lse, rows=None):
    """Max |delta| of out and lse over the rows the oracle computed (NaN rows are skipped).  For bf16
    outputs it also prints, and asserts, the diagnostic gate |delta| <= |ref| 2^-8 + 2e-3 element by
    element, with the largest error beyond the output's own bf16 rounding (|delta| - |ref| 2^-9)."""
    got = widen_out(out)
    mask = ~np.isnan(ref_out[:, 0, 0]) if rows is None else rows
    delta = np.abs(got[mask] - ref_out[mask])
    d_out = float(np.max(delta))
    d_lse = float("nan")
    if lse is not None:
        gl = lse.detach().cpu().numpy().astype(np.float64)
        d_lse = float(np.max(np.abs(gl[mask] - ref_lse[mask])))
    if out.dtype == torch.bfloat16:
        mag = np.abs(ref_out[mask])
        beyond = float(np.max(delta - mag * 2.0 ** -9))
        slack = float(np.max(delta - (mag * BF16_DIAG_REL + BF16_DIAG_ABS)))
        print(f"   bf16 diagnostic: beyond own rounding {beyond:.3e}, gate margin {-slack:.3e}", flush=True)
        assert np.isfinite(slack) and slack <= 0.0, (
            f"bf16 diagnostic gate |d| <= |ref| 2^-8 + 2e-3 exceeded by {slack:.3e}")
    return d_out, d_lse
