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


def run_library(w: Workload, device, partition_size=0, path=_lib.PATH_AUTO, with_lse=True,
                ragged=None, k_cache=None, v_cache=None, schedule=0, depth=0):
    meta = w.device_meta(device)
    out = torch.empty_like(w.q)
    lse = torch.empty((w.total_q, w.spec.num_heads), dtype=torch.float32, device=device) if with_lse else None
    use_qlens = (not w.uniform_q) if ragged is None else ragged
    _lib.paged_attn_decode(w.q, w.k_cache if k_cache is None else k_cache,
                           w.v_cache if v_cache is None else v_cache,
                           meta["block_tables"], meta["context_lens"], meta["q_lens"] if use_qlens else None,
                           out, lse, w.spec.num_heads, w.spec.num_kv_heads, w.spec.head_dim,
                           w.spec.block_size, w.scale, w.max_context_len, max_q_len=w.max_q_len,
                           partition_size=partition_size, path=path, schedule=schedule, depth=depth,
                           k_scale=w.spec.k_scale if w.kv_fp8 else 0.0, v_scale=w.spec.v_scale if w.kv_fp8 else 0.0)
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


def oracle_sampled(w: Workload, seqs, k_cache=None, v_cache=None):
    """Oracle on a few sequences of a large workload: only their pages are copied to the host
    (a compacted pool with the block tables renumbered to match)."""
    kc_d = w.k_cache if k_cache is None else k_cache
    vc_d = w.v_cache if v_cache is None else v_cache
    B = w.spec.block_size
    ids = []
    for s in seqs:
        n = int(w.context_lens[s])
        ids.extend(int(b) for b in w.block_tables[s, : (n + B - 1) // B])
    uniq = np.unique(np.asarray(ids, dtype=np.int64))
    remap = {int(b): i for i, b in enumerate(uniq)}
    idx = torch.from_numpy(uniq).to(kc_d.device)
    kc, vc = _pools(w, host_bits(kc_d.index_select(0, idx)), host_bits(vc_d.index_select(0, idx)))
    table = np.full_like(w.block_tables, -1)
    for s in seqs:
        n = int(w.context_lens[s])
        for j in range((n + B - 1) // B):
            table[s, j] = remap[int(w.block_tables[s, j])]
    return O.paged_decode_attention(host_bits(w.q), kc, vc, table, w.context_lens, w.q_lens, w.scale,
                                    w.spec.num_kv_heads, B, seqs=list(seqs))


def tolerance(w: Workload) -> float:
    return F32_TOL if w.spec.dtype == "f32" else BF16_TOL


def compare(w: Workload, out, lse, ref_out, ref_lse, rows=None):
    """Max |delta| of out and lse over the rows the oracle computed (NaN rows are skipped)."""
    got = widen_out(out)
    mask = ~np.isnan(ref_out[:, 0, 0]) if rows is None else rows
    d_out = float(np.max(np.abs(got[mask] - ref_out[mask])))
    d_lse = float("nan")
    if lse is not None:
        gl = lse.detach().cpu().numpy().astype(np.float64)
        d_lse = float(np.max(np.abs(gl[mask] - ref_lse[mask])))
    return d_out, d_lse
