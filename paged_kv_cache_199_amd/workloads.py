"""Seeded synthetic decode workloads: the one module both the HIP path and the oracle consume.

This module draws inputs only. It holds none of the attention arithmetic: it picks context lengths,
lays out a physical block pool, hands out block ids through per-sequence block tables, draws Q/K/V
values and (optionally) poisons the slots that no sequence may read.  The shapes follow the workloads
the pages describe: 16-token pages (lfm25-inference, "Run Inference" and "Production Defaults": page
size 16 as a startup policy), concurrency 32 (inferd, results table), a shared ~512-token document
prefix (lfm25-inference, radix prefix-cache table), gamma drafts plus one bonus token (inferd,
speculative-decoding acceptance rule) and long ragged contexts split into partitions (lfm25-inference,
"Runtime Design", split-K decode).  The pages publish no dataset for this path; these seeded draws
stand in for it.

Memory layout of the cache pool (the library's ABI; the pages fix none):
  k_cache [num_blocks, num_kv_heads, block_size, head_dim]   token-major rows inside a block
  v_cache [num_blocks, num_kv_heads, head_dim, block_size]   dim-major rows inside a block
q / out are [total_q, num_heads, head_dim], rows packed sequence after sequence.

Draw order (fixed, so a seed reproduces a config bit for bit on one device kind):
  numpy default_rng(seed): context lengths -> block permutation -> (q lengths if ragged)
  torch Generator(seed) on the target device: q -> k pool -> v pool -> new k -> new v
The torch stream differs between CPU and GPU generators, so a workload is reproducible per device
kind; the oracle always reads the very tensors the kernels read (copied to the host).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

BLOCK_SIZE = 16
DTYPES = ("f32", "bf16")


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one decode workload."""

    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    # context lengths: an explicit list, or ("uniform", lo, hi) inclusive, or
    # ("lognormal", median, sigma, lo, hi)
    ctx: object
    # query tokens per sequence: an int (uniform) or an explicit list (ragged)
    q_len: object = 1
    block_size: int = BLOCK_SIZE
    # pool sizing: explicit block count, else ceil(pool_factor * unique blocks needed)
    pool_blocks: Optional[int] = None
    pool_factor: float = 1.25
    # number of leading logical blocks every sequence shares (radix-style prefix reuse)
    shared_prefix_blocks: int = 0
    # append one new token per sequence through slot_mapping (its position is ctx - 1)
    write_new_token: bool = False
    # partition size the bench times this workload with (0 = library policy)
    partition_size: int = 0
    seed: int = 0
    # K/V pools of 8-bit E4M3 codes (q, out and new rows stay bf16) standing for code * scale
    kv_fp8: bool = False
    k_scale: float = 1.0 / 32
    v_scale: float = 1.0 / 32
    # many new tokens per sequence: timed through the prefill entry point
    prefill: bool = False


# The five named workloads.  Index i is seeded with 1000 + i.
NAMED: List[Spec] = [
    Spec("tiny_fp32", 4, 4, 2, 64, "f32", ctx=[1, 7, 16, 33], pool_blocks=16, seed=1000),
    Spec("conc32_bf16", 32, 32, 8, 128, "bf16", ctx=("uniform", 256, 2048),
         write_new_token=True, seed=1001),
    Spec("shared_prefix_bf16", 8, 32, 8, 64, "bf16", ctx=("uniform", 128, 4096),
         shared_prefix_blocks=32, seed=1002),
    Spec("spec_verify_bf16", 32, 32, 8, 128, "bf16", ctx=("uniform", 512, 8192), q_len=5,
         seed=1003),
    Spec("long_ctx_splitk_bf16", 256, 64, 8, 128, "bf16", ctx=("lognormal", 4096, 0.8, 64, 32768),
         seed=1004),
    # a system-prompt-heavy batch: 64 requests behind one 4096-token shared prefix, private tails of
    # 128..1024 tokens (the read-once decode's case; a stand-in sized for this chip)
    Spec("shared_prefix_64x4k_bf16", 64, 32, 8, 128, "bf16", ctx=("uniform", 4096 + 128, 4096 + 1024),
         shared_prefix_blocks=256, seed=1005),
    # chunked prefill: 16 sequences each appending a 512-token chunk to 0..3584 cached tokens
    Spec("prefill_chunk_bf16", 16, 32, 8, 128, "bf16", ctx=("uniform", 512, 4096), q_len=512, seed=1006,
         prefill=True),
    # the same two batches over E4M3 pools (the FP8 KV cache): half the cache bytes
    Spec("conc32_fp8kv", 32, 32, 8, 128, "bf16", ctx=("uniform", 256, 2048), write_new_token=True, seed=1001,
         kv_fp8=True),
    Spec("long_ctx_fp8kv", 256, 64, 8, 128, "bf16", ctx=("lognormal", 4096, 0.8, 64, 32768), seed=1004,
         kv_fp8=True),
    Spec("prefill_chunk_fp8kv", 16, 32, 8, 128, "bf16", ctx=("uniform", 512, 4096), q_len=512, seed=1006,
         prefill=True, kv_fp8=True),
]


def named(index_or_name) -> Spec:
    if isinstance(index_or_name, int):
        return NAMED[index_or_name]
    for s in NAMED:
        if s.name == index_or_name:
            return s
    raise KeyError(index_or_name)


@dataclasses.dataclass
class Workload:
    spec: Spec
    scale: float
    context_lens: np.ndarray          # int32 [S], includes the new query tokens
    q_lens: np.ndarray                # int32 [S]
    block_tables: np.ndarray          # int32 [S, max_blocks_per_seq], -1 padding
    num_blocks: int
    used_blocks: np.ndarray           # sorted unique physical block ids referenced
    slot_mapping: Optional[np.ndarray]  # int64 [T_new] or None
    q: torch.Tensor                   # [total_q, H, D]
    k_cache: torch.Tensor             # [num_blocks, KVH, B, D]
    v_cache: torch.Tensor             # [num_blocks, KVH, D, B]
    new_k: Optional[torch.Tensor]     # [T_new, KVH, D]
    new_v: Optional[torch.Tensor]

    @property
    def kv_fp8(self) -> bool:
        return self.spec.kv_fp8

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max())

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def uniform_q(self) -> bool:
        return bool((self.q_lens == self.q_lens[0]).all())

    def device_meta(self, device):
        """Metadata tensors on `device` (block tables, lengths, slots)."""
        d = {
            "block_tables": torch.from_numpy(self.block_tables).to(device),
            "context_lens": torch.from_numpy(self.context_lens).to(device),
            "q_lens": torch.from_numpy(self.q_lens).to(device),
        }
        if self.slot_mapping is not None:
            d["slot_mapping"] = torch.from_numpy(self.slot_mapping).to(device)
        return d


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _draw_context_lens(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    c = spec.ctx
    if isinstance(c, (list, tuple)) and c and not isinstance(c[0], str):
        out = np.asarray(c, dtype=np.int64)
        assert out.shape[0] == spec.num_seqs
    elif c[0] == "uniform":
        _, lo, hi = c
        out = rng.integers(lo, hi + 1, size=spec.num_seqs)
    elif c[0] == "lognormal":
        _, median, sigma, lo, hi = c
        out = np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=spec.num_seqs))),
                      lo, hi)
    else:
        raise ValueError(f"unknown context distribution {c!r}")
    return out.astype(np.int32)


def _q_lens(spec: Spec) -> np.ndarray:
    if isinstance(spec.q_len, (list, tuple)):
        out = np.asarray(spec.q_len, dtype=np.int32)
        assert out.shape[0] == spec.num_seqs
        return out
    return np.full(spec.num_seqs, int(spec.q_len), dtype=np.int32)


def _assign_blocks(spec: Spec, ctx: np.ndarray, rng: np.random.Generator):
    B = spec.block_size
    nblk = (ctx.astype(np.int64) + B - 1) // B
    shared = spec.shared_prefix_blocks
    unique_needed = int(sum(max(0, int(n) - shared) for n in nblk)) + (shared if shared else 0)
    if spec.pool_blocks is not None:
        pool = int(spec.pool_blocks)
    else:
        pool = int(math.ceil(spec.pool_factor * unique_needed))
    if pool < unique_needed:
        raise ValueError("pool too small for the drawn context lengths")
    perm = rng.permutation(pool).astype(np.int32)
    cursor = 0
    shared_ids = perm[cursor:cursor + shared]
    cursor += shared
    max_blocks = int(nblk.max())
    table = np.full((spec.num_seqs, max_blocks), -1, dtype=np.int32)
    for s, n in enumerate(nblk):
        n = int(n)
        k = min(n, shared)
        table[s, :k] = shared_ids[:k]
        rest = n - k
        table[s, k:n] = perm[cursor:cursor + rest]
        cursor += rest
    used = np.unique(table[table >= 0])
    return table, pool, used


def _randn(shape, gen: torch.Generator, device, dtype: str, chunk_elems: int = 1 << 27) -> torch.Tensor:
    """N(0,1) draws as fp32, rounded to nearest-even into bf16 where asked; generated in chunks so a
    multi-GB pool never needs a full fp32 temporary."""
    out = torch.empty(shape, dtype=torch_dtype(dtype), device=device)
    flat = out.view(-1)
    n = flat.numel()
    for start in range(0, n, chunk_elems):
        m = min(chunk_elems, n - start)
        x = torch.randn(m, generator=gen, device=device, dtype=torch.float32)
        flat[start:start + m].copy_(x.to(out.dtype))
    return out


def _randn_fp8(shape, gen: torch.Generator, device, scale: float, chunk_elems: int = 1 << 27) -> torch.Tensor:
    """E4M3 codes (uint8) of N(0,1) draws divided by `scale`, by torch's float8_e4m3fn conversion
    (|x / scale| stays far below 448 at the scales used here)."""
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for start in range(0, n, chunk_elems):
        m = min(chunk_elems, n - start)
        x = torch.randn(m, generator=gen, device=device, dtype=torch.float32)
        flat[start:start + m].copy_((x / scale).to(torch.float8_e4m3fn).view(torch.uint8))
    return out


def build(spec_or_index, device="cpu", poison: bool = False) -> Workload:
    """Draw a workload on `device`.

    poison=True writes NaN into every slot no sequence may read: the tail of each sequence's last
    block (positions >= its context length) and every pool block no block table references.
    A correct kernel's output does not change.
    """
    spec = named(spec_or_index) if isinstance(spec_or_index, (int, str)) else spec_or_index
    assert spec.dtype in DTYPES
    assert spec.num_heads % spec.num_kv_heads == 0
    rng = np.random.default_rng(spec.seed)
    ctx = _draw_context_lens(spec, rng)
    qlens = _q_lens(spec)
    if (qlens > ctx).any() or (qlens < 1).any():
        raise ValueError("each sequence needs 1 <= q_len <= context_len")
    table, pool, used = _assign_blocks(spec, ctx, rng)

    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed)
    S, H, KVH, D, B = spec.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    total_q = int(qlens.sum())
    q = _randn((total_q, H, D), gen, device, spec.dtype)
    if spec.kv_fp8:
        k_cache = _randn_fp8((pool, KVH, B, D), gen, device, spec.k_scale)
        v_cache = _randn_fp8((pool, KVH, D, B), gen, device, spec.v_scale)
    else:
        k_cache = _randn((pool, KVH, B, D), gen, device, spec.dtype)
        v_cache = _randn((pool, KVH, D, B), gen, device, spec.dtype)
    slot_mapping = new_k = new_v = None
    if spec.write_new_token:
        pos = ctx.astype(np.int64) - 1
        blk = table[np.arange(S), pos // B].astype(np.int64)
        slot_mapping = blk * B + pos % B
        new_k = _randn((S, KVH, D), gen, device, spec.dtype)
        new_v = _randn((S, KVH, D), gen, device, spec.dtype)

    if poison:
        nan = 0x7F if spec.kv_fp8 else float("nan")          # E4M3's NaN code
        for s in range(S):
            n = int(ctx[s])
            tail = n % B
            if tail:
                last = int(table[s, (n - 1) // B])
                k_cache[last, :, tail:, :] = nan
                v_cache[last, :, :, tail:] = nan
        unused = np.setdiff1d(np.arange(pool), used)
        if unused.size:
            idx = torch.from_numpy(unused.astype(np.int64)).to(device)
            k_cache.index_fill_(0, idx, nan)
            v_cache.index_fill_(0, idx, nan)

    return Workload(spec=spec, scale=1.0 / math.sqrt(D), context_lens=ctx, q_lens=qlens,
                    block_tables=table, num_blocks=pool, used_blocks=used,
                    slot_mapping=slot_mapping, q=q, k_cache=k_cache, v_cache=v_cache,
                    new_k=new_k, new_v=new_v)


def custom(name: str, ctx: Sequence[int], q_len=1, num_heads=8, num_kv_heads=2, head_dim=128,
           dtype="bf16", seed=7, **kw) -> Spec:
    """Spec for an explicit list of context lengths (edge-case parity runs)."""
    return Spec(name, len(ctx), num_heads, num_kv_heads, head_dim, dtype, ctx=list(ctx),
                q_len=q_len, seed=seed, **kw)


def share_prefixes(w: Workload, groups):
    """Make consecutive sequences share prefix blocks: groups = [(first, end, prefix_tokens)], prefix
    a multiple of 16.  Each group takes its prefix ids from its longest member (cut to that member's
    blocks) and every member's table points its leading blocks (as many as it has, up to the prefix)
    at them.  Rewrites w.block_tables in place; returns (group_starts [n+1], prefix_lens [n],
    prefix_blocks [n, max prefix blocks]) int32 arrays describing the groups."""
    B = w.spec.block_size
    nblk = (w.context_lens.astype(np.int64) + B - 1) // B
    starts, lens, rows = [], [], []
    for first, end, prefix in groups:
        assert prefix % B == 0 and 0 <= first <= end <= w.num_seqs
        members = list(range(first, end))
        donor = max(members, key=lambda s: int(nblk[s])) if members else first
        pb = min(prefix // B, int(nblk[donor])) if members else 0
        ids = w.block_tables[donor, :pb].copy()
        for s in members:
            k = min(int(nblk[s]), pb)
            w.block_tables[s, :k] = ids[:k]
        if starts and starts[-1] != first:
            raise ValueError("groups must be consecutive")
        if not starts:
            starts.append(first)
        starts.append(end)
        lens.append(pb * B)
        rows.append(ids)
    width = max([len(r) for r in rows] + [1])
    blocks = np.zeros((len(rows), width), dtype=np.int32)
    for g, r in enumerate(rows):
        blocks[g, :len(r)] = r
    return np.asarray(starts, dtype=np.int32), np.asarray(lens, dtype=np.int32), blocks
