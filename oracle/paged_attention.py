"""CPU float64 oracle for paged decode attention and the slot-mapped KV-cache write.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The HIP library never calls it, and it shares no code, header, table or helper
with the HIP library: it reads the documented memory layout on its own and does the arithmetic in
plain numpy float64.

What it computes
----------------
Paging moves K/V rows into fixed-size physical blocks reached through a per-sequence block table; it
does not change the attention result.  The inferd page says so twice: its repository tree lists a
plain "paged-attention reference" beside the block allocator/page table, and its results table reports
the paged path matching the unpaged one with zero logit difference.  The lfm25-inference page
("Runtime Design") names the same operation for grouped-query heads (GQA/XQA) with a split-K
reduction.  So the oracle is the textbook definition written out, on the K/V rows gathered through
the block table:

  for sequence s, query row i in [0, q_s), query head h:
    kv head         g = h // (H / KVH)                (consecutive query heads share a KV head)
    visible keys    t = 0 .. ctx_s - q_s + i           (the q_s new tokens are the last positions)
    score           x_t  = scale * <q[row, h], K_s[t]>
    output          out  = sum_t softmax(x)_t * V_s[t]
    log-sum-exp     lse  = log sum_t exp(x_t)          (natural log)

Readings the pages leave open (all listed with reasons in the design notes):
  * context_lens counts the new query tokens (the newest token attends to itself);
  * row i of a q-token step sees keys up to ctx - q + i (causal among the new tokens);
  * query head h reads KV head h // (H / KVH);
  * bf16 values are widened exactly (bits << 16 -> fp32 -> fp64) before any arithmetic;
  * lse uses the natural log of the sum over visible, scaled scores.

Memory layout read here (the library's ABI):
  q        [total_q, H, D]       rows packed sequence after sequence (row offset = sum of earlier q_lens)
  k_cache  [num_blocks, KVH, B, D]
  v_cache  [num_blocks, KVH, D, B]
  block_tables [S, max_blocks_per_seq] int32, context_lens [S] int32, q_lens [S] int32
Floating inputs are numpy float32 arrays or uint16 arrays holding bf16 bit patterns.
"""
from __future__ import annotations

import numpy as np


def widen(x: np.ndarray) -> np.ndarray:
    """Exact widening to float64.  uint16 arrays are bf16 bit patterns: a bf16 value is the upper half
    of the fp32 with the same bits, so shifting the pattern left by 16 gives that fp32 exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype == np.float32 or x.dtype == np.float64:
        return x.astype(np.float64)
    raise TypeError(f"unsupported element type {x.dtype}")


def gather_kv(k_cache, v_cache, block_table_row, context_len, kv_head, block_size):
    """K and V rows 0..context_len-1 of one sequence and one KV head, as float64 [n, D].

    Logical token t lives in physical block block_table_row[t // B] at offset t % B (the page-table
    indirection of the inferd page's block allocator + page table).  Only the blocks the sequence
    covers are read; table entries past them are never looked at."""
    n = int(context_len)
    nblk = -(-n // block_size)
    ids = np.asarray(block_table_row[:nblk], dtype=np.int64)
    kb = widen(k_cache[ids, kv_head])            # [nblk, B, D]
    vb = widen(v_cache[ids, kv_head])            # [nblk, D, B]
    D = kb.shape[-1]
    K = kb.reshape(nblk * block_size, D)[:n]
    V = np.transpose(vb, (0, 2, 1)).reshape(nblk * block_size, D)[:n]
    return K, V


def attend(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, last_visible: np.ndarray):
    """Softmax attention of query rows over K/V with a per-row last visible key index.

    qrows [R, D], K/V [n, D] float64; row r sees keys 0..last_visible[r].  Returns out [R, D] and the
    natural-log lse [R].  Max subtraction is exact algebra: it only keeps exp in range."""
    x = scale * (qrows @ K.T)                                 # [R, n]
    t = np.arange(K.shape[0])[None, :]
    visible = t <= last_visible[:, None]
    x = np.where(visible, x, -np.inf)
    m = x.max(axis=1, keepdims=True)
    w = np.exp(x - m)                                        # exp(-inf) = 0 on hidden keys
    z = w.sum(axis=1, keepdims=True)
    out = (w / z) @ V
    lse = m[:, 0] + np.log(z[:, 0])
    return out, lse


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, q_lens, scale,
                           num_kv_heads, block_size=16, seqs=None, heads=None):
    """Decode attention over a paged cache: the definition in the module docstring.

    Returns (out [total_q, H, D] float64, lse [total_q, H] float64).  `seqs` / `heads` restrict the
    work to a subset (rows of other sequences / heads are left NaN) so large workloads can be
    checked on samples."""
    q = np.asarray(q)
    total_q, H, D = q.shape
    KVH = int(num_kv_heads)
    if H % KVH:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = H // KVH
    S = len(context_lens)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(q_lens)])
    if starts[-1] != total_q:
        raise ValueError("sum(q_lens) must equal the number of q rows")
    out = np.full((total_q, H, D), np.nan)
    lse = np.full((total_q, H), np.nan)
    seq_list = range(S) if seqs is None else seqs
    head_set = None if heads is None else set(int(h) for h in heads)
    for s in seq_list:
        n = int(context_lens[s])
        qs = int(q_lens[s])
        if not (1 <= qs <= n):
            raise ValueError("each sequence needs 1 <= q_len <= context_len")
        base = int(starts[s])
        last = n - qs + np.arange(qs)                     # last visible key of each new token
        for g in range(KVH):
            hs = [h for h in range(g * G, (g + 1) * G) if head_set is None or h in head_set]
            if not hs:
                continue
            K, V = gather_kv(k_cache, v_cache, block_tables[s], n, g, block_size)
            rows = widen(q[base:base + qs][:, hs, :]).reshape(qs * len(hs), D)
            o, l = attend(rows, K, V, scale, np.repeat(last, len(hs)))
            out[base:base + qs, hs, :] = o.reshape(qs, len(hs), D)
            lse[base:base + qs, hs] = l.reshape(qs, len(hs))
    return out, lse


def partition_attention(q, k_cache, v_cache, block_tables, context_lens, q_lens, scale,
                        num_kv_heads, partition_size, block_size=16):
    """The same attention restricted to key partitions [p*P, (p+1)*P): the split-K step the
    lfm25-inference page names for decode ("Runtime Design").  Returns lists over p of
    (out_p, lse_p); a row with no visible key in a partition gets out_p = 0 and lse_p = -inf."""
    q = np.asarray(q)
    total_q, H, D = q.shape
    G = H // int(num_kv_heads)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(q_lens)])
    nparts = int(-(-int(np.max(context_lens)) // partition_size))
    outs = [np.zeros((total_q, H, D)) for _ in range(nparts)]
    lses = [np.full((total_q, H), -np.inf) for _ in range(nparts)]
    for s in range(len(context_lens)):
        n = int(context_lens[s])
        qs = int(q_lens[s])
        base = int(starts[s])
        last = n - qs + np.arange(qs)
        for g in range(int(num_kv_heads)):
            K, V = gather_kv(k_cache, v_cache, block_tables[s], n, g, block_size)
            rows = widen(q[base:base + qs, g * G:(g + 1) * G, :]).reshape(qs * G, D)
            lastr = np.repeat(last, G)
            for p in range(-(-n // partition_size)):
                lo, hi = p * partition_size, min(n, (p + 1) * partition_size)
                seen = lastr >= lo
                if not seen.any():
                    continue
                o, l = attend(rows[seen], K[lo:hi], V[lo:hi], scale, lastr[seen] - lo)
                ob = np.zeros((qs * G, D))
                lb = np.full(qs * G, -np.inf)
                ob[seen], lb[seen] = o, l
                outs[p][base:base + qs, g * G:(g + 1) * G, :] = ob.reshape(qs, G, D)
                lses[p][base:base + qs, g * G:(g + 1) * G] = lb.reshape(qs, G)
    return outs, lses


def lse_combine(outs, lses):
    """Merge per-partition results: lse = log sum_p exp(lse_p) and out = sum_p exp(lse_p - lse) out_p.
    Each partial is a softmax over its own keys; rescaling by exp(lse_p - lse) turns it into its share
    of the softmax over all keys.  Partitions with lse_p = -inf weigh nothing."""
    L = np.stack(lses)                                  # [P, ...]
    m = L.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(L - m_safe)                              # exp(-inf) = 0
    z = w.sum(axis=0)
    lse = m_safe + np.log(z)
    out = sum(w[p][..., None] * outs[p] for p in range(len(outs))) / z[..., None]
    return out, lse


def shared_len(context_len, q_len, group_prefix, block_size=16):
    """Keys of a group member read through the group's shared blocks: the group's prefix, cut to the
    whole pages before the member's new tokens (those tokens are its own, never shared)."""
    return min(int(group_prefix), (int(context_len) - int(q_len)) // block_size * block_size)


def shared_prefix_attention(q, k_cache, v_cache, block_tables, context_lens, q_lens, scale, num_kv_heads,
                            group_starts, prefix_lens, prefix_blocks, block_size=16):
    """Decode attention computed the read-once way (lfm25-inference, "Runtime Design": prefix reuse
    through a radix tree, and the log-sum-exp merge of split-K parts): for each group of consecutive
    sequences, the query rows of all members attend the group's shared blocks in one product (member
    s sees its first P_s keys there, P_s = shared_len), each sequence attends its keys P_s .. ctx - 1
    through its own block table, and the two parts merge with lse_combine.  Sequences outside every
    group have P_s = 0.  Returns (out, lse) like paged_decode_attention, which it equals up to
    rounding: a softmax over a key set is the merge of softmaxes over any partition of it."""
    q = np.asarray(q)
    total_q, H, D = q.shape
    KVH = int(num_kv_heads)
    G = H // KVH
    S = len(context_lens)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(q_lens)])
    P = np.zeros(S, dtype=np.int64)
    owner = np.full(S, -1)
    for g in range(len(prefix_lens)):
        for s in range(int(group_starts[g]), int(group_starts[g + 1])):
            owner[s] = g
            P[s] = shared_len(context_lens[s], q_lens[s], prefix_lens[g], block_size)
    pre_o = np.zeros((total_q, H, D))
    pre_l = np.full((total_q, H), -np.inf)
    # the shared part: one product per (group, kv head) over the stacked rows of its members
    for g in range(len(prefix_lens)):
        members = [s for s in range(int(group_starts[g]), int(group_starts[g + 1])) if P[s] > 0]
        if not members:
            continue
        pg = int(prefix_lens[g])
        for kv in range(KVH):
            K, V = gather_kv(k_cache, v_cache, prefix_blocks[g], pg, kv, block_size)
            rows, last, where = [], [], []
            for s in members:
                for i in range(int(q_lens[s])):
                    for h in range(kv * G, (kv + 1) * G):
                        rows.append(widen(q[starts[s] + i, h]))
                        last.append(P[s] - 1)
                        where.append((starts[s] + i, h))
            o, l = attend(np.stack(rows), K, V, scale, np.asarray(last))
            for r, (row, h) in enumerate(where):
                pre_o[row, h], pre_l[row, h] = o[r], l[r]
    # each sequence's own keys
    suf_o = np.zeros((total_q, H, D))
    suf_l = np.full((total_q, H), -np.inf)
    for s in range(S):
        n, qs, base, ps = int(context_lens[s]), int(q_lens[s]), int(starts[s]), int(P[s])
        last = n - qs + np.arange(qs) - ps
        for kv in range(KVH):
            K, V = gather_kv(k_cache, v_cache, block_tables[s], n, kv, block_size)
            rows = widen(q[base:base + qs, kv * G:(kv + 1) * G, :]).reshape(qs * G, D)
            o, l = attend(rows, K[ps:], V[ps:], scale, np.repeat(last, G))
            suf_o[base:base + qs, kv * G:(kv + 1) * G] = o.reshape(qs, G, D)
            suf_l[base:base + qs, kv * G:(kv + 1) * G] = l.reshape(qs, G)
    return lse_combine([pre_o, suf_o], [pre_l, suf_l])


def kv_cache_write(k_cache, v_cache, k, v, slot_mapping, block_size=16):
    """Slot-mapped append: new row t goes to physical slot slot_mapping[t] = block * B + offset, i.e.
    k_cache[block, :, offset, :] = k[t] and v_cache[block, :, :, offset] = v[t]; a negative slot
    skips the row.  Bits are moved unchanged.  Returns new arrays; the inputs are left alone.
    (The inferd page's follow-up plan wires the block allocator into live decode: this is the write
    that puts each step's new K/V into its page.)"""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        kc[blk, :, off, :] = k[t]
        vc[blk, :, :, off] = v[t]
    return kc, vc
