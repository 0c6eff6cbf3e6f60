// Launch arguments shared by the host API and the decode kernels (internal; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct DecodeArgs {
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *q_lens;       // NULL: every sequence has max_q_len rows
  const int32_t *q_start;      // exclusive prefix of q_lens (workspace), NULL when q_lens is NULL
  void *out;
  float *lse;                  // may be NULL
  float *part_o;               // [num_parts][total_q][H][D] fp32, NULL when num_parts == 1
  float *part_lse;             // [num_parts][total_q][H], log2 units
  int64_t num_blocks;
  int num_seqs;
  int max_blocks_per_seq;
  int total_q;
  int max_q_len;
  int max_context_len;
  int num_heads;
  int num_kv_heads;
  int group;                   // num_heads / num_kv_heads
  float scale_log2;            // scale * log2(e) (* the K pool's scale): scores live in log2 units
  float v_scale;               // the V pool's scale (1 for bf16 pools)
  float k_scale;               // the K pool's scale (1 for bf16 pools; scale_log2 already holds it)
  int part_size;               // keys per partition
  int num_parts;               // ceil(max_context_len / part_size)
  int row_tiles;               // row tiles per (sequence, kv head)
  int units;                   // num_kv_heads * num_parts * num_seqs * row_tiles
  int per_xcd;                 // ceil(units / 8)
  // balanced (persistent) schedule only
  int32_t *item_pre;           // [num_seqs + 1] stream pages of one kv head before each sequence
  int64_t spill_base;          // first spill row of part_o / part_lse; -1: no spill rows (grid)
  int share_waves;             // waves per XCD in the persistent grid
  int cut_align;               // share boundaries inside a work item fall on multiples of this
  int item_cost;               // pages of stream charged to each work item's start (its pipeline restart)
  int rows_per_tile;
  // balanced schedule without fixed partitions: piece k < max_pieces of a work item (in stream order,
  // piece 0 at the item's start) leaves its partial in partition row k, later pieces in their wave's
  // spill rows, and the piece that ends an item writes the item's piece count to item_cnt
  // (max_pieces + 1 when there are more).  The merge then finds a row's sources with no search.
  // 0: no such slots (fixed partitions, grid schedule).
  int max_pieces;
  int32_t *item_cnt;           // [num_seqs][num_kv_heads][row_tiles]
  // append in the same pass: the new tokens' K/V rows, [total_q, num_kv_heads, head_dim] packed like
  // q; NULL when nothing is appended
  const void *new_k;
  const void *new_v;
};

// Read-once decode over shared prefixes: groups of consecutive sequences whose first tokens sit in
// the group's shared physical blocks.
constexpr int kPrefixRows = 32;   // rows per prefix wave: two 16-row matrix-core tiles
struct PrefixArgs {
  const int32_t *group_starts;   // [num_groups + 1]
  const int32_t *prefix_lens;    // [num_groups]
  const int32_t *prefix_blocks;  // [num_groups, max_prefix_len / 16]
  int num_groups;
  int max_group_size;
  int max_prefix_len;            // a multiple of 16
  int rows_max;                  // max_group_size * max_q_len * G
  int row_tiles;                 // ceil(rows_max / 32)
  int chunk_pages;
  int chunks;                    // ceil(max_prefix_len / 16 / chunk_pages)
  int32_t *skip;                 // [num_seqs]: P_s
  int32_t *sfx_ctx;              // [num_seqs]: context_lens - P_s
  int32_t *sfx_table;            // [num_seqs, sfx_stride]
  int sfx_stride;                // ceil(max_context_len / 16)
  const int32_t *q_start;        // NULL: s * max_q_len
  float *sfx_lse;                // [total_q, H]: the suffix pass's natural-log LSE when the caller wants none
  float *pre_o;                  // [items * 32, D]
  float *pre_lse;                // [items * 32], log2
};

// Per-unit sequence facts with the clamps that keep bad metadata memory-safe.
struct SeqInfo {
  int ctx;      // context length, clamped to the table width and max_context_len
  int qs;       // new tokens, clamped to [1, ctx]
  int qbase;    // first packed q row
  int nparts;   // partitions this sequence spans
};

__device__ __forceinline__ SeqInfo load_seq(const DecodeArgs &a, int s) {
  SeqInfo si;
  int ctx = a.context_lens[s];
  ctx = min(ctx, a.max_context_len);
  ctx = min(ctx, a.max_blocks_per_seq * 16);
  si.ctx = max(ctx, 0);
  int qs = a.q_lens ? a.q_lens[s] : a.max_q_len;
  si.qs = max(1, min(qs, si.ctx));
  si.qbase = a.q_start ? a.q_start[s] : s * a.max_q_len;
  si.nparts = (si.ctx + a.part_size - 1) / a.part_size;
  return si;
}

// Group g's prefix in whole pages, within max_prefix_len.
__device__ __forceinline__ int prefix_tokens(const PrefixArgs &p, int g) {
  return min(max(p.prefix_lens[g], 0), p.max_prefix_len) / 16 * 16;
}

// Group holding sequence s (the last g with starts[g] <= s, if s < starts[num_groups]) and its
// clamped bounds; -1 when s is in no group or past the group's first max_group_size members.
__device__ __forceinline__ int group_of(const DecodeArgs &a, const PrefixArgs &p, int s, int &gs, int &pg) {
  const int S = a.num_seqs;
  auto start = [&](int g) { return min(max(p.group_starts[g], 0), S); };
  if (p.num_groups <= 0 || s < start(0) || s >= start(p.num_groups)) return -1;
  int g0 = 0, g1 = p.num_groups;
  while (g1 - g0 > 1) {
    const int mid = (g0 + g1) >> 1;
    if (start(mid) <= s) g0 = mid;
    else g1 = mid;
  }
  gs = start(g0);
  if (s - gs >= p.max_group_size) return -1;
  pg = prefix_tokens(p, g0);
  return g0;
}

// Shared length of sequence s: the group's prefix, cut to the whole pages before its new tokens.
__device__ __forceinline__ int shared_len(const SeqInfo &si, int pg) {
  return min(pg, (si.ctx - si.qs) / 16 * 16);
}

// The balanced schedule's page stream: for each kv head, for each sequence, for each row tile, a work
// item of C = item_cost virtual pages (the time a wave loses restarting its page pipeline on a new
// item) followed by the sequence's pages in logical order; a sequence with no pages has empty items.
// Kv head kvh's part starts at kvh * I (I = stream pages per kv head, so L = I * num_kv_heads in
// all).  Share `ord` of the NW = 8 W waves starts at floor(L ord / NW); ord = x * W + wx is wave wx
// of XCD x, so each XCD takes one contiguous eighth of the stream.  A boundary that falls in an
// item's virtual pages moves to the item's start; one that falls on its real pages moves down to a
// multiple of cut_align pages from the first of them (1 when no partitions are asked for), so a
// share starts where its ring cycles can, or at an item start when that multiple is 0.
// L ord < 2^53, so the double quotient has the exact floor: it is correctly rounded, and an integer
// quotient is representable.
__device__ __forceinline__ int64_t share_raw(int64_t L, int NW, int ord) {
  return (int64_t)floor((double)L * (double)ord / (double)NW);
}

// Smallest share whose raw start lies above pos (NW when none does, pos >= 0).  floor(L c / NW) > pos
// exactly when L c >= (pos + 1) NW = t, so the answer is ceil(t / L) when t < L NW.  There t / L < NW
// <= 2^13, and the single-precision quotient (three roundings, each within 2^-24 relative) is within
// 2^-9 of it: its integer part is at most two below the answer and never above it.  Exact integer
// products settle it (the downward step only guards that bound).
__device__ __forceinline__ int first_share_above(int64_t L, int NW, int64_t pos) {
  const int64_t t = (pos + 1) * NW;
  if (t >= L * NW) return NW;
  int c = min(max((int)((float)t / (float)L), 0), NW);
  while ((int64_t)c * L < t) ++c;
  while (c > 0 && (int64_t)(c - 1) * L >= t) --c;
  return c;
}

// Piece index, within its work item, of the piece that share o starts inside the item's real pages
// (no fixed partitions).  The item occupies stream [pos0, pos0 + C + nblk); piece 0 starts at the
// item's start.  When every share holds at least one page of stream (L >= NW), every share whose raw
// start lies past the item's C virtual pages starts one more piece, so share o's piece is o minus the
// first such share, plus one.  Otherwise shares can be empty, and cap is returned: those pieces take
// their wave's spill rows and the merge searches for them.  The result is capped at cap.
__device__ __forceinline__ int piece_index(int64_t L, int NW, int C, int64_t pos0, int o, int cap) {
  if (L < NW) return cap;
  return min(o - first_share_above(L, NW, pos0 + C) + 1, cap);
}

// Workgroup-wave slot of share ord: workgroup (wx / 4) * 8 + x, wave wx % 4.
__device__ __forceinline__ int share_slot(int W, int ord) {
  const int x = ord / W;
  const int wx = ord - x * W;
  return (((wx >> 2) << 3) + x) * 4 + (wx & 3);
}

}  // namespace pkv
