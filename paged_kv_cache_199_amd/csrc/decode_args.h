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
  float scale_log2;            // scale * log2(e): scores live in log2 units
  int part_size;               // keys per partition
  int num_parts;               // ceil(max_context_len / part_size)
  int row_tiles;               // row tiles per (sequence, kv head)
  int units;                   // num_kv_heads * num_parts * num_seqs * row_tiles
  int per_xcd;                 // ceil(units / 8)
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

}  // namespace pkv
