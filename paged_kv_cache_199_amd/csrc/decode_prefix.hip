// Read-once decode over a shared prefix.
//
// The lfm25-inference page reuses the KV blocks of a common prompt prefix across requests through its
// radix tree ("Runtime Design"), and decodes long contexts with a split-K pass merged by log-sum-exp.
// When several sequences of a batch hold the same physical blocks for their first P tokens, the keys
// of those blocks can be attended once for all of them: softmax attention over a key set splits into
// any partition of the keys, each part leaving (o_part, lse_part), merged exactly by the same rule
// the split-K combine uses.  Here the parts are the group's shared prefix (attended once, with the
// query rows of every member of the group stacked into one matrix-core tile set) and each
// sequence's own suffix (attended by the ordinary paged decode over a block table that starts after
// the prefix).  The group's shared block ids come in their own table, so no member has to hold the
// whole prefix.
//
//   prep:   per sequence, its shared length P_s (whole pages before its new tokens), the suffix
//           block-table row and suffix context length (extra workgroups of the prefix launch).
//   prefix: one wave per (group, kv head, page chunk, 32-row tile); rows = the group's members x new
//           tokens x the G query heads of the kv head.  Over bf16 pools the four waves of a
//           workgroup are four row tiles of one chunk and read its pages from LDS, staged once
//           (lds_pages.h); over E4M3 pools each wave streams and widens its pages itself.  Each wave
//           leaves an fp32 partial row and its log2 LSE.
//   merge:  in the suffix pass's split-K combine (decode_combine.hip): each row's suffix result
//           merged with its prefix chunks by the same log-sum-exp rule.
#include "decode_args.h"
#include "device_common.h"
#include "lds_pages.h"

namespace pkv {

// One wave per sequence: P_s, the suffix row of the block table and the suffix length.
__device__ __forceinline__ void prefix_prep(const DecodeArgs &a, const PrefixArgs &p, int s, int lane) {
  if (s >= a.num_seqs) return;
  const SeqInfo si = load_seq(a, s);
  int gs = 0, pg = 0;
  const int g = group_of(a, p, s, gs, pg);
  const int ps = g >= 0 ? max(shared_len(si, pg), 0) : 0;
  const int skip_pages = ps / kBlock;
  const int pages = (si.ctx - ps + kBlock - 1) / kBlock;
  const int32_t *src = a.block_tables + (int64_t)s * a.max_blocks_per_seq + skip_pages;
  int32_t *dst = p.sfx_table + (int64_t)s * p.sfx_stride;
  for (int j = lane; j < pages; j += 64) dst[j] = src[j];
  if (lane == 0) {
    p.skip[s] = ps;
    p.sfx_ctx[s] = si.ctx - ps;
  }
}

// The rows of row tile rt (32 rows) of group g for kv head kvh: member m, new token i, head offset
// hg in member-major order; a row sees prefix keys < P_s.  Returns the fewest and the most visible
// keys minus one over the tile's live rows (INT_MAX / -1 when it has none).
template <int D, int NT>
__device__ __forceinline__ void prefix_rows(const DecodeArgs &a, const PrefixArgs &p, int gs, int members, int pg,
                                            int kvh, int rt, int col, int grp, WaveRows<D, NT> &w, int &lowest,
                                            int &highest) {
  const int G = a.group;
  const int Qm = a.max_q_len;
  lowest = 0x7fffffff;
  highest = -1;
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int gr = rt * kPrefixRows + n * 16 + col;
    const int m = gr / (Qm * G);
    const int rem = gr - m * Qm * G;
    const int i = rem / G;
    const int hg = rem - i * G;
    int last = -1, qrow = 0;
    if (gr < p.rows_max && m < members) {
      const int s = gs + m;
      const SeqInfo si = load_seq(a, s);
      qrow = (p.q_start ? p.q_start[s] : s * Qm) + i;
      const int ps = shared_len(si, pg);
      if (i < si.qs && qrow < a.total_q && ps > 0) last = ps - 1;
    }
    w.last[n] = last;
    w.orow[n] = qrow * a.num_heads + kvh * G + hg;
    const char *qp = static_cast<const char *>(a.q) + (int64_t)w.orow[n] * (D * 2);
    #pragma unroll
    for (int k = 0; k < WaveRows<D, NT>::NK; ++k) {
      const uint4 v = last >= 0 ? ld16(qp + (4 * k + grp) * 16) : make_uint4(0, 0, 0, 0);
      w.qB[n][k] = __builtin_bit_cast(bf16x8_t, v);
    }
    if (last >= 0) {
      lowest = min(lowest, last);
      highest = max(highest, last);
    }
  }
  for (int o = 1; o < 64; o <<= 1) {
    lowest = min(lowest, __shfl_xor(lowest, o));
    highest = max(highest, __shfl_xor(highest, o));
  }
  w.first_last = lowest;
}

// The prefix as one sequence of pg tokens (every page in it is full).
__device__ __forceinline__ SeqInfo prefix_seq(int pg) {
  SeqInfo si;
  si.ctx = pg;
  si.qs = 1;
  si.qbase = 0;
  si.nparts = 1;
  return si;
}

// bf16 pools.  Workgroups [0, item_wgs) run the shared pass, one per (group, kv head, chunk, block of
// four row tiles): the chunk's pages go through LDS once for the four waves (lds_pages.h).  The
// workgroups after them build the suffix tables.
// D = 128: pages reach LDS through gfx950's global-to-LDS loads (lds_pages.h), faster on a
// 64-sequence, 4096-token prefix than staging through registers (2-page stages: 1.6%; 4-page stages
// at one workgroup per CU: 66.5 -> 65.3 us more).  Limiting the kernel to three waves per SIMD there
// spills and is 4-6% slower.
template <int D>
__global__ __launch_bounds__(256) void prefix_attend_lds_kernel(DecodeArgs a, PrefixArgs p, int item_wgs) {
  constexpr int NT = kPrefixRows / 16;
  constexpr bool DMA = D == 128;
  constexpr int SP = 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // the shared-pass workgroups are padded to a multiple of 8 and spread over the XCDs in contiguous
  // ranges (xcd_unit), so the row blocks of one chunk, which read the same pages, share an L2
  const int per_xcd = (item_wgs + 7) / 8;
  if ((int)blockIdx.x >= 8 * per_xcd) {
    prefix_prep(a, p, ((int)blockIdx.x - 8 * per_xcd) * 4 + wave, lane);
    return;
  }
  const int RT = p.row_tiles;
  const int RB = (RT + 3) / 4;
  const int C = p.chunks;
  const int KVH = a.num_kv_heads;
  // workgroup = ((g * KVH + kvh) * C + c) * RB + rb: the row blocks of one chunk are neighbours
  const int wi = xcd_unit(blockIdx.x, per_xcd);
  if (wi >= item_wgs) return;
  const int rb = wi % RB;
  const int c = (wi / RB) % C;
  const int kvh = (wi / (RB * C)) % KVH;
  const int g = wi / (RB * C * KVH);
  const int S = a.num_seqs;
  const int gs = min(max(p.group_starts[g], 0), S);
  const int ge = min(max(p.group_starts[g + 1], gs), S);
  const int members = min(ge - gs, p.max_group_size);
  const int pg = prefix_tokens(p, g);
  const int jb = c * p.chunk_pages;
  const int je = min(jb + p.chunk_pages, pg / kBlock);
  if (members <= 0 || jb >= je) return;   // the whole workgroup

  const int rt = rb * 4 + wave;
  WaveRows<D, NT> w;
  int lowest = 0x7fffffff, highest = -1;
  if (rt < RT) prefix_rows<D, NT>(a, p, gs, members, pg, kvh, rt, lane & 15, lane >> 4, w, lowest, highest);
  const bool live = highest >= 0;
  // this wave's pages: up to its rows' last visible key
  const int jw = live ? min(je, highest / kBlock + 1) : jb;
  WaveAcc<D, NT> st;
  init_acc<D, NT>(st);
  const int32_t *bt_row = p.prefix_blocks + (int64_t)g * (p.max_prefix_len / kBlock);
  DecodeArgs ap = a;
  ap.part_o = p.pre_o;
  ap.part_lse = p.pre_lse;
  if constexpr (DMA) {
    __shared__ __attribute__((aligned(16))) char buf0[DmaPages<SP>::BYTES];
    __shared__ __attribute__((aligned(16))) char buf1[DmaPages<SP>::BYTES];
    lds_stream_pages_dma<NT, SP>(ap, prefix_seq(pg), kvh, bt_row, jb, je, jw, buf0, buf1, w, st);
  } else {
    __shared__ __attribute__((aligned(16))) char lds[LdsPages<D, SP>::BYTES];
    lds_stream_pages<D, NT, SP>(ap, prefix_seq(pg), kvh, bt_row, jb, je, jw, lds, w, st);
  }
  const int64_t item = (((int64_t)g * KVH + kvh) * C + c) * RT + rt;
  if (live) finish_wave<D, NT>(ap, 0, false, lane, w, st, item * kPrefixRows);
}

// E4M3 pools: one wave per (group, kv head, chunk, row tile), pages widened in registers.
template <int D, int NBUF>
__global__ __launch_bounds__(256) void prefix_attend_f8_kernel(DecodeArgs a, PrefixArgs p, int item_wgs) {
  constexpr int NT = kPrefixRows / 16;
  const int lane = threadIdx.x & 63;
  if ((int)blockIdx.x >= item_wgs) {
    prefix_prep(a, p, ((int)blockIdx.x - item_wgs) * 4 + (threadIdx.x >> 6), lane);
    return;
  }
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int RT = p.row_tiles;
  const int C = p.chunks;
  const int KVH = a.num_kv_heads;
  if (item >= (int64_t)p.num_groups * KVH * C * RT) return;
  // item = ((g * KVH + kvh) * C + c) * RT + rt: the row tiles of one chunk are neighbours
  const int rt = (int)(item % RT);
  const int c = (int)((item / RT) % C);
  const int kvh = (int)((item / ((int64_t)RT * C)) % KVH);
  const int g = (int)(item / ((int64_t)RT * C * KVH));
  const int S = a.num_seqs;
  const int gs = min(max(p.group_starts[g], 0), S);
  const int ge = min(max(p.group_starts[g + 1], gs), S);
  const int members = min(ge - gs, p.max_group_size);
  const int pg = prefix_tokens(p, g);
  const int jb = c * p.chunk_pages;
  const int je = min(jb + p.chunk_pages, pg / kBlock);
  if (members <= 0 || jb >= je) return;

  WaveRows<D, NT> w;
  int lowest, highest;
  prefix_rows<D, NT>(a, p, gs, members, pg, kvh, rt, lane & 15, lane >> 4, w, lowest, highest);
  if (highest < 0) return;   // no live row in this tile
  WaveAcc<D, NT> st;
  init_acc<D, NT>(st);
  const int32_t *bt_row = p.prefix_blocks + (int64_t)g * (p.max_prefix_len / kBlock);
  DecodeArgs ap = a;
  ap.part_o = p.pre_o;
  ap.part_lse = p.pre_lse;
  stream_pages<D, NT, NBUF, true>(
      ap, prefix_seq(pg), kvh, bt_row, jb, je, 1 << 30, lane, w, st,
      [&](int, int, int) { finish_wave<D, NT>(ap, 0, false, lane, w, st, item * kPrefixRows); },
      [&](int, uint4 *, uint2 *) {}, [] {});
}

hipError_t launch_prefix_attend(const DecodeArgs &a, const PrefixArgs &p, int head_dim, bool f8, hipStream_t st) {
  const int64_t tiles = p.chunks > 0 ? (int64_t)p.num_groups * a.num_kv_heads * p.chunks : 0;
  // bf16: a workgroup per four row tiles; E4M3: a wave per row tile
  const int item_wgs = (int)(f8 ? (tiles * p.row_tiles + 3) / 4 : tiles * ((p.row_tiles + 3) / 4));
  const int prep_wgs = (a.num_seqs + 3) / 4;
  const dim3 grid((unsigned)(item_wgs + prep_wgs));
  const dim3 grid_lds((unsigned)(8 * ((item_wgs + 7) / 8) + prep_wgs));   // shared pass padded for xcd_unit
  if (head_dim == 64) {
    if (f8) prefix_attend_f8_kernel<64, 2><<<grid, 256, 0, st>>>(a, p, item_wgs);
    else prefix_attend_lds_kernel<64><<<grid_lds, 256, 0, st>>>(a, p, item_wgs);
  } else {
    if (f8) prefix_attend_f8_kernel<128, 2><<<grid, 256, 0, st>>>(a, p, item_wgs);
    else prefix_attend_lds_kernel<128><<<grid_lds, 256, 0, st>>>(a, p, item_wgs);
  }
  return hipGetLastError();
}

}  // namespace pkv
