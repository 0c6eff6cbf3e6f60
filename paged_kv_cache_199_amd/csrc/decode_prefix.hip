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
//   merge:  per (sequence, new token, head): the suffix result (already in out, with a natural-log
//           LSE) merged with the row's prefix chunks.
#include "decode_args.h"
#include "device_common.h"
#include "lds_pages.h"

namespace pkv {

// Group g's prefix in whole pages, within max_prefix_len.
__device__ __forceinline__ int prefix_tokens(const PrefixArgs &p, int g) {
  return min(max(p.prefix_lens[g], 0), p.max_prefix_len) / kBlock * kBlock;
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
  return min(pg, (si.ctx - si.qs) / kBlock * kBlock);
}

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
template <int D>
__global__ __launch_bounds__(256) void prefix_attend_lds_kernel(DecodeArgs a, PrefixArgs p, int item_wgs) {
  constexpr int NT = kPrefixRows / 16;
  constexpr int SP = 4;
  __shared__ __attribute__((aligned(16))) char lds[LdsPages<D, SP>::BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if ((int)blockIdx.x >= item_wgs) {
    prefix_prep(a, p, ((int)blockIdx.x - item_wgs) * 4 + wave, lane);
    return;
  }
  const int RT = p.row_tiles;
  const int RB = (RT + 3) / 4;
  const int C = p.chunks;
  const int KVH = a.num_kv_heads;
  // workgroup = ((g * KVH + kvh) * C + c) * RB + rb: the row blocks of one chunk are neighbours
  const int wi = blockIdx.x;
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
  lds_stream_pages<D, NT, SP>(ap, prefix_seq(pg), kvh, bt_row, jb, je, jw, lds, w, st);
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
      [&](int, uint4 *, uint2 *) {});
}

// One wave per (sequence, new token, head).  The row's chunk LSEs are read at once (lane c holds chunk
// c; the plan keeps chunks <= 64), their max and weight sum are wave reductions, and the partial rows
// stream with the weights broadcast from the lanes that hold them, eight loads in flight.
template <int D>
__global__ __launch_bounds__(256) void prefix_merge_kernel(DecodeArgs a, PrefixArgs p) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = a.num_heads;
  if (wid >= (int64_t)a.num_seqs * a.max_q_len * H) return;
  const int h = (int)(wid % H);
  const int i = (int)((wid / H) % a.max_q_len);
  const int s = (int)(wid / ((int64_t)H * a.max_q_len));
  const SeqInfo si = load_seq(a, s);
  if (i >= si.qs) return;
  const int qrow = (p.q_start ? p.q_start[s] : s * a.max_q_len) + i;
  if (qrow >= a.total_q) return;
  const int64_t orow = (int64_t)qrow * H + h;
  const int G = a.group;
  const int kvh = h / G;
  const int hg = h - kvh * G;
  int gs = 0, pg = 0;
  const int g = group_of(a, p, s, gs, pg);
  const int ps = g >= 0 ? shared_len(si, pg) : 0;
  const int nc = min((ps / kBlock + p.chunk_pages - 1) / p.chunk_pages, p.chunks);   // chunks with keys < P_s
  const int gr = ((s - gs) * a.max_q_len + i) * G + hg;
  const float lse_s = p.sfx_lse[orow];
  if (nc <= 0 || gr >= p.rows_max) {
    // no shared keys: the suffix pass's result is the answer
    if (lane == 0 && a.lse) a.lse[orow] = lse_s;
    return;
  }
  const int rt = gr / kPrefixRows;
  const int64_t prow0 = ((((int64_t)g * a.num_kv_heads + kvh) * p.chunks) * p.row_tiles + rt) * kPrefixRows +
                        (gr - rt * kPrefixRows);
  const int64_t cstride = (int64_t)p.row_tiles * kPrefixRows;    // between chunks of one row
  const float l2s = lse_s * kLog2e;
  const float l = lane < nc ? p.pre_lse[prow0 + lane * cstride] : -INFINITY;
  const float mx = fmaxf(wave_max(l), l2s);
  const float wl = exp2_hw(l - mx);                               // 0 on lanes past nc
  const float ws = exp2_hw(l2s - mx);
  const float wsum = wave_sum(wl) + ws;
  uint16_t *out = static_cast<uint16_t *>(a.out) + orow * D + lane * DPL;
  float acc[DPL];
  #pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = ws * __uint_as_float((uint32_t)out[e] << 16);
  const float *po = p.pre_o + prow0 * D + lane * DPL;
  for (int c0 = 0; c0 < nc; c0 += 8) {
    float v[8][DPL];
    #pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = min(c0 + u, nc - 1);
      #pragma unroll
      for (int e = 0; e < DPL; ++e) v[u][e] = po[c * cstride * D + e];
    }
    #pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wc = c0 + u < nc ? __shfl(wl, c0 + u) : 0.f;
      #pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += wc * v[u][e];
    }
  }
  const float inv = 1.f / wsum;
  #pragma unroll
  for (int e = 0; e < DPL; ++e) out[e] = f32_to_bf16(acc[e] * inv);
  if (lane == 0 && a.lse) a.lse[orow] = (mx + log2_hw(wsum)) * kLn2;
}

hipError_t launch_prefix_attend(const DecodeArgs &a, const PrefixArgs &p, int head_dim, bool f8, hipStream_t st) {
  const int64_t tiles = p.chunks > 0 ? (int64_t)p.num_groups * a.num_kv_heads * p.chunks : 0;
  // bf16: a workgroup per four row tiles; E4M3: a wave per row tile
  const int item_wgs = (int)(f8 ? (tiles * p.row_tiles + 3) / 4 : tiles * ((p.row_tiles + 3) / 4));
  const dim3 grid((unsigned)(item_wgs + (a.num_seqs + 3) / 4));
  if (head_dim == 64) {
    if (f8) prefix_attend_f8_kernel<64, 2><<<grid, 256, 0, st>>>(a, p, item_wgs);
    else prefix_attend_lds_kernel<64><<<grid, 256, 0, st>>>(a, p, item_wgs);
  } else {
    if (f8) prefix_attend_f8_kernel<128, 2><<<grid, 256, 0, st>>>(a, p, item_wgs);
    else prefix_attend_lds_kernel<128><<<grid, 256, 0, st>>>(a, p, item_wgs);
  }
  return hipGetLastError();
}

hipError_t launch_prefix_merge(const DecodeArgs &a, const PrefixArgs &p, int head_dim, hipStream_t st) {
  const int64_t waves = (int64_t)a.num_seqs * a.max_q_len * a.num_heads;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (head_dim == 64) prefix_merge_kernel<64><<<grid, 256, 0, st>>>(a, p);
  else prefix_merge_kernel<128><<<grid, 256, 0, st>>>(a, p);
  return hipGetLastError();
}

}  // namespace pkv
