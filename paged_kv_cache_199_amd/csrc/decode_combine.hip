// Split-K merge and ragged-q bookkeeping for paged decode.
//
// The lfm25-inference page ("Runtime Design") decodes long contexts with a split-K reduction.  Each
// partition p of a row leaves a softmax over its own keys, o_p, and its log-sum-exp, lse_p.  The
// merged row is  out = sum_p w_p o_p / sum_p w_p  with  w_p = exp(lse_p - max_p lse_p), and
// lse = max + log(sum_p w_p); a partition in which the row saw no key has lse_p = -inf and weight 0
// (exp2 of -inf is 0, so it needs no special case).
#include "decode_args.h"
#include "device_common.h"

namespace pkv {

typedef float float4_v __attribute__((ext_vector_type(4)));

// One wave per (sequence, new token, head); partial LSEs are in log2 units.  The sources of a row are
// its partitions and, under the balanced schedule, the spill rows of the shares that start inside
// the row's work item.  The LSEs of up to 64 sources are read at once (one per lane), their max and
// weight sum are wave reductions, and the weights and row offsets are broadcast from the lane that
// holds them, so the partial outputs stream with several loads in flight instead of one dependent
// load per source.
//
// PRE (read-once shared-prefix decode): this pass attended each sequence's keys past its shared
// prefix; a row whose sequence shares a prefix is then merged, by the same rule, with the prefix
// pass's chunk partials (p.pre_o / p.pre_lse), whether its own result came out of this merge or was
// already final in out / lse.
template <int D>
__device__ __forceinline__ void merge_prefix_chunks(const DecodeArgs &a, const PrefixArgs &p, int64_t base, int lane,
                                                    const float *o_s, float l2s, int nc, int64_t crow0,
                                                    int64_t cstride) {
  constexpr int DPL = D / 64;
  const float l = lane < nc ? p.pre_lse[crow0 + lane * cstride] : -INFINITY;
  const float mx = fmaxf(wave_max(l), l2s);
  const float wl = exp2_hw(l - mx);                         // 0 on lanes past nc
  const float ws = exp2_hw(l2s - mx);
  const float wsum = wave_sum(wl) + ws;
  float acc[DPL];
  #pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = ws * o_s[k];
  const float *po = p.pre_o + crow0 * D + lane;
  for (int c0 = 0; c0 < nc; c0 += 8) {
    float v[8][DPL];
    #pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = min(c0 + u, nc - 1);
      #pragma unroll
      for (int k = 0; k < DPL; ++k) v[u][k] = po[c * cstride * D + 64 * k];
    }
    #pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wc = c0 + u < nc ? __shfl(wl, c0 + u) : 0.f;
      #pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wc, v[u][k], acc[k]);
    }
  }
  const float inv = 1.f / wsum;
  uint16_t *out = static_cast<uint16_t *>(a.out) + base * D + lane;
  #pragma unroll
  for (int k = 0; k < DPL; ++k) out[64 * k] = f32_to_bf16(acc[k] * inv);
  if (lane == 0 && a.lse) a.lse[base] = (mx + log2_hw(wsum)) * kLn2;
}

// With piece slots on and the same number of new tokens in every sequence, a row's position and its
// work item follow from (s, i, h) alone, and its first pieces sit in partition rows 0 .. max_pieces - 1:
// the item's piece count and the partials of all its slots are requested before any of them returns,
// one round trip where the general merge takes two (the lengths, then the sources).  The slots past
// the count are read for nothing; with few rows that costs less than waiting for the count first
// (measured on the concurrency-32, shared-prefix and E4M3 batches).  Returns false when the item has
// more pieces than NS (the general merge takes over).
template <bool BF16, int D, int NS>
__device__ __forceinline__ bool merge_slots(const DecodeArgs &a, int s, int i, int h, int lane) {
  constexpr int DPL = D / 64;
  const int H = a.num_heads;
  const int G = a.group;
  const int kvh = h / G;
  const int rt = (i * G + h - kvh * G) / a.rows_per_tile;
  const int row = s * a.max_q_len + i;
  const int64_t stride = (int64_t)a.total_q * H;
  const int64_t base = (int64_t)row * H + h;
  const int mp = a.max_pieces;
  const int ctx_raw = a.context_lens[s];
  const int cnt = a.item_cnt[((int64_t)s * a.num_kv_heads + kvh) * a.row_tiles + rt];
  const float l = lane < mp && lane < NS ? a.part_lse[lane * stride + base] : -INFINITY;
  float v[NS][DPL];
  #pragma unroll
  for (int u = 0; u < NS; ++u) {
    const float *op = a.part_o + ((int64_t)u * stride + base) * D + lane;
    #pragma unroll
    for (int k = 0; k < DPL; ++k) v[u][k] = u < mp ? op[64 * k] : 0.f;
  }
  // the row's validity, clamped as the partition pass clamps it
  int ctx = min(min(ctx_raw, a.max_context_len), a.max_blocks_per_seq * kBlock);
  ctx = max(ctx, 0);
  const int qs = max(1, min(a.max_q_len, ctx));
  if (i >= qs || ctx <= 0 || row >= a.total_q) return true;
  if (cnt <= 1) return true;                // one piece: the partition pass wrote the final row
  if (cnt > NS || cnt > mp) return false;
  const float ls = lane < cnt ? l : -INFINITY;
  const float M = wave_max(ls);
  const float Ms = M == -INFINITY ? 0.f : M;
  const float wl = ls == -INFINITY ? 0.f : exp2_hw(ls - Ms);
  float acc[DPL];
  #pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  #pragma unroll
  for (int u = 0; u < NS; ++u) {
    const float wp = __shfl(wl, u);
    #pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = u < cnt ? fmaf(wp, v[u][k], acc[k]) : acc[k];   // slots past cnt hold anything
  }
  const float L2 = wave_sum(wl);
  const bool seen = L2 > 0.f;
  const float inv = seen ? 1.f / L2 : 0.f;
  #pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const float o = acc[k] * inv;
    if constexpr (BF16) {
      static_cast<uint16_t *>(a.out)[base * D + lane + 64 * k] = f32_to_bf16(o);
    } else {
      static_cast<float *>(a.out)[base * D + lane + 64 * k] = o;
    }
  }
  if (lane == 0 && a.lse) a.lse[base] = seen ? (Ms + log2_hw(L2)) * kLn2 : -INFINITY;
  return true;
}

template <bool BF16, int D, bool PRE, int NS = 0>
__device__ __forceinline__ void combine_row(const DecodeArgs &a, const PrefixArgs &p, int s, int i, int h, int lane) {
  constexpr int DPL = D / 64;
  const int H = a.num_heads;
  if constexpr (NS > 0 && !PRE) {
    if (merge_slots<BF16, D, NS>(a, s, i, h, lane)) return;
  }
  // issued before the sequence's lengths come back: they do not depend on them
  const bool spill = a.spill_base >= 0;
  const int pre_s = spill ? a.item_pre[s] : 0;
  const int pre_all = spill ? a.item_pre[a.num_seqs] : 0;
  const SeqInfo si = load_seq(a, s);
  if (i >= si.qs || si.ctx <= 0) return;
  const int row = si.qbase + i;
  if (row >= a.total_q) return;
  const int64_t stride = (int64_t)a.total_q * H;          // between partitions
  const int64_t base = (int64_t)row * H + h;
  // read-once decode: the prefix chunks this row merges (none when its sequence shares nothing)
  int nc = 0;
  int64_t crow0 = 0, cstride = 0;
  if constexpr (PRE) {
    int gs = 0, pg = 0;
    const int g = group_of(a, p, s, gs, pg);
    const int ps = g >= 0 ? p.skip[s] : 0;
    const int G = a.group;
    const int kvh = h / G;
    const int gr = ((s - gs) * a.max_q_len + i) * G + (h - kvh * G);
    if (ps > 0 && gr < p.rows_max && p.chunk_pages > 0) {
      nc = min((ps / kBlock + p.chunk_pages - 1) / p.chunk_pages, p.chunks);
      const int rt = gr / kPrefixRows;
      crow0 = ((((int64_t)g * a.num_kv_heads + kvh) * p.chunks) * p.row_tiles + rt) * kPrefixRows +
              (gr - rt * kPrefixRows);
      cstride = (int64_t)p.row_tiles * kPrefixRows;
    }
  }

  // shares that start inside this row's work item [pos0, pos1) of the balanced stream
  int ncand = 0, ord0 = 0, srow = 0;
  int64_t pos0 = 0, pos1 = 0, L = 0;
  const int W = a.share_waves;
  const int NW = 8 * W;
  const int N = a.cut_align;                              // 1, 2 or 4
  const int C = a.item_cost;                              // virtual pages at each item's start
  const int PP = a.part_size / kBlock;
  int nblk = 0;
  if (spill) {
    const int G = a.group;
    const int rloc = i * G + h % G;
    const int rt = rloc / a.rows_per_tile;
    srow = rloc - rt * a.rows_per_tile;
    nblk = (si.ctx + kBlock - 1) / kBlock;
    const int I = pre_all;
    L = (int64_t)I * a.num_kv_heads;
    pos0 = (int64_t)(h / G) * I + pre_s + (int64_t)rt * (nblk + C);
    pos1 = pos0 + nblk + C;
    ord0 = first_share_above(L, NW, pos0);
    ncand = max(0, first_share_above(L, NW, pos1 - 1) - ord0);
  }
  // source idx < nparts: partition idx; else candidate share ord0 + idx - nparts, a source when its
  // rounded start is inside the item, not on a partition start, and its share is not empty
  auto source = [&](int idx, int64_t &prow, bool &cut) -> bool {
    cut = false;
    if (idx < si.nparts) {
      prow = idx * stride + base;
      return true;
    }
    const int ord = ord0 + idx - si.nparts;
    // real page offset in the item where a raw share start lands (0: the item's start)
    auto real_off = [&](int64_t b) {
      const int ro = (int)(b - pos0) - C;
      return ro > 0 ? ro & ~(N - 1) : 0;
    };
    const int64_t b = share_raw(L, NW, ord);                // in (pos0, pos1)
    const int ob = real_off(b);
    if (ob <= 0) return false;
    cut = true;
    if (ob % PP == 0) return false;
    const int64_t bn = share_raw(L, NW, ord + 1);
    const int obn = bn < pos1 ? real_off(bn) : nblk;
    if (obn <= ob) return false;
    // piece slots on (then there is one partition): pieces below max_pieces sit in partition rows
    const int kp = a.max_pieces > 1 ? piece_index(L, NW, C, pos0, ord, a.max_pieces) : a.max_pieces;
    prow = kp < a.max_pieces ? kp * stride + base
                             : a.spill_base + (int64_t)share_slot(W, ord) * a.rows_per_tile + srow;
    return true;
  };
  const int nsrc = si.nparts + ncand;

  // whether the row needs a merge is arithmetic: decide it before any load of partials
  bool any_cut = false;
  for (int c0 = si.nparts; c0 < nsrc && !any_cut; c0 += 64) {
    int64_t prow = base;
    bool cut = false;
    if (c0 + lane < nsrc) source(c0 + lane, prow, cut);
    any_cut = __builtin_amdgcn_ballot_w64(cut) != 0;
  }
  // a row whose item one wave covered in one piece already holds its final output
  if (si.nparts <= 1 && !any_cut) {
    if constexpr (PRE) {
      if (nc > 0) {
        float o_s[DPL];
        const uint16_t *os = static_cast<const uint16_t *>(a.out) + base * D + lane;
        #pragma unroll
        for (int k = 0; k < DPL; ++k) o_s[k] = __uint_as_float((uint32_t)os[64 * k] << 16);
        merge_prefix_chunks<D>(a, p, base, lane, o_s, a.lse[base] * kLog2e, nc, crow0, cstride);
      }
    }
    return;
  }

  float acc[DPL];
  #pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  float L2 = 0.f;
  float Ms = 0.f;
  if (nsrc <= 16) {
    // the usual case: the LSEs and the partial rows of all sources are loaded together (the rows do
    // not depend on the weights), so the merge waits for memory once
    int64_t prow = base;   // a non-source lane points at partition 0's row (always written), weight 0
    bool cut = false;
    const bool ok = lane < nsrc && source(lane, prow, cut);
    const float l = ok ? a.part_lse[prow] : -INFINITY;
    const int lo = (int)prow;
    const int hi = (int)(prow >> 32);
    float v[16][DPL];
    #pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t pr = u < nsrc ? ((int64_t)__shfl(hi, u) << 32) | (uint32_t)__shfl(lo, u) : base;
      const float *op = a.part_o + pr * D + lane;
      #pragma unroll
      for (int k = 0; k < DPL; ++k) v[u][k] = op[64 * k];
    }
    const float M = wave_max(l);
    Ms = M == -INFINITY ? 0.f : M;
    const float wl = l == -INFINITY ? 0.f : exp2_hw(l - Ms);
    L2 = wl;
    #pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float wp = u < nsrc ? __shfl(wl, u) : 0.f;
      #pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wp, v[u][k], acc[k]);
    }
  } else {
    // many sources: max over all LSEs first, then the weighted rows in batches of 16
    float M = -INFINITY;
    int64_t prow0 = base;
    float lse0 = -INFINITY;
    for (int c0 = 0; c0 < nsrc; c0 += 64) {
      int64_t prow = base;
      bool cut = false;
      const bool ok = c0 + lane < nsrc && source(c0 + lane, prow, cut);
      const float l = ok ? a.part_lse[prow] : -INFINITY;
      if (c0 == 0) {
        prow0 = prow;
        lse0 = l;
      }
      M = fmaxf(M, l);
    }
    M = wave_max(M);
    Ms = M == -INFINITY ? 0.f : M;
    for (int c0 = 0; c0 < nsrc; c0 += 64) {
      int64_t prow = prow0;
      float l = lse0;
      if (c0 > 0) {
        bool cut = false;
        prow = base;
        l = c0 + lane < nsrc && source(c0 + lane, prow, cut) ? a.part_lse[prow] : -INFINITY;
      }
      const float wl = l == -INFINITY ? 0.f : exp2_hw(l - Ms);
      L2 += wl;
      const int lo = (int)prow;
      const int hi = (int)(prow >> 32);
      const int n = min(64, nsrc - c0);
      for (int j = 0; j < n; j += 16) {
        float v[16][DPL];
        #pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int src = min(j + u, 63);
          const int64_t pr = j + u < n ? ((int64_t)__shfl(hi, src) << 32) | (uint32_t)__shfl(lo, src) : base;
          const float *op = a.part_o + pr * D + lane;
          #pragma unroll
          for (int k = 0; k < DPL; ++k) v[u][k] = op[64 * k];
        }
        #pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float wp = j + u < n ? __shfl(wl, min(j + u, 63)) : 0.f;
          #pragma unroll
          for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wp, v[u][k], acc[k]);
        }
      }
    }
  }
  L2 = wave_sum(L2);
  const bool seen = L2 > 0.f;
  const float inv = seen ? 1.f / L2 : 0.f;
  if constexpr (PRE) {
    if (nc > 0) {
      float o_s[DPL];
      #pragma unroll
      for (int k = 0; k < DPL; ++k) o_s[k] = acc[k] * inv;
      merge_prefix_chunks<D>(a, p, base, lane, o_s, seen ? Ms + log2_hw(L2) : -INFINITY, nc, crow0, cstride);
      return;
    }
  }
  #pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const float o = acc[k] * inv;
    if constexpr (BF16) {
      static_cast<uint16_t *>(a.out)[base * D + lane + 64 * k] = f32_to_bf16(o);
    } else {
      static_cast<float *>(a.out)[base * D + lane + 64 * k] = o;
    }
  }
  if (lane == 0 && a.lse) a.lse[base] = seen ? (Ms + log2_hw(L2)) * kLn2 : -INFINITY;
}

// NS > 0: piece slots on and uniform new tokens; the first NS slots are read in the first round trip.
template <bool BF16, int D, bool PRE, int NS>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a, PrefixArgs p) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int H = a.num_heads;
  const int64_t nw = (int64_t)a.num_seqs * a.max_q_len * H;
  if (wid >= nw) return;
  const int h = (int)(wid % H);
  const int64_t t = wid / H;
  combine_row<BF16, D, PRE, NS>(a, p, (int)(t / a.max_q_len), (int)(t % a.max_q_len), h, lane);
}

// The G rows' merge once the sources are known: lane j G + hg holds source j's log2 LSE l for head hg
// (-inf: not a source), v[u] this lane's E floats of source u's G x D block (anything past nsrc).
template <bool BF16, int D, int E>
__device__ __forceinline__ void group_merge(const DecodeArgs &a, int64_t base, int lane, float l,
                                            const float4_v v[][E / 4], int nsrc) {
  constexpr int G = E * 64 / D;
  constexpr int LG = G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : 4;
  const int e0 = lane * E;
  const int hgd = e0 / D;
  // per-head max and weight sum over the sources: lanes hg, hg + G, hg + 2G, ...
  float M = l;
  #pragma unroll
  for (int o = G; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float Ms = M == -INFINITY ? 0.f : M;
  const float wl = l == -INFINITY ? 0.f : exp2_hw(l - Ms);
  float S2 = wl;
  #pragma unroll
  for (int o = G; o < 64; o <<= 1) S2 += __shfl_xor(S2, o);
  float4_v acc[E / 4];
  #pragma unroll
  for (int k = 0; k < E / 4; ++k) acc[k] = float4_v{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
  for (int u = 0; u < 64 / G; ++u) {
    const float wp = __shfl(wl, (u << LG) + hgd);
    #pragma unroll
    for (int k = 0; k < E / 4; ++k) acc[k] = u < nsrc ? acc[k] + wp * v[u][k] : acc[k];
  }
  const float Sd = __shfl(S2, hgd);
  const float inv = Sd > 0.f ? 1.f / Sd : 0.f;
  #pragma unroll
  for (int k = 0; k < E / 4; ++k) {
    const float4_v o = acc[k] * inv;
    const int64_t off = base * D + e0 + 4 * k;
    if constexpr (BF16) {
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + off) =
          make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    } else {
      *reinterpret_cast<float4_v *>(static_cast<float *>(a.out) + off) = o;
    }
  }
  if (lane < G && a.lse) a.lse[base + lane] = S2 > 0.f ? (Ms + log2_hw(S2)) * kLn2 : -INFINITY;
}

// The same merge for the G query heads of one kv head at once: one wave per (sequence, new token, kv
// head).  Those G rows belong to the same work item (when they sit in one row tile), so they have the
// same sources, and their partial rows are G consecutive rows of every source: the wave finds the
// sources once, reads the G x sources LSEs one per lane, and streams each source's G x D block with
// E = G D / 64 consecutive floats per lane.  Rows that do not fit (sources x G > 64, or heads split
// over two row tiles) take the per-row merge.  With piece slots on and uniform new tokens the sources
// need no search: the item's piece count comes back with the sequence's length, and then only the
// slots it names are read (with this many rows, reading every slot up front costs more than the wait).
template <bool BF16, int D, int E>
__global__ __launch_bounds__(256) void combine_group_kernel(DecodeArgs a) {
  constexpr int G = E * 64 / D;             // heads per kv head, a power of two
  constexpr int LG = G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : 4;
  static_assert((1 << LG) == G, "G must be 2, 4, 8 or 16");
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int H = a.num_heads;
  const int KVH = a.num_kv_heads;
  const int64_t nw = (int64_t)a.num_seqs * a.max_q_len * KVH;
  if (wid >= nw) return;
  const int kvh = (int)(wid % KVH);
  const int64_t t = wid / KVH;
  const int i = (int)(t % a.max_q_len);
  const int s = (int)(t / a.max_q_len);
  const int rpt = a.rows_per_tile;
  const int rt = i * G / rpt;
  const bool one_tile = rt == (i * G + G - 1) / rpt;
  const int64_t stride = (int64_t)a.total_q * H;          // between partitions
  // lane = j G + hg: source j's LSE for head hg; this lane's E floats of each source's G x D block:
  // head hgd, dims d0 .. d0 + E - 1
  const int j = lane >> LG;
  const int hgl = lane & (G - 1);
  const int e0 = lane * E;
  float4_v v[64 / G][E / 4];
  if (a.max_pieces > 1 && !a.q_lens && one_tile) {
    const int row = s * a.max_q_len + i;
    const int64_t base = (int64_t)row * H + kvh * G;
    const int mp = a.max_pieces;
    const int ctx_raw = a.context_lens[s];
    const int cnt = a.item_cnt[((int64_t)s * KVH + kvh) * a.row_tiles + rt];
    const float l0 = j < mp ? a.part_lse[j * stride + base + hgl] : -INFINITY;
    int ctx = min(min(ctx_raw, a.max_context_len), a.max_blocks_per_seq * kBlock);
    ctx = max(ctx, 0);
    const int qs = max(1, min(a.max_q_len, ctx));
    if (i >= qs || ctx <= 0 || row >= a.total_q) return;
    if (cnt <= 1) return;                                 // one piece: the G rows are final already
    if (cnt <= mp && cnt <= 64 / G) {
      // many rows: the slots are read once the count is known, so no load is spent on unused ones
      #pragma unroll
      for (int u = 0; u < 64 / G; ++u) {
        const float4_v *op = reinterpret_cast<const float4_v *>(a.part_o + ((int64_t)u * stride + base) * D + e0);
        #pragma unroll
        for (int k = 0; k < E / 4; ++k) v[u][k] = u < cnt ? op[k] : float4_v{0.f, 0.f, 0.f, 0.f};
      }
      group_merge<BF16, D, E>(a, base, lane, j < cnt ? l0 : -INFINITY, v, cnt);
      return;
    }
  }
  const bool spill = a.spill_base >= 0;
  const int pre_s = spill ? a.item_pre[s] : 0;
  const int pre_all = spill ? a.item_pre[a.num_seqs] : 0;
  const SeqInfo si = load_seq(a, s);
  if (i >= si.qs || si.ctx <= 0) return;
  const int row = si.qbase + i;
  if (row >= a.total_q) return;
  const int64_t base = (int64_t)row * H + kvh * G;        // head kvh G + hg: row base + hg
  if (!one_tile) {                                        // heads split over two row tiles
    for (int hg = 0; hg < G; ++hg) combine_row<BF16, D, false>(a, PrefixArgs{}, s, i, kvh * G + hg, lane);
    return;
  }
  const int srow = i * G - rt * rpt;                      // head hg: spill row srow + hg

  int ncand = 0, ord0 = 0;
  int64_t pos0 = 0, pos1 = 0, L = 0;
  const int W = a.share_waves;
  const int NW = 8 * W;
  const int N = a.cut_align;
  const int C = a.item_cost;
  const int PP = a.part_size / kBlock;
  int nblk = 0;
  if (spill) {
    nblk = (si.ctx + kBlock - 1) / kBlock;
    const int I = pre_all;
    L = (int64_t)I * KVH;
    pos0 = (int64_t)kvh * I + pre_s + (int64_t)rt * (nblk + C);
    pos1 = pos0 + nblk + C;
    ord0 = first_share_above(L, NW, pos0);
    ncand = max(0, first_share_above(L, NW, pos1 - 1) - ord0);
  }
  // source idx: as in the per-row merge, with the row of head 0 (head hg adds hg)
  auto source = [&](int idx, int64_t &prow, bool &cut) -> bool {
    cut = false;
    if (idx < si.nparts) {
      prow = idx * stride + base;
      return true;
    }
    const int ord = ord0 + idx - si.nparts;
    auto real_off = [&](int64_t b) {
      const int ro = (int)(b - pos0) - C;
      return ro > 0 ? ro & ~(N - 1) : 0;
    };
    const int64_t b = share_raw(L, NW, ord);
    const int ob = real_off(b);
    if (ob <= 0) return false;
    cut = true;
    if (ob % PP == 0) return false;
    const int64_t bn = share_raw(L, NW, ord + 1);
    const int obn = bn < pos1 ? real_off(bn) : nblk;
    if (obn <= ob) return false;
    // piece slots on (then there is one partition): pieces below max_pieces sit in partition rows
    const int kp = a.max_pieces > 1 ? piece_index(L, NW, C, pos0, ord, a.max_pieces) : a.max_pieces;
    prow = kp < a.max_pieces ? kp * stride + base : a.spill_base + (int64_t)share_slot(W, ord) * rpt + srow;
    return true;
  };
  const int nsrc = si.nparts + ncand;
  bool any_cut = false;
  for (int c0 = si.nparts; c0 < nsrc && !any_cut; c0 += 64) {
    int64_t prow = base;
    bool cut = false;
    if (c0 + lane < nsrc) source(c0 + lane, prow, cut);
    any_cut = __builtin_amdgcn_ballot_w64(cut) != 0;
  }
  if (si.nparts <= 1 && !any_cut) return;                 // the G rows are final already
  if (nsrc * G > 64) {
    for (int hg = 0; hg < G; ++hg) combine_row<BF16, D, false>(a, PrefixArgs{}, s, i, kvh * G + hg, lane);
    return;
  }

  // a non-source points at partition 0's rows (always written) with weight 0
  int64_t prow = base;
  bool cut = false;
  const bool ok = j < nsrc && source(j, prow, cut);
  if (!ok) prow = base;
  const float l = ok ? a.part_lse[prow + hgl] : -INFINITY;
  const int lo = (int)prow;
  const int hi = (int)(prow >> 32);
  #pragma unroll
  for (int u = 0; u < 64 / G; ++u) {
    const int src = u << LG;                              // the lane holding source u's row
    const int64_t pr = u < nsrc ? ((int64_t)__shfl(hi, src) << 32) | (uint32_t)__shfl(lo, src) : base;
    const float4_v *op = reinterpret_cast<const float4_v *>(a.part_o + pr * D + e0);
    #pragma unroll
    for (int k = 0; k < E / 4; ++k) v[u][k] = op[k];
  }
  group_merge<BF16, D, E>(a, base, lane, l, v, nsrc);
}

// Exclusive prefix sum of q_lens into q_start[0..n]; one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void q_start_kernel(const int32_t *q_lens, int32_t *q_start, int n) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int lo = min(n, tid * per);
  const int hi = min(n, lo + per);
  int32_t local = 0;
  for (int k = lo; k < hi; ++k) local += max(q_lens[k], 0);
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - local;             // exclusive prefix of this thread's range
  for (int k = lo; k < hi; ++k) {
    q_start[k] = run;
    run += max(q_lens[k], 0);
  }
  if (tid == 1023) q_start[n] = part[1023];
}

// Floats per lane of the grouped merge (G heads x D dims over 64 lanes), or 0 when it does not apply:
// G a power of two from 2 to 16 with 4 <= G D / 64 <= 16, the balanced schedule without fixed
// partitions (a row's sources are then its item's pieces, a few), and at least 4096 rows.  With
// fewer rows the per-row merge's waves all run at once and grouping only lengthens each wave's chain
// (measured: 1024 rows +1.2%; 5120 rows -2%; 16384 rows -1.3%).
static int group_e(const DecodeArgs &a, int head_dim) {
  const int G = a.group;
  if (G < 2 || G > 16 || (G & (G - 1)) != 0) return 0;
  if (a.spill_base < 0 || a.num_parts != 1) return 0;
  if ((int64_t)a.num_seqs * a.max_q_len * a.num_heads < 4096) return 0;
  const int e = G * head_dim / 64;
  return e >= 4 && e <= 16 ? e : 0;
}

// pre: the read-once decode's prefix pass to merge (bf16 only), or nullptr.
hipError_t launch_combine(const DecodeArgs &a, bool bf16, int head_dim, const PrefixArgs *pre, hipStream_t st) {
  const int64_t waves = (int64_t)a.num_seqs * a.max_q_len * a.num_heads;
  const int grid = (int)((waves + 3) / 4);
  const PrefixArgs none{};
  // per-row merge: the first 16 or 32 piece slots in its first round trip (uniform new tokens only)
  const int ns = a.max_pieces > 1 && !a.q_lens ? (a.max_pieces <= 16 ? 16 : 32) : 0;
  if (pre) {
    if (head_dim == 64) combine_kernel<true, 64, true, 0><<<grid, 256, 0, st>>>(a, *pre);
    else combine_kernel<true, 128, true, 0><<<grid, 256, 0, st>>>(a, *pre);
  } else if (bf16 && group_e(a, head_dim) > 0) {
    const int gg = (int)(((int64_t)a.num_seqs * a.max_q_len * a.num_kv_heads + 3) / 4);
    switch (head_dim * 1000 + group_e(a, head_dim)) {
      case 64004: combine_group_kernel<true, 64, 4><<<gg, 256, 0, st>>>(a); break;
      case 64008: combine_group_kernel<true, 64, 8><<<gg, 256, 0, st>>>(a); break;
      case 64016: combine_group_kernel<true, 64, 16><<<gg, 256, 0, st>>>(a); break;
      case 128004: combine_group_kernel<true, 128, 4><<<gg, 256, 0, st>>>(a); break;
      case 128008: combine_group_kernel<true, 128, 8><<<gg, 256, 0, st>>>(a); break;
      default: combine_group_kernel<true, 128, 16><<<gg, 256, 0, st>>>(a); break;
    }
  } else {
    // bf16 / fp32 output x head dim x slots read up front
    auto go = [&](auto kernel) { kernel<<<grid, 256, 0, st>>>(a, none); };
    const int key = (bf16 ? 1000 : 0) + (head_dim == 64 ? 100 : 0) + ns;
    switch (key) {
      case 1100: go(combine_kernel<true, 64, false, 0>); break;
      case 1116: go(combine_kernel<true, 64, false, 16>); break;
      case 1132: go(combine_kernel<true, 64, false, 32>); break;
      case 1000: go(combine_kernel<true, 128, false, 0>); break;
      case 1016: go(combine_kernel<true, 128, false, 16>); break;
      case 1032: go(combine_kernel<true, 128, false, 32>); break;
      case 100: go(combine_kernel<false, 64, false, 0>); break;
      case 116: go(combine_kernel<false, 64, false, 16>); break;
      case 132: go(combine_kernel<false, 64, false, 32>); break;
      case 16: go(combine_kernel<false, 128, false, 16>); break;
      case 32: go(combine_kernel<false, 128, false, 32>); break;
      default: go(combine_kernel<false, 128, false, 0>); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_q_start(const int32_t *q_lens, int32_t *q_start, int n, hipStream_t st) {
  q_start_kernel<<<1, 1024, 0, st>>>(q_lens, q_start, n);
  return hipGetLastError();
}

}  // namespace pkv
