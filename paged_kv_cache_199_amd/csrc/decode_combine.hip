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

template <bool BF16, int D, bool PRE>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a, PrefixArgs p) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = a.num_heads;
  const int64_t nw = (int64_t)a.num_seqs * a.max_q_len * H;
  if (wid >= nw) return;
  const int h = (int)(wid % H);
  const int64_t t = wid / H;
  const int i = (int)(t % a.max_q_len);
  const int s = (int)(t / a.max_q_len);
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
    prow = a.spill_base + (int64_t)share_slot(W, ord) * a.rows_per_tile + srow;
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

// pre: the read-once decode's prefix pass to merge (bf16 only), or nullptr.
hipError_t launch_combine(const DecodeArgs &a, bool bf16, int head_dim, const PrefixArgs *pre, hipStream_t st) {
  const int64_t waves = (int64_t)a.num_seqs * a.max_q_len * a.num_heads;
  const int grid = (int)((waves + 3) / 4);
  const PrefixArgs none{};
  if (pre) {
    if (head_dim == 64) combine_kernel<true, 64, true><<<grid, 256, 0, st>>>(a, *pre);
    else combine_kernel<true, 128, true><<<grid, 256, 0, st>>>(a, *pre);
  } else if (bf16) {
    if (head_dim == 64) combine_kernel<true, 64, false><<<grid, 256, 0, st>>>(a, none);
    else combine_kernel<true, 128, false><<<grid, 256, 0, st>>>(a, none);
  } else {
    if (head_dim == 64) combine_kernel<false, 64, false><<<grid, 256, 0, st>>>(a, none);
    else combine_kernel<false, 128, false><<<grid, 256, 0, st>>>(a, none);
  }
  return hipGetLastError();
}

hipError_t launch_q_start(const int32_t *q_lens, int32_t *q_start, int n, hipStream_t st) {
  q_start_kernel<<<1, 1024, 0, st>>>(q_lens, q_start, n);
  return hipGetLastError();
}

}  // namespace pkv
