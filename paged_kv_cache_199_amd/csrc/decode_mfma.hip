// Paged decode attention, matrix-core (MFMA) partition kernel for bf16 K/V.
//
// Same operation and work units as the vector-ALU kernel (GQA decode over K/V gathered through the
// block table, one key partition per workgroup, online softmax; inferd page: paged-attention
// reference beside the page table; lfm25-inference page, "Runtime Design": paged GQA/XQA decode with
// split-K).  The rows that share a kv head (G query heads times the new tokens) form the N side of
// two small matrix products per 16-token page:
//
//   S^T[t][r] = sum_d K[t][d] Q[r][d]      v_mfma_f32_16x16x32_bf16, D/32 steps
//   O^T[d][r] += sum_t V^T[d][t] P^T[t][r]  v_mfma_f32_16x16x16_bf16, one per 16 output dims
//
// The 16x16 accumulator layout (lane l holds column l % 16, rows 4*(l/16) .. +3) makes the score
// tile of one product the B operand of the next: after the softmax each lane packs its own four
// probabilities to bf16 and feeds them straight into the P.V product, with no lane exchange.  The
// V^T operand wants four consecutive tokens of one dim per lane, which is why V pages are stored
// dim-major.  Rows are 16 per N tile; up to two N tiles (32 rows) share each page's K/V registers.
//
// Pipelining: each wave preloads the physical ids of all pages it will visit (one per lane) and
// issues the next page's K and V loads before computing on the current page.
#include "decode_args.h"
#include "device_common.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

template <int D, int NT>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NW = 4;
  constexpr int ROWB = D * 2;          // bytes of a K token row / a V dim row pair... (bf16)
  constexpr int NK = D / 32;           // QK k-steps
  constexpr int ND = D / 16;           // PV output tiles
  constexpr int ROWS = 16 * NT;

  __shared__ float mrg_acc[NW][ROWS][D];
  __shared__ float mrg_m[NW][ROWS];
  __shared__ float mrg_l[NW][ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;           // N index (row of the tile) this lane owns
  const int grp = lane >> 4;           // k-group / 4-row group

  int u = xcd_unit(blockIdx.x, a.per_xcd);
  if (u >= a.units) return;
  const int rt = u % a.row_tiles;
  u /= a.row_tiles;
  const int s = u % a.num_seqs;
  u /= a.num_seqs;
  const int p = u % a.num_parts;
  const int kvh = u / a.num_parts;

  const SeqInfo si = load_seq(a, s);
  if (p >= si.nparts) return;
  const int G = a.group;
  const int rows = si.qs * G;
  const int row0 = rt * ROWS;
  if (row0 >= rows) return;
  const int H = a.num_heads;
  const int KVH = a.num_kv_heads;

  // ---- the rows this lane's column stands for, one per N tile
  int last[NT];
  bf16x8_t qB[NT][NK];
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int rr = row0 + n * 16 + col;
    const int i = rr / G;
    const int qrow = si.qbase + i;
    const int head = kvh * G + (rr - i * G);
    const bool ok = rr < rows && qrow < a.total_q;
    last[n] = ok ? si.ctx - si.qs + i : -1;
    const char *qp = static_cast<const char *>(a.q) + ((int64_t)qrow * H + head) * ROWB;
    #pragma unroll
    for (int c = 0; c < NK; ++c) {
      const uint4 w = ok ? ld16(qp + (4 * c + grp) * 16) : make_uint4(0, 0, 0, 0);
      qB[n][c] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  const int first_last = si.ctx - si.qs + row0 / G;   // fewest visible keys among the tile's rows

  float m[NT], lsum[NT];
  float4_t acc[NT][ND];
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    m[n] = kNegBig;
    lsum[n] = 0.f;
    #pragma unroll
    for (int t = 0; t < ND; ++t) acc[n][t] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int tok0 = p * a.part_size;
  const int tok1 = min(si.ctx, tok0 + a.part_size);
  const int blk0 = tok0 / kBlock;
  const int nblk = (tok1 - tok0 + kBlock - 1) / kBlock;
  const int niter = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;
  const int32_t *bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq + blk0 + wave;
  const char *kbase = static_cast<const char *>(a.k_cache);
  const char *vbase = static_cast<const char *>(a.v_cache);
  const int64_t page_bytes = (int64_t)kBlock * ROWB;
  const int64_t nb = a.num_blocks;

  // page ids of iterations [base, base + 64), one per lane
  int ids = 0;
  auto load_ids = [&](int base) {
    const int k = base + lane;
    ids = k < niter ? bt[(int64_t)NW * k] : 0;
  };
  auto page_of = [&](int it, bool &ok) -> int64_t {
    int bid = __builtin_amdgcn_readlane(ids, it & 63);
    ok = bid >= 0 && bid < nb;
    return ((int64_t)(ok ? bid : 0) * KVH + kvh) * page_bytes;
  };
  uint4 kC[NK], kN[NK];
  uint2 vC[ND], vN[ND];
  bool okC = true, okN = true;
  auto issue = [&](int it, uint4 *kr, uint2 *vr, bool &ok) {
    const int64_t off = page_of(it, ok);
    const char *kp = kbase + off + col * ROWB + grp * 16;
    #pragma unroll
    for (int c = 0; c < NK; ++c) kr[c] = ld16(kp + c * 64);
    const char *vp = vbase + off + (col * kBlock + 4 * grp) * 2;
    #pragma unroll
    for (int t = 0; t < ND; ++t) vr[t] = *reinterpret_cast<const uint2 *>(vp + t * 16 * kBlock * 2);
  };

  if (niter > 0) {
    load_ids(0);
    issue(0, kC, vC, okC);
  }
  for (int it = 0; it < niter; ++it) {
    if (it + 1 < niter) {
      if (((it + 1) & 63) == 0) load_ids(it + 1);
      issue(it + 1, kN, vN, okN);
    }
    // S^T for this page: lane holds tokens 4*grp .. +3 of its column's row
    float4_t sc[NT];
    #pragma unroll
    for (int n = 0; n < NT; ++n) {
      float4_t c4 = {0.f, 0.f, 0.f, 0.f};
      #pragma unroll
      for (int c = 0; c < NK; ++c)
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kC[c]), qB[n][c], c4, 0, 0, 0);
      sc[n] = c4 * a.scale_log2;
    }
    const int bstart = (blk0 + wave + it * NW) * kBlock;
    if (!okC || bstart + kBlock > first_last + 1) {
      const int pos0 = bstart + 4 * grp;
      #pragma unroll
      for (int n = 0; n < NT; ++n) {
        #pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!okC || pos0 + e > last[n]) sc[n][e] = -INFINITY;
      }
      const int valid = okC ? si.ctx - bstart : 0;
      if (valid < kBlock) {
        // slots past the context may hold anything: zero them so p = 0 contributes exactly 0
        #pragma unroll
        for (int t = 0; t < ND; ++t) {
          if (4 * grp >= valid) vC[t].x = 0u;
          else if (4 * grp + 1 >= valid) vC[t].x &= 0xffffu;
          if (4 * grp + 2 >= valid) vC[t].y = 0u;
          else if (4 * grp + 3 >= valid) vC[t].y &= 0xffffu;
        }
      }
    }
    bool need = false;
    #pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float th = m[n] + kRescaleSlack;
      need |= sc[n][0] > th || sc[n][1] > th || sc[n][2] > th || sc[n][3] > th;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      #pragma unroll
      for (int n = 0; n < NT; ++n) {
        float bm = fmaxf(fmaxf(sc[n][0], sc[n][1]), fmaxf(sc[n][2], sc[n][3]));
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mn = fmaxf(m[n], bm);
        const float alpha = exp2_hw(m[n] - mn);
        m[n] = mn;
        lsum[n] *= alpha;
        #pragma unroll
        for (int t = 0; t < ND; ++t) acc[n][t] *= alpha;
      }
    }
    #pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float p0 = exp2_hw(sc[n][0] - m[n]);
      const float p1 = exp2_hw(sc[n][1] - m[n]);
      const float p2 = exp2_hw(sc[n][2] - m[n]);
      const float p3 = exp2_hw(sc[n][3] - m[n]);
      lsum[n] += (p0 + p1) + (p2 + p3);
      const uint2 pw = make_uint2(pack_bf16x2(p0, p1), pack_bf16x2(p2, p3));
      const short4_t pB = __builtin_bit_cast(short4_t, pw);
      #pragma unroll
      for (int t = 0; t < ND; ++t)
        acc[n][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, vC[t]), pB,
                                                              acc[n][t], 0, 0, 0);
    }
    #pragma unroll
    for (int c = 0; c < NK; ++c) kC[c] = kN[c];
    #pragma unroll
    for (int t = 0; t < ND; ++t) vC[t] = vN[t];
    okC = okN;
  }

  // ---- per-wave state to LDS, then merge the waves
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    float l = lsum[n];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    #pragma unroll
    for (int t = 0; t < ND; ++t) {
      #pragma unroll
      for (int e = 0; e < 4; ++e) mrg_acc[wave][n * 16 + col][t * 16 + 4 * grp + e] = acc[n][t][e];
    }
    if (grp == 0) {
      mrg_m[wave][n * 16 + col] = m[n];
      mrg_l[wave][n * 16 + col] = l;
    }
  }
  __syncthreads();

  const bool single = si.nparts == 1;
  for (int idx = threadIdx.x; idx < ROWS * D; idx += 256) {
    const int r = idx / D;
    const int d = idx - r * D;
    const int rr = row0 + r;
    if (rr >= rows) continue;
    const int i = rr / G;
    const int qrow = si.qbase + i;
    if (qrow >= a.total_q) continue;
    const int head = kvh * G + (rr - i * G);
    float M = mrg_m[0][r];
    #pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, mrg_m[w][r]);
    float L = 0.f, O = 0.f;
    #pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sw = exp2_hw(mrg_m[w][r] - M);
      L += mrg_l[w][r] * sw;
      O += mrg_acc[w][r][d] * sw;
    }
    const bool seen = L > 0.f;
    const float o = seen ? O / L : 0.f;
    const float lse2 = seen ? M + log2_hw(L) : -INFINITY;
    const int64_t orow = (int64_t)qrow * H + head;
    if (single) {
      static_cast<uint16_t *>(a.out)[orow * D + d] = f32_to_bf16(o);
      if (d == 0 && a.lse) a.lse[orow] = lse2 * kLn2;
    } else {
      const int64_t prow = (int64_t)p * a.total_q * H + orow;
      a.part_o[prow * D + d] = o;
      if (d == 0) a.part_lse[prow] = lse2;
    }
  }
}

// Rows one launch covers per workgroup: 16 per N tile, at most two N tiles.
int mfma_rows_per_tile(int rows) { return rows > 16 ? 32 : 16; }

hipError_t launch_decode_mfma(const DecodeArgs &a, int head_dim, int rows_per_tile, hipStream_t st) {
  const int grid = a.per_xcd * 8;
  if (head_dim == 64) {
    if (rows_per_tile > 16) decode_mfma_kernel<64, 2><<<grid, 256, 0, st>>>(a);
    else decode_mfma_kernel<64, 1><<<grid, 256, 0, st>>>(a);
  } else {
    if (rows_per_tile > 16) decode_mfma_kernel<128, 2><<<grid, 256, 0, st>>>(a);
    else decode_mfma_kernel<128, 1><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace pkv
