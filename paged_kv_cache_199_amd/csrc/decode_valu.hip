// Paged decode attention, vector-ALU partition kernel (any dtype / head_dim / row count).
//
// Operation: GQA decode attention over K/V gathered through the block table, restricted to one key
// partition, with an online softmax (inferd page: paged-attention reference beside the page table;
// lfm25-inference page, "Runtime Design": paged GQA/XQA decode with split-K).  A sequence that fits
// one partition writes its final output and LSE here; otherwise this kernel writes a normalized
// partial and its log2-sum-exp for the combine kernel.
//
// Work unit = (kv head, partition, sequence, row tile); one 256-thread workgroup (4 waves) per unit.
// Rows of a unit are the G query heads sharing the kv head times the sequence's new tokens
// (row r -> token r / G, head kvh * G + r % G), R of them per row tile.  The 4 waves take the
// partition's 16-token pages round robin and merge their softmax states through LDS at the end.
//
// Per page and wave:
//   QK  lane = (token t = lane / 4, quarter j = lane % 4): the lane holds 16-byte chunks j, j+4, ...
//       of K row t (K pages are token-major, so each load instruction reads 64 contiguous bytes of
//       each of 16 rows) and the matching q chunks in registers; a quad DPP sum gives the score.
//       bf16 pairs go through v_dot2_f32_bf16 (exact products, fp32 sum).
//   softmax: the running max is wave-uniform per row and moves only when some score exceeds it by
//       more than kRescaleSlack (checked with one ballot), so the cross-lane max and the rescale of
//       the accumulators are rare events; every lane keeps its own share of the exp-sum.
//   PV  lane = (token group, dims): V pages are dim-major, so one 16-byte load is 8 (bf16) or 4 (fp32)
//       consecutive tokens of one dim and each load instruction reads 1 KiB contiguous.  The
//       probabilities cross lanes through a per-wave LDS row; the per-token-group partial sums are
//       folded once at the end.
#include "decode_args.h"
#include "device_common.h"

namespace pkv {

template <bool BF16, int D, int R>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  constexpr int E = BF16 ? 2 : 4;          // element bytes
  constexpr int ROWB = D * E;              // bytes of one K token row
  constexpr int NCH = ROWB / 16;           // 16-byte chunks per K row
  constexpr int CPL = NCH / 4;             // K chunks per lane
  constexpr int TPC = 16 / E;              // tokens per 16-byte V chunk
  constexpr int NTG = kBlock / TPC;        // token groups per V dim row
  constexpr int LPG = 64 / NTG;            // lanes per token group
  constexpr int DPL = D / LPG;             // V dims per lane
  constexpr int NW = 4;
  static_assert(CPL >= 1 && DPL >= 1, "layout");

  __shared__ float pbuf[NW][R][kBlock];
  __shared__ float mrg_acc[NW][R][D];
  __shared__ float mrg_m[NW][R];
  __shared__ float mrg_l[NW][R];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

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
  const int row0 = rt * R;
  if (row0 >= rows) return;
  const int H = a.num_heads;
  const int KVH = a.num_kv_heads;

  // ---- rows of this tile
  int last[R];        // last visible key position of each row (-1: inactive row)
  int qrow[R], head[R];
  #pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = row0 + r;
    const int i = rr / G;
    qrow[r] = si.qbase + i;
    head[r] = kvh * G + (rr - i * G);
    const bool ok = rr < rows && qrow[r] < a.total_q;
    last[r] = ok ? si.ctx - si.qs + i : -1;
  }
  const int first_last = last[0];   // rows are in token order: row 0 sees the fewest keys

  // ---- q chunks in registers (raw element bits)
  const int t_lane = lane >> 2;
  const int j_lane = lane & 3;
  uint4 qreg[R][CPL];
  #pragma unroll
  for (int r = 0; r < R; ++r) {
    const char *qp = static_cast<const char *>(a.q) + ((int64_t)qrow[r] * H + head[r]) * ROWB;
    #pragma unroll
    for (int c = 0; c < CPL; ++c) {
      qreg[r][c] = last[r] >= 0 ? ld16(qp + (j_lane + 4 * c) * 16) : make_uint4(0, 0, 0, 0);
    }
  }

  float m[R], lsum[R], acc[R][DPL];
  #pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegBig;
    lsum[r] = 0.f;
    #pragma unroll
    for (int k = 0; k < DPL; ++k) acc[r][k] = 0.f;
  }

  const int tok0 = p * a.part_size;
  const int tok1 = min(si.ctx, tok0 + a.part_size);
  const int blk0 = tok0 / kBlock;
  const int nblk = (tok1 - tok0 + kBlock - 1) / kBlock;
  const int32_t *bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const char *kbase = static_cast<const char *>(a.k_cache);
  const char *vbase = static_cast<const char *>(a.v_cache);
  const int tg = lane / LPG;       // V token group of this lane
  const int dl = lane % LPG;       // first V dim of this lane

  for (int jb = wave; jb < nblk; jb += NW) {
    const int lb = blk0 + jb;
    const int bid = bt[lb];
    if (bid < 0 || bid >= a.num_blocks) continue;     // bad metadata: skip the page (memory safety)
    const char *kt = kbase + ((int64_t)bid * KVH + kvh) * (kBlock * ROWB);
    const char *vt = vbase + ((int64_t)bid * KVH + kvh) * (kBlock * ROWB);
    uint4 kc[CPL];
    #pragma unroll
    for (int c = 0; c < CPL; ++c) kc[c] = ld16(kt + t_lane * ROWB + (j_lane + 4 * c) * 16);
    uint4 vc[DPL];
    #pragma unroll
    for (int k = 0; k < DPL; ++k) vc[k] = ld16(vt + ((dl + LPG * k) * kBlock + tg * TPC) * E);

    // scores (log2 units)
    float sc[R];
    #pragma unroll
    for (int r = 0; r < R; ++r) {
      float d0 = 0.f;
      #pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const uint32_t *qw = reinterpret_cast<const uint32_t *>(&qreg[r][c]);
        const uint32_t *kw = reinterpret_cast<const uint32_t *>(&kc[c]);
        #pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (BF16) {
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
            d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, qw[w]),
                                                 __builtin_bit_cast(bf2, kw[w]), d0, false);
          } else {
            d0 = fmaf(__uint_as_float(qw[w]), __uint_as_float(kw[w]), d0);
          }
        }
      }
      sc[r] = quad_sum(d0) * a.scale_log2;
    }

    const int bstart = lb * kBlock;
    if (bstart + kBlock > first_last + 1) {
      // the page reaches past some row's last visible key (causal edge or context tail)
      const int pos = bstart + t_lane;
      #pragma unroll
      for (int r = 0; r < R; ++r)
        if (pos > last[r]) sc[r] = -INFINITY;
      const int valid = si.ctx - bstart;               // tokens of this page inside the context
      if (valid < kBlock) {
        // tail slots may hold anything (even NaN): zero them so that p = 0 gives exactly 0
        #pragma unroll
        for (int k = 0; k < DPL; ++k) {
          uint32_t *vw = reinterpret_cast<uint32_t *>(&vc[k]);
          #pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (BF16) {
              const int t0 = tg * TPC + 2 * w;
              if (t0 >= valid) vw[w] = 0u;
              else if (t0 + 1 >= valid) vw[w] &= 0xffffu;
            } else {
              if (tg * TPC + w >= valid) vw[w] = 0u;
            }
          }
        }
      }
    }

    // lazy running max
    bool need = false;
    #pragma unroll
    for (int r = 0; r < R; ++r) need |= sc[r] > m[r] + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      #pragma unroll
      for (int r = 0; r < R; ++r) {
        const float bm = quads_max(sc[r]);
        const float mn = fmaxf(m[r], bm);
        const float alpha = exp2_hw(m[r] - mn);
        m[r] = mn;
        lsum[r] *= alpha;
        #pragma unroll
        for (int k = 0; k < DPL; ++k) acc[r][k] *= alpha;
      }
    }

    float pr[R];
    #pragma unroll
    for (int r = 0; r < R; ++r) {
      pr[r] = exp2_hw(sc[r] - m[r]);
      lsum[r] += pr[r];
      if ((r & 3) == j_lane) pbuf[wave][r][t_lane] = pr[r];
    }
    wave_lds_sync();

    // PV
    #pragma unroll
    for (int r = 0; r < R; ++r) {
      float pw[TPC];
      #pragma unroll
      for (int e = 0; e < TPC; e += 4) {
        const float4 f = *reinterpret_cast<const float4 *>(&pbuf[wave][r][tg * TPC + e]);
        pw[e] = f.x;
        pw[e + 1] = f.y;
        pw[e + 2] = f.z;
        pw[e + 3] = f.w;
      }
      #pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const uint32_t *vw = reinterpret_cast<const uint32_t *>(&vc[k]);
        float x = acc[r][k];
        #pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (BF16) {
            x = fmaf(pw[2 * w], bf16_lo(vw[w]), x);
            x = fmaf(pw[2 * w + 1], bf16_hi(vw[w]), x);
          } else {
            x = fmaf(pw[w], __uint_as_float(vw[w]), x);
          }
        }
        acc[r][k] = x;
      }
    }
    asm volatile("" ::: "memory");
  }

  // ---- fold lanes, then merge the 4 waves
  #pragma unroll
  for (int r = 0; r < R; ++r) {
    const float l = quads_sum(lsum[r]);
    #pragma unroll
    for (int k = 0; k < DPL; ++k) {
      float x = acc[r][k];
      if constexpr (NTG == 4) x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[r][k] = x;
    }
    if (lane < LPG) {
      #pragma unroll
      for (int k = 0; k < DPL; ++k) mrg_acc[wave][r][dl + LPG * k] = acc[r][k];
    }
    if (lane == 0) {
      mrg_m[wave][r] = m[r];
      mrg_l[wave][r] = l;
    }
  }
  __syncthreads();

  const bool single = si.nparts == 1;
  for (int idx = threadIdx.x; idx < R * D; idx += 256) {
    const int r = idx / D;
    const int d = idx - r * D;
    if (last[r] < 0) continue;
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
    const int64_t orow = (int64_t)qrow[r] * H + head[r];
    if (single) {
      if constexpr (BF16) {
        static_cast<uint16_t *>(a.out)[orow * D + d] = f32_to_bf16(o);
      } else {
        static_cast<float *>(a.out)[orow * D + d] = o;
      }
      if (d == 0 && a.lse) a.lse[orow] = lse2 * kLn2;
    } else {
      const int64_t prow = (int64_t)p * a.total_q * H + orow;
      a.part_o[prow * D + d] = o;
      if (d == 0) a.part_lse[prow] = lse2;
    }
  }
}

template <bool BF16, int D, int R>
static hipError_t launch_valu_rd(const DecodeArgs &a, hipStream_t st) {
  const int grid = a.per_xcd * 8;
  decode_valu_kernel<BF16, D, R><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <bool BF16, int D>
static hipError_t launch_valu_d(const DecodeArgs &a, int R, hipStream_t st) {
  switch (R) {
    case 1: return launch_valu_rd<BF16, D, 1>(a, st);
    case 2: return launch_valu_rd<BF16, D, 2>(a, st);
    case 4: return launch_valu_rd<BF16, D, 4>(a, st);
    default:
      if constexpr (BF16) return launch_valu_rd<BF16, D, 8>(a, st);
      return hipErrorInvalidValue;
  }
}

// Rows per tile the VALU kernel is built for: up to 8 (bf16) or 4 (fp32).
int valu_max_rows(bool bf16) { return bf16 ? 8 : 4; }

hipError_t launch_decode_valu(const DecodeArgs &a, bool bf16, int head_dim, int rows_per_tile,
                              hipStream_t st) {
  if (bf16) {
    return head_dim == 64 ? launch_valu_d<true, 64>(a, rows_per_tile, st)
                          : launch_valu_d<true, 128>(a, rows_per_tile, st);
  }
  return head_dim == 64 ? launch_valu_d<false, 64>(a, rows_per_tile, st)
                        : launch_valu_d<false, 128>(a, rows_per_tile, st);
}

}  // namespace pkv
