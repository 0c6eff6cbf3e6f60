// One wave's share of paged decode attention on the matrix cores (bf16 K/V), shared by the
// one-workgroup-per-partition kernel and the persistent kernel.
//
// A wave owns up to 16 * NT query rows that read one kv head (the G query heads sharing it times the
// sequence's new tokens; row r -> token r / G, head kvh * G + r % G).  Per 16-token page it forms
//   S^T[t][r] = sum_d K[t][d] Q[r][d]       v_mfma_f32_16x16x32_bf16, D/32 steps
//   O^T[d][r] += sum_t V^T[d][t] P^T[t][r]   v_mfma_f32_16x16x16_bf16, one per 16 output dims
// The 16x16 accumulator layout (lane l holds column l % 16, rows 4*(l/16) .. +3) makes the score tile
// the B operand of the P.V product: each lane softmaxes its own four scores, packs them to bf16 and
// feeds them in, with no lane exchange.  The V^T operand wants four consecutive tokens of one dim per
// lane, which dim-major V pages give with one 8-byte load.
//
// Pages stream through a ring of NBUF register buffers: the loads of page j + NBUF - 1 are issued
// before page j is computed.  Buffers are indexed by compile-time constants (the loop is unrolled
// NBUF times) and every issue is unconditional (past the last page it re-reads the last page), so the
// compiler counts the loads in flight exactly and waits only for the page it is about to use.
#pragma once

#include "decode_args.h"
#include "device_common.h"
#include "e4m3.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));


template <int D, int NT>
struct WaveRows {
  static constexpr int NK = D / 32;
  int last[NT];          // last visible key position of this lane's row per N tile; -1: no row
  int orow[NT];          // q row * H + head of this lane's row
  bf16x8_t qB[NT][NK];   // B operands of the score product
  int first_last;        // fewest visible keys among the rows (rows are in token order)
};

template <int D, int NT>
struct WaveAcc {
  static constexpr int ND = D / 16;
  float m[NT];           // running max (log2 units), equal on the 4 lanes of a column
  float lsum[NT];        // this lane's share of the exp-sum
  float4_t acc[NT][ND];  // O^T: lane holds dims 16 t + 4 (l/16) + e of its column's row
};

// Rows [row0, row0 + 16 NT) of (sequence, kv head); `rows` = q_s * G of the sequence.
template <int D, int NT>
__device__ __forceinline__ void load_rows(const DecodeArgs &a, const SeqInfo &si, int kvh, int row0,
                                          int rows, int col, int grp, WaveRows<D, NT> &w) {
  const int G = a.group;
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int rr = row0 + n * 16 + col;
    const int i = rr / G;
    const int qrow = si.qbase + i;
    const int head = kvh * G + (rr - i * G);
    const bool ok = rr < rows && qrow < a.total_q;
    w.last[n] = ok ? si.ctx - si.qs + i : -1;
    w.orow[n] = qrow * a.num_heads + head;
    const char *qp = static_cast<const char *>(a.q) + (int64_t)w.orow[n] * (D * 2);
    #pragma unroll
    for (int c = 0; c < WaveRows<D, NT>::NK; ++c) {
      const uint4 v = ok ? ld16(qp + (4 * c + grp) * 16) : make_uint4(0, 0, 0, 0);
      w.qB[n][c] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  w.first_last = si.ctx - si.qs + row0 / G;
}

template <int D, int NT>
__device__ __forceinline__ void init_acc(WaveAcc<D, NT> &s) {
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    s.m[n] = kNegBig;
    s.lsum[n] = 0.f;
    #pragma unroll
    for (int t = 0; t < WaveAcc<D, NT>::ND; ++t) s.acc[n][t] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// One 16-token page starting at logical position bstart: scores, mask, online softmax, P.V.
template <int D, int NT>
__device__ __forceinline__ void mfma_page(const DecodeArgs &a, const SeqInfo &si, int bstart,
                                          const uint4 *kr, uint2 *vr, bool ok, int lane,
                                          const WaveRows<D, NT> &w, WaveAcc<D, NT> &st) {
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  const int grp = lane >> 4;
  // x = raw score * scale - running max in one rounding: the exp2 argument.  The raw scores stay
  // for the rare step that moves the max (the max may still be the seed, which x cannot resolve).
  float4_t c[NT], x[NT];
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    float4_t c4 = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int k = 0; k < NK; ++k)
      c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[k]), w.qB[n][k], c4, 0, 0, 0);
    c[n] = c4;
    #pragma unroll
    for (int e = 0; e < 4; ++e) x[n][e] = fmaf(c4[e], a.scale_log2, -st.m[n]);
  }
  if (!ok || bstart + kBlock > w.first_last + 1) {
    // the page reaches past some row's last visible key (causal edge or context tail)
    const int pos0 = bstart + 4 * grp;
    #pragma unroll
    for (int n = 0; n < NT; ++n) {
      #pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!ok || pos0 + e > w.last[n]) x[n][e] = -INFINITY;
    }
    const int valid = ok ? si.ctx - bstart : 0;
    if (valid < kBlock) {
      // slots past the context may hold anything (even NaN): zero them so p = 0 adds exactly 0
      #pragma unroll
      for (int t = 0; t < ND; ++t) {
        if (4 * grp >= valid) vr[t].x = 0u;
        else if (4 * grp + 1 >= valid) vr[t].x &= 0xffffu;
        if (4 * grp + 2 >= valid) vr[t].y = 0u;
        else if (4 * grp + 3 >= valid) vr[t].y &= 0xffffu;
      }
    }
  }
  // lazy running max: moves only when a score exceeds it by more than kRescaleSlack.  x is never NaN
  // (masked scores are -inf), and for a threshold >= 0 a float exceeds it exactly when its bits, read
  // as a signed integer, do: integer maxima need no NaN quieting, which float maxima pay per operand
  static_assert(kRescaleSlack >= 0.f, "the integer comparison needs a non-negative threshold");
  int xbits = __float_as_int(x[0][0]);
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    #pragma unroll
    for (int e = 0; e < 4; ++e) xbits = max(xbits, __float_as_int(x[n][e]));
  }
  const bool need = xbits > __float_as_int(kRescaleSlack);
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    #pragma unroll
    for (int n = 0; n < NT; ++n) {
      // masked scores are exactly -inf in x; every other x is finite
      float4_t sc;
      #pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = x[n][e] == -INFINITY ? -INFINITY : c[n][e] * a.scale_log2;
      float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mn = fmaxf(st.m[n], bm);
      const float alpha = exp2_hw(st.m[n] - mn);
      st.m[n] = mn;
      st.lsum[n] *= alpha;
      #pragma unroll
      for (int t = 0; t < ND; ++t) st.acc[n][t] *= alpha;
      #pragma unroll
      for (int e = 0; e < 4; ++e) x[n][e] = sc[e] - mn;
    }
  }
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float p0 = exp2_hw(x[n][0]);
    const float p1 = exp2_hw(x[n][1]);
    const float p2 = exp2_hw(x[n][2]);
    const float p3 = exp2_hw(x[n][3]);
    st.lsum[n] += (p0 + p1) + (p2 + p3);
    const uint2 pw = make_uint2(pack_bf16x2(p0, p1), pack_bf16x2(p2, p3));
    const short4_t pB = __builtin_bit_cast(short4_t, pw);
    #pragma unroll
    for (int t = 0; t < ND; ++t)
      st.acc[n][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, vr[t]), pB,
                                                               st.acc[n][t], 0, 0, 0);
  }
}

// Attend the pages with logical block numbers blk_first + j * blk_stride, j < npages (npages <= 64),
// of one sequence (block-table row bt_row) and one kv head.
template <int D, int NT, int NBUF>
__device__ __forceinline__ void attend_pages(const DecodeArgs &a, const SeqInfo &si, int kvh,
                                             const int32_t *bt_row, int blk_first, int blk_stride,
                                             int npages, int lane, const WaveRows<D, NT> &w,
                                             WaveAcc<D, NT> &st) {
  constexpr int ROWB = D * 2;
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  if (npages <= 0) return;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int KVH = a.num_kv_heads;
  const int64_t nb = a.num_blocks;
  const int64_t page_bytes = (int64_t)kBlock * ROWB;
  const char *kbase = static_cast<const char *>(a.k_cache);
  const char *vbase = static_cast<const char *>(a.v_cache);
  const int ids = lane < npages ? bt_row[blk_first + lane * blk_stride] : 0;

  uint4 kb[NBUF][NK];
  uint2 vb[NBUF][ND];
  bool okb[NBUF];
  auto issue = [&](int j, uint4 *kr, uint2 *vr, bool &ok) {
    const int bid = __builtin_amdgcn_readlane(ids, j);
    ok = bid >= 0 && bid < nb;
    const int64_t off = ((int64_t)(ok ? bid : 0) * KVH + kvh) * page_bytes;
    const char *kp = kbase + off + col * ROWB + grp * 16;
    #pragma unroll
    for (int c = 0; c < NK; ++c) kr[c] = ld16(kp + c * 64);
    const char *vp = vbase + off + (col * kBlock + 4 * grp) * 2;
    #pragma unroll
    for (int t = 0; t < ND; ++t) vr[t] = *reinterpret_cast<const uint2 *>(vp + t * 16 * kBlock * 2);
  };
  auto compute = [&](int j, const uint4 *kr, uint2 *vr, bool ok) {
    mfma_page<D, NT>(a, si, (blk_first + j * blk_stride) * kBlock, kr, vr, ok, lane, w, st);
  };

  const int last_j = npages - 1;
  #pragma unroll
  for (int j = 0; j < NBUF - 1; ++j) issue(min(j, last_j), kb[j], vb[j], okb[j]);
  int j0 = 0;
  for (; j0 + NBUF <= npages; j0 += NBUF) {
    #pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int bn = (b + NBUF - 1) % NBUF;   // a constant once the loop is unrolled
      issue(min(j0 + b + NBUF - 1, last_j), kb[bn], vb[bn], okb[bn]);
      compute(j0 + b, kb[b], vb[b], okb[b]);
    }
  }
  // fewer than NBUF pages left: their loads are already in flight
  #pragma unroll
  for (int b = 0; b < NBUF - 1; ++b)
    if (j0 + b < npages) compute(j0 + b, kb[b], vb[b], okb[b]);
}

typedef const __attribute__((address_space(4))) int32_t const_i32;

// Attend the consecutive logical pages [jb, je) of one (sequence, kv head, row tile), flushing the
// softmax state through flush(partition, first page, end page) of each piece: after the last page of
// every partition of PP pages and after page je - 1.  Either jb and PP are multiples of NBUF, or
// the run lies inside one partition (PP >= je); so partition ends fall on the last page of a ring
// cycle (or the run's end) and the flush sits outside the unrolled cycle.  Page ids come through the scalar cache
// (the block table is read-only here): the id of the page issued NBUF steps later is fetched while
// the current page is computed, so those loads never hold up the vector loads and a run of any
// length streams without a restart.
// Two E4M3 codes (the low or high half of w) to two bf16 in one word, exactly: every E4M3 value is a
// bf16 value, so the hardware's exact fp8 -> f32 conversion followed by dropping the low 16 bits
// loses nothing.
typedef float float2_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  const float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}

// Registers of one page for one lane as loaded (bf16: already the MFMA operand layout; E4M3: half the
// bytes, widened to it just before use).
template <bool F8> struct KvRaw {
  typedef uint4 K;      // 8 bf16 of one token row: the score product's A operand
  typedef uint2 V;      // 4 tokens of one dim: the value product's A operand
  static constexpr int VT = 1;   // value-product tiles (16 dims each) per V register
};
// E4M3 pages are read with 16-byte loads: the vector-memory address unit spends about the same time on a
// load whatever its width, and with the 4-byte loads that the value operand's layout asks for (4 codes
// of one dim per lane) it, not HBM, bounded the E4M3 decode (busy ~95% of the kernel with few memory
// stalls).  So a lane loads a whole 16-token dim row and a transpose across the wave's four 16-lane
// rows hands each lane its 4 codes of each of 4 tiles.
template <> struct KvRaw<true> {
  typedef uint2 K;      // 8 E4M3 codes
  typedef uint4 V;      // lane (c, r): dim row 64 h + 16 r + c (16 tokens) as loaded
  static constexpr int VT = 4;
};

// 4x4 transpose of 32-bit words across the four 16-lane rows of the wave (every lane active): lane
// (c, r), holding words A[r][0..3], ends with A[t][r] as its word t.  Two rounds of gfx950's lane swaps:
// between the 32-lane halves (words 0/2 and 1/3), then between neighbouring 16-lane rows (0/1, 2/3).
__device__ __forceinline__ uint4 transpose_rows4(uint4 v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  return make_uint4(c[0], c[1], d[0], d[1]);
}

template <int D>
__device__ __forceinline__ void widen_page(const uint4 *kin, const uint2 *vin, uint4 *kout, uint2 *vout) {
  #pragma unroll
  for (int c = 0; c < D / 32; ++c) kout[c] = kin[c];
  #pragma unroll
  for (int t = 0; t < D / 16; ++t) vout[t] = vin[t];
}
template <int D>
__device__ __forceinline__ void widen_page(const uint2 *kin, const uint4 *vin, uint4 *kout, uint2 *vout) {
  #pragma unroll
  for (int c = 0; c < D / 32; ++c)
    kout[c] = make_uint4(fp8x2_to_bf16x2<false>(kin[c].x), fp8x2_to_bf16x2<true>(kin[c].x),
                         fp8x2_to_bf16x2<false>(kin[c].y), fp8x2_to_bf16x2<true>(kin[c].y));
  #pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    // word t of lane (c, r): codes of tokens 4 r .. 4 r + 3 of dim 64 h + 16 t + c, i.e. tile 4 h + t
    const uint4 w = transpose_rows4(vin[h]);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    #pragma unroll
    for (int t = 0; t < 4; ++t)
      vout[4 * h + t] = make_uint2(fp8x2_to_bf16x2<false>(ws[t]), fp8x2_to_bf16x2<true>(ws[t]));
  }
}

// F8: the pools hold E4M3 codes (1 byte per element) instead of bf16; pages are half as large and are
// widened in registers right before their products.
// start() runs once the first pages' loads are out, for work that can wait on them.
template <int D, int NT, int NBUF, bool F8, class Flush, class Patch, class Start>
__device__ __forceinline__ void stream_pages(const DecodeArgs &a, const SeqInfo &si, int kvh,
                                             const int32_t *bt_row, int jb, int je, int PP, int lane,
                                             const WaveRows<D, NT> &w, WaveAcc<D, NT> &st,
                                             Flush flush, Patch patch, Start start) {
  constexpr int EB = F8 ? 1 : 2;          // bytes per cache element
  constexpr int ROWB = D * EB;
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  typedef typename KvRaw<F8>::K KR;
  typedef typename KvRaw<F8>::V VR;
  const int n = je - jb;
  if (n <= 0) return;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int KVH = a.num_kv_heads;
  const int64_t nb = a.num_blocks;
  const int64_t page_bytes = (int64_t)kBlock * ROWB;
  const char *kbase = static_cast<const char *>(a.k_cache);
  const char *vbase = static_cast<const char *>(a.v_cache);
  const_i32 *btc = (const_i32 *)(bt_row);   // a C-style cast is the only way into address space 4
  const int last = je - 1;
  auto id_of = [&](int j) -> int { return btc[__builtin_amdgcn_readfirstlane(min(j, last))]; };

  constexpr int NV = ND / KvRaw<F8>::VT;   // V registers per page
  KR kb[NBUF][NK];
  VR vb[NBUF][NV];
  bool okb[NBUF];
  auto issue = [&](int bid, KR *kr, VR *vr, bool &ok) {
    ok = bid >= 0 && bid < nb;
    const int64_t off = ((int64_t)(ok ? bid : 0) * KVH + kvh) * page_bytes;
    const char *kp = kbase + off + col * ROWB + grp * 8 * EB;
    #pragma unroll
    for (int c = 0; c < NK; ++c) kr[c] = *reinterpret_cast<const KR *>(kp + c * 32 * EB);
    if constexpr (F8) {
      // whole dim rows: lane (col, grp) reads row 64 h + 16 grp + col
      const char *vp = vbase + off + (16 * grp + col) * kBlock * EB;
      #pragma unroll
      for (int h = 0; h < NV; ++h) vr[h] = *reinterpret_cast<const VR *>(vp + h * 64 * kBlock * EB);
    } else {
      const char *vp = vbase + off + (col * kBlock + 4 * grp) * EB;
      #pragma unroll
      for (int t = 0; t < ND; ++t) vr[t] = *reinterpret_cast<const VR *>(vp + t * 16 * kBlock * EB);
    }
  };
  // widen (E4M3) or take (bf16) page b of the ring, then substitute appended tokens, then compute
  auto compute = [&](int j, const KR *kr, const VR *vr, bool ok) {
    uint4 kc[NK];
    uint2 vc[ND];
    widen_page<D>(kr, vr, kc, vc);
    patch(j, kc, vc);
    mfma_page<D, NT>(a, si, j * kBlock, kc, vc, ok, lane, w, st);
  };

  int sid[NBUF];
  #pragma unroll
  for (int j = 0; j < NBUF - 1; ++j) issue(id_of(jb + j), kb[j], vb[j], okb[j]);
  #pragma unroll
  for (int b = 0; b < NBUF; ++b) sid[b] = id_of(jb + NBUF - 1 + b);
  start();
  int j0 = 0;
  int piece = jb;
  for (; j0 + NBUF <= n; j0 += NBUF) {
    #pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int bn = (b + NBUF - 1) % NBUF;   // constants once the loop is unrolled
      issue(sid[b], kb[bn], vb[bn], okb[bn]);
      sid[b] = id_of(jb + j0 + b + 2 * NBUF - 1);
      compute(jb + j0 + b, kb[b], vb[b], okb[b]);
    }
    const int jl = jb + j0 + NBUF - 1;
    if ((jl + 1) % PP == 0 || jl == last) {
      flush(jl / PP, piece, jl + 1);
      piece = jl + 1;
    }
  }
  if (j0 < n) {
    #pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) {
      if (j0 + b < n) compute(jb + j0 + b, kb[b], vb[b], okb[b]);
    }
    flush(last / PP, piece, je);
  }
}

// New tokens appended in the decode pass itself.  The q_s new tokens of a sequence sit at its last
// positions ctx - q_s .. ctx - 1 (one or two pages).  A wave whose run reaches them loads their K/V
// rows for its kv head into registers when it starts the run (those loads fly with the first
// pages); on each page that holds new tokens it stages them through its LDS area and substitutes
// them for the cache rows it just loaded (so no other wave's write has to come first); after the
// run, row tile 0 stores them into their cache slots.  The K/V row of token i is row qbase + i of
// new_k / new_v [total_q, KVH, D] (bf16).  Over E4M3 pools (F8) the rows are quantized once when
// loaded, exactly as the slot-mapped write does it (x / scale in fp32, nearest code): the codes are
// what gets stored, and what the page walk substitutes is their exact bf16 value, the same value a
// separate write followed by decode would read back.
template <int D, bool F8 = false>
struct AppendRows {
  static constexpr int ROWB = D * 2;
  static constexpr int CH = ROWB / 16;                    // 16-byte chunks per bf16 row
  static constexpr int MAXQ = 8;                          // new tokens per sequence on this path
  static constexpr int PER_LANE = (MAXQ * CH + 63) / 64;
  uint4 k[PER_LANE];                                      // bf16 (F8: the codes' exact values)
  uint4 v[PER_LANE];
  uint2 kq[F8 ? PER_LANE : 1];                            // F8: the 8 codes of each chunk
  uint2 vq[F8 ? PER_LANE : 1];
  int first;       // position of new token 0
  int n;           // new tokens
  bool staged;
};

// 8 bf16 (one 16-byte chunk) -> their 8 E4M3 codes under `scale`, and the codes' exact bf16 values.
__device__ __forceinline__ void quantize_chunk(const uint4 &x, float scale, uint2 &codes, uint4 &back) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t c[2] = {0u, 0u};
  #pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
    c[e >> 2] |= e4m3_code(__uint_as_float(h << 16) / scale) << (8 * (e & 3));
  }
  codes = make_uint2(c[0], c[1]);
  back = make_uint4(fp8x2_to_bf16x2<false>(c[0]), fp8x2_to_bf16x2<true>(c[0]), fp8x2_to_bf16x2<false>(c[1]),
                    fp8x2_to_bf16x2<true>(c[1]));
}

template <int D, bool F8>
__device__ __forceinline__ void append_load(const DecodeArgs &a, const SeqInfo &si, int kvh, int lane,
                                            AppendRows<D, F8> &r) {
  constexpr int CH = AppendRows<D, F8>::CH;
  r.first = si.ctx - si.qs;
  r.n = min(si.qs, AppendRows<D, F8>::MAXQ);   // more new tokens than that is a broken precondition
  r.staged = false;
  const char *nk = static_cast<const char *>(a.new_k);
  const char *nv = static_cast<const char *>(a.new_v);
  #pragma unroll
  for (int u = 0; u < AppendRows<D, F8>::PER_LANE; ++u) {
    const int c = lane + 64 * u;
    const int tok = c / CH;
    const bool ok = tok < r.n && si.qbase + tok < a.total_q;
    const int64_t off = (((int64_t)(ok ? si.qbase + tok : 0) * a.num_kv_heads + kvh) * CH + c % CH) * 16;
    r.k[u] = ok ? ld16(nk + off) : make_uint4(0, 0, 0, 0);
    r.v[u] = ok ? ld16(nv + off) : make_uint4(0, 0, 0, 0);
    if constexpr (F8) {
      quantize_chunk(r.k[u], a.k_scale, r.kq[u], r.k[u]);
      quantize_chunk(r.v[u], a.v_scale, r.vq[u], r.v[u]);
    }
  }
}

// Page j (logical) of the run: substitute the new tokens it holds for the (widened) cache rows just
// loaded.  lds: this wave's staging area, 2 * MAXQ * CH chunks.
template <int D, bool F8>
__device__ __forceinline__ void append_patch(int j, int lane, AppendRows<D, F8> &r, uint4 *lds, uint4 *kr,
                                             uint2 *vr) {
  constexpr int CH = AppendRows<D, F8>::CH;
  constexpr int MAXQ = AppendRows<D, F8>::MAXQ;
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  const int p0 = j * kBlock;
  if (p0 + kBlock <= r.first) return;                     // wave-uniform: no new token on this page
  const int col = lane & 15;
  const int grp = lane >> 4;
  if (!r.staged) {
    #pragma unroll
    for (int u = 0; u < AppendRows<D, F8>::PER_LANE; ++u) {
      const int c = lane + 64 * u;
      if (c < r.n * CH) {
        lds[c] = r.k[u];
        lds[MAXQ * CH + c] = r.v[u];
      }
    }
    wave_lds_sync();
    r.staged = true;
  }
  const uint16_t *lv = reinterpret_cast<const uint16_t *>(lds + MAXQ * CH);
  const int kpos = p0 + col;
  if (kpos >= r.first && kpos < r.first + r.n) {
    const int tok = kpos - r.first;
    #pragma unroll
    for (int c = 0; c < NK; ++c) kr[c] = lds[tok * CH + c * 4 + grp];
  }
  #pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int vpos = p0 + 4 * grp + e;
    if (vpos >= r.first && vpos < r.first + r.n) {
      const int tok = vpos - r.first;
      #pragma unroll
      for (int t = 0; t < ND; ++t) {
        const uint32_t x = lv[tok * D + col + 16 * t];
        if (e == 0) vr[t].x = (vr[t].x & 0xffff0000u) | x;
        else if (e == 1) vr[t].x = (vr[t].x & 0x0000ffffu) | (x << 16);
        else if (e == 2) vr[t].y = (vr[t].y & 0xffff0000u) | x;
        else vr[t].y = (vr[t].y & 0x0000ffffu) | (x << 16);
      }
    }
  }
}

// After the run: store the new tokens that live on its pages [jb, je) into their cache slots (row
// tile 0 only, so each slot is written once): bf16 rows, or (F8) their codes.  Stores wait until the
// page loads are done: on this chip they share the counter the page ring waits on.
template <int D, bool F8>
__device__ __forceinline__ void append_store(const DecodeArgs &a, int kvh, const int32_t *bt_row, int jb, int je,
                                             int lane, const AppendRows<D, F8> &r) {
  constexpr int CH = AppendRows<D, F8>::CH;
  constexpr int EB = F8 ? 1 : 2;                          // bytes per cache element
  char *kc = static_cast<char *>(const_cast<void *>(a.k_cache));
  char *vc = static_cast<char *>(const_cast<void *>(a.v_cache));
  #pragma unroll
  for (int u = 0; u < AppendRows<D, F8>::PER_LANE; ++u) {
    const int c = lane + 64 * u;
    const int tok = c / CH;
    const int pos = r.first + tok;
    const int j = pos / kBlock;
    if (tok < r.n && j >= jb && j < je) {
      const int64_t bid = bt_row[j];
      if (bid >= 0 && bid < a.num_blocks) {
        const int cc = c % CH;                            // elements cc * 8 .. cc * 8 + 7 of the row
        const int off = pos - j * kBlock;
        const int64_t page = bid * a.num_kv_heads + kvh;
        if constexpr (F8) {
          *reinterpret_cast<uint2 *>(kc + (page * kBlock + off) * D + cc * 8) = r.kq[u];
          const uint32_t vw[2] = {r.vq[u].x, r.vq[u].y};
          #pragma unroll
          for (int q = 0; q < 8; ++q)
            vc[(page * D + cc * 8 + q) * kBlock + off] = (char)((vw[q >> 2] >> (8 * (q & 3))) & 0xffu);
        } else {
          *reinterpret_cast<uint4 *>(kc + (page * kBlock + off) * D * EB + cc * 16) = r.k[u];
          const uint16_t *e = reinterpret_cast<const uint16_t *>(&r.v[u]);
          uint16_t *v16 = reinterpret_cast<uint16_t *>(vc);
          #pragma unroll
          for (int q = 0; q < 8; ++q) v16[(page * D + cc * 8 + q) * kBlock + off] = e[q];
        }
      }
    }
  }
}

// Finish one wave's rows without other waves: fold the exp-sum over the column's 4 lanes and write
// either the final output (bf16) + natural-log LSE, or an fp32 partial + log2 LSE: the row of
// partition p, or, when spill_row0 >= 0, partial row spill_row0 + (row within the tile).
template <int D, int NT>
__device__ __forceinline__ void finish_wave(const DecodeArgs &a, int p, bool single, int lane,
                                            const WaveRows<D, NT> &w, const WaveAcc<D, NT> &st,
                                            int64_t spill_row0 = -1) {
  constexpr int ND = D / 16;
  const int grp = lane >> 4;
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    float l = st.lsum[n];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (w.last[n] < 0) continue;
    const bool seen = l > 0.f;
    const float inv = seen ? a.v_scale / l : 0.f;   // v_scale: the V pool's scale (1 for bf16 pools)
    const float lse2 = seen ? st.m[n] + log2_hw(l) : -INFINITY;
    const int64_t orow = w.orow[n];
    if (single) {
      uint16_t *o = static_cast<uint16_t *>(a.out) + orow * D + 4 * grp;
      #pragma unroll
      for (int t = 0; t < ND; ++t) {
        const float4_t v = st.acc[n][t] * inv;
        *reinterpret_cast<uint2 *>(o + t * 16) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
      if (grp == 0 && a.lse) a.lse[orow] = lse2 * kLn2;
    } else {
      const int64_t prow = spill_row0 >= 0 ? spill_row0 + n * 16 + (lane & 15)
                                           : (int64_t)p * a.total_q * a.num_heads + orow;
      float *o = a.part_o + prow * D + 4 * grp;
      #pragma unroll
      for (int t = 0; t < ND; ++t) *reinterpret_cast<float4_t *>(o + t * 16) = st.acc[n][t] * inv;
      if (grp == 0) a.part_lse[prow] = lse2;
    }
  }
}

}  // namespace pkv
