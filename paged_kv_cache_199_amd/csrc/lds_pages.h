// K/V pages streamed through LDS for a whole workgroup: the four waves of a 256-thread workgroup each
// own different query rows of one kv head and read the same pages, so every page is fetched from
// HBM once per workgroup instead of once per wave.  SP pages make a stage; two stages alternate, so
// the next stage's loads are in flight while this one is computed.  Each wave then runs the
// decode's matrix-core page step (mfma_wave.h) on the staged pages.
//
// LDS layout of a page: K rows of D bf16 (one per token), each followed by PKV_LDS_KPAD bytes; V as
// D rows of 16 tokens, each row's four 4-token groups stored in slots g ^ vswz(d).  A value read
// serves 16 lanes per LDS cycle: the 16 dims of one 4-token group, whose rows are 32 bytes apart, so
// without the swizzle dims d, d + 4, d + 8, d + 12 would hit the same banks; XOR-ing the slot with
// bits 2-3 of the dim puts all 16 reads in different bank pairs (and the staging writes too).
#pragma once

#include <type_traits>

#include "mfma_wave.h"

#ifndef PKV_LDS_KPAD
#define PKV_LDS_KPAD 16   // bytes after each token row of a K page (a multiple of 16)
#endif

namespace pkv {

__device__ __forceinline__ int vswz(int d) { return (d >> 2) & 3; }

// ---- Value products at the full matrix-core rate (two 16-row tiles per wave, D = 64 or 128) ----
// A 16-token page gives the P.V product only 16 keys, so v_mfma_f32_16x16x16_bf16 runs it at half
// the matrix cores' rate (16 of the page step's 24 matrix-core instructions).  v_mfma_f32_32x32x16_bf16
// takes the same 16 keys at the full rate: O^T[d][r] += sum_t V^T[d][t] P^T[t][r] for 32 dims x 32
// rows, four instructions per page at D = 128 instead of sixteen.  Its operands (lane l: column
// l % 32, keys 8 (l / 32) .. + 7; accumulator: column l % 32, rows 8 q + 4 (l / 32) + e in register
// 4 q + e) take the V^T rows straight from LDS (16 bytes: 8 tokens of one dim) and the
// probabilities from the score tiles with one lane swap per word: lane (c, g) of the 16x16 score
// layout holds keys 4 g .. 4 g + 3 of row c of each tile, and v_permlane16_swap exchanges the odd
// 16-lane rows of one register with the even rows of another, which puts tile 0's keys 0..7 and
// 8..15 of row c on lanes c and c + 32 and tile 1's on lanes c + 16 and c + 48.
typedef float float16_t __attribute__((ext_vector_type(16)));

template <int D>
struct WaveAccWide {
  static constexpr int NB = D / 32;
  float m[2];            // running max per score tile (log2 units), equal on the 4 lanes of a column
  float lsum[2];         // this lane's share of each tile's exp-sum
  float16_t acc[NB];     // O^T for dims 32 b .. 32 b + 31: lane l holds row l % 32 (tile (l / 16) % 2)
};

template <int D>
__device__ __forceinline__ void init_acc(WaveAccWide<D> &s) {
  #pragma unroll
  for (int n = 0; n < 2; ++n) {
    s.m[n] = kNegBig;
    s.lsum[n] = 0.f;
  }
  #pragma unroll
  for (int b = 0; b < WaveAccWide<D>::NB; ++b)
    #pragma unroll
    for (int e = 0; e < 16; ++e) s.acc[b][e] = 0.f;
}

// One 16-token page: the scores, mask and online softmax of mfma_page, then the value product at the
// full rate.  vr[b]: this lane's V^T operand for dims 32 b + l % 32, tokens 8 (l / 32) .. + 7.
template <int D>
__device__ __forceinline__ void mfma_page_wide(const DecodeArgs &a, const SeqInfo &si, int bstart,
                                               const uint4 *kr, uint4 *vr, bool ok, int lane,
                                               const WaveRows<D, 2> &w, WaveAccWide<D> &st) {
  constexpr int NK = D / 32;
  constexpr int NB = D / 32;
  const int grp = lane >> 4;
  float4_t c[2], x[2];
  #pragma unroll
  for (int n = 0; n < 2; ++n) {
    float4_t c4 = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int k = 0; k < NK; ++k)
      c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[k]), w.qB[n][k], c4, 0, 0, 0);
    c[n] = c4;
    #pragma unroll
    for (int e = 0; e < 4; ++e) x[n][e] = fmaf(c4[e], a.scale_log2, -st.m[n]);
  }
  if (!ok || bstart + kBlock > w.first_last + 1) {
    const int pos0 = bstart + 4 * grp;
    #pragma unroll
    for (int n = 0; n < 2; ++n) {
      #pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!ok || pos0 + e > w.last[n]) x[n][e] = -INFINITY;
    }
    const int valid = ok ? si.ctx - bstart : 0;
    if (valid < kBlock) {
      // slots past the context may hold anything (even NaN): zero them so p = 0 adds exactly 0
      const int k0 = 8 * (lane >> 5);
      #pragma unroll
      for (int b = 0; b < NB; ++b) {
        uint32_t wd[4] = {vr[b].x, vr[b].y, vr[b].z, vr[b].w};
        #pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (k0 + 2 * q >= valid) wd[q] = 0u;
          else if (k0 + 2 * q + 1 >= valid) wd[q] &= 0xffffu;
        }
        vr[b] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    }
  }
  static_assert(kRescaleSlack >= 0.f, "the integer comparison needs a non-negative threshold");
  int xbits = __float_as_int(x[0][0]);
  #pragma unroll
  for (int n = 0; n < 2; ++n) {
    #pragma unroll
    for (int e = 0; e < 4; ++e) xbits = max(xbits, __float_as_int(x[n][e]));
  }
  const bool need = xbits > __float_as_int(kRescaleSlack);
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    float alpha[2];
    #pragma unroll
    for (int n = 0; n < 2; ++n) {
      float4_t sc;
      #pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = x[n][e] == -INFINITY ? -INFINITY : c[n][e] * a.scale_log2;
      float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mn = fmaxf(st.m[n], bm);
      alpha[n] = exp2_hw(st.m[n] - mn);
      st.m[n] = mn;
      st.lsum[n] *= alpha[n];
      #pragma unroll
      for (int e = 0; e < 4; ++e) x[n][e] = sc[e] - mn;
    }
    // lane l's accumulator rows are row l % 32 of tile (l / 16) % 2, the same column it holds there
    const float al = (lane & 16) ? alpha[1] : alpha[0];
    #pragma unroll
    for (int b = 0; b < NB; ++b) st.acc[b] *= al;
  }
  uint32_t pw[2][2];
  #pragma unroll
  for (int n = 0; n < 2; ++n) {
    const float p0 = exp2_hw(x[n][0]);
    const float p1 = exp2_hw(x[n][1]);
    const float p2 = exp2_hw(x[n][2]);
    const float p3 = exp2_hw(x[n][3]);
    st.lsum[n] += (p0 + p1) + (p2 + p3);
    pw[n][0] = pack_bf16x2(p0, p1);
    pw[n][1] = pack_bf16x2(p2, p3);
  }
  // even 16-lane rows: own tile-0 keys, then the next row's; odd rows: the previous row's tile-1
  // keys, then their own
  const auto s0 = __builtin_amdgcn_permlane16_swap(pw[0][0], pw[1][0], false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(pw[0][1], pw[1][1], false, false);
  const bf16x8_t pB = __builtin_bit_cast(bf16x8_t, make_uint4(s0[0], s1[0], s0[1], s1[1]));
  #pragma unroll
  for (int b = 0; b < NB; ++b)
    st.acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vr[b]), pB, st.acc[b], 0, 0, 0);
}

// The final output (bf16) and natural-log LSE of the wave's rows from the wide accumulator.
template <int D>
__device__ __forceinline__ void finish_wave_wide(const DecodeArgs &a, int lane, const WaveRows<D, 2> &w,
                                                 const WaveAccWide<D> &st) {
  float l[2];
  #pragma unroll
  for (int n = 0; n < 2; ++n) {
    l[n] = st.lsum[n];
    l[n] += __shfl_xor(l[n], 16);
    l[n] += __shfl_xor(l[n], 32);
  }
  const int t = (lane >> 4) & 1;
  const float lt = t ? l[1] : l[0];
  if ((t ? w.last[1] : w.last[0]) < 0) return;
  const bool seen = lt > 0.f;
  const float inv = seen ? a.v_scale / lt : 0.f;
  const float lse2 = seen ? (t ? st.m[1] : st.m[0]) + log2_hw(lt) : -INFINITY;
  const int64_t orow = t ? w.orow[1] : w.orow[0];
  uint16_t *o = static_cast<uint16_t *>(a.out) + orow * D + 4 * (lane >> 5);
  #pragma unroll
  for (int b = 0; b < WaveAccWide<D>::NB; ++b) {
    #pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v0 = st.acc[b][4 * q] * inv, v1 = st.acc[b][4 * q + 1] * inv;
      const float v2 = st.acc[b][4 * q + 2] * inv, v3 = st.acc[b][4 * q + 3] * inv;
      *reinterpret_cast<uint2 *>(o + 32 * b + 8 * q) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
    }
  }
  if (lane < 32 && a.lse) a.lse[orow] = lse2 * kLn2;
}

// Two E4M3 codes (the low or high half of w) to two bf16 in one instruction: gfx950's scaled
// conversion straight to bf16, at scale 1.  Every E4M3 value is a bf16 value, so it is exact; an
// in-bounds probe over all 256 codes in both halves matched the fp8 -> f32 conversion with its low
// 16 bits dropped (fp8x2_to_bf16x2) bit for bit, NaN codes included.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2_1(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

template <int D, int SP>
struct LdsPages {
  static constexpr int ROWB = D * 2;
  static constexpr int KPAD = ROWB + PKV_LDS_KPAD;   // LDS row stride of a K page
  static constexpr int KBYTES = kBlock * KPAD;
  static constexpr int VROW = kBlock * 2;            // LDS stride of a V dim row (16 tokens)
  static constexpr int VBYTES = D * VROW;
  static constexpr int PBYTES = KBYTES + VBYTES;
  static constexpr int CH = ROWB / 16;               // 16-byte chunks per K row
  static constexpr int BYTES = 2 * SP * PBYTES;
};

// Logical pages [jb, je) of block-table row bt (kv head kvh) through LDS buffer `lds`
// (LdsPages<D, SP>::BYTES).  Every thread of the workgroup must call it (it holds barriers); this
// wave computes the pages j < jw with its rows (jw <= je; a wave with no rows passes jw = jb).
// F8: the pools hold E4M3 codes; each 16-code chunk is widened exactly to bf16 as it is staged, so
// LDS and everything after it are as for bf16 pools (the pools' scales sit in the score scale and
// the epilogue).
// WIDE: the value products at the full rate (mfma_page_wide; st a WaveAccWide, NT = 2), with each V
// dim row's two 8-token halves swapped where bit 3 of the dim is set.
template <int D, int NT, int SP, bool F8 = false, bool WIDE = false, class ST>
__device__ __forceinline__ void lds_stream_pages(const DecodeArgs &a, const SeqInfo &si, int kvh,
                                                 const int32_t *bt, int jb, int je, int jw, char *lds,
                                                 const WaveRows<D, NT> &w, ST &st) {
  typedef LdsPages<D, SP> L;
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  constexpr int EB = F8 ? 1 : 2;               // bytes per cache element
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int n = je - jb;
  if (n <= 0) return;
  const int nstages = (n + SP - 1) / SP;
  const char *kbase = static_cast<const char *>(a.k_cache);
  const char *vbase = static_cast<const char *>(a.v_cache);
  const int64_t page_bytes = (int64_t)kBlock * D * EB;
  // each thread moves 8 elements of every K page and 8 of every V page (a 16-byte chunk of bf16, or
  // 8 bytes of codes); D = 64: threads < 128
  typedef typename std::conditional<F8, uint2, uint4>::type Chunk;
  const bool mover = tid < kBlock * D / 8;
  Chunk kn[SP], vn[SP];
  int okn = 0;                               // bit p: page p of the stage has a valid id
  // block ids through the scalar cache, read a stage before they are used; the page test and page
  // bases stay in scalar registers and each load takes a scalar base plus the thread's 32-bit offset
  // (a block id is an int, so comparing it with the pool size clamped to int range is exact)
  const_i32 *btc = (const_i32 *)(bt + jb);
  const uint32_t nb32 = (uint32_t)min(a.num_blocks, (int64_t)0x7fffffff);
  int nid[SP];
  auto load_ids = [&](int stage) {
    #pragma unroll
    for (int p = 0; p < SP; ++p) nid[p] = btc[__builtin_amdgcn_readfirstlane(min(stage * SP + p, n - 1))];
  };
  auto fetch = [&]() {   // the stage whose ids are in nid; past the end the last page again
    okn = 0;
    #pragma unroll
    for (int p = 0; p < SP; ++p) {
      const int bid = nid[p];
      const bool ok = (uint32_t)bid < nb32;
      okn |= ok ? 1 << p : 0;
      const int64_t page = ((int64_t)(ok ? bid : 0) * a.num_kv_heads + kvh) * page_bytes;
      if (mover) {
        uint32_t to = (uint32_t)tid * (uint32_t)sizeof(Chunk);
        asm volatile("" : "+v"(to));   // keeps the offset 32-bit, so the loads use the scalar base
        kn[p] = *reinterpret_cast<const Chunk *>(kbase + page + to);
        vn[p] = *reinterpret_cast<const Chunk *>(vbase + page + to);
      }
    }
  };
  auto stage_to = [&](int b) {
    if (mover) {
      #pragma unroll
      for (int p = 0; p < SP; ++p) {
        char *pg = lds + (b * SP + p) * L::PBYTES;
        // widened to 8 bf16 (F8: exact), the thread's elements are in the bf16 page's order
        uint4 k8, v8;
        if constexpr (F8) {
          k8 = make_uint4(fp8x2_to_bf16x2_1<false>(kn[p].x), fp8x2_to_bf16x2_1<true>(kn[p].x),
                          fp8x2_to_bf16x2_1<false>(kn[p].y), fp8x2_to_bf16x2_1<true>(kn[p].y));
          v8 = make_uint4(fp8x2_to_bf16x2_1<false>(vn[p].x), fp8x2_to_bf16x2_1<true>(vn[p].x),
                          fp8x2_to_bf16x2_1<false>(vn[p].y), fp8x2_to_bf16x2_1<true>(vn[p].y));
        } else {
          k8 = kn[p];
          v8 = vn[p];
        }
        // K: elements 8 tid .. +7 are dims (8 tid) % D .. +7 of token 8 tid / D
        *reinterpret_cast<uint4 *>(pg + (tid / L::CH) * L::KPAD + (tid % L::CH) * 16) = k8;
        // V: elements 8 tid .. +7 are tokens 8 (tid & 1) .. +7 of dim tid / 2, i.e. its 4-token groups
        // 2 (tid & 1) and 2 (tid & 1) + 1, stored in slots group ^ vswz(dim)
        const int d = tid >> 1;
        char *vrow = pg + L::KBYTES + d * L::VROW;
        if constexpr (WIDE) {
          *reinterpret_cast<uint4 *>(vrow + (((tid & 1) ^ ((d >> 3) & 1)) * 16)) = v8;
        } else {
          const int g0 = ((tid & 1) * 2) ^ vswz(d);
          *reinterpret_cast<uint2 *>(vrow + g0 * 8) = make_uint2(v8.x, v8.y);
          *reinterpret_cast<uint2 *>(vrow + (g0 ^ 1) * 8) = make_uint2(v8.z, v8.w);
        }
      }
    }
  };

  load_ids(0);
  fetch();
  load_ids(1);
  stage_to(0);
  int ok_cur = __builtin_amdgcn_readfirstlane(okn);
  __syncthreads();
  for (int g = 0; g < nstages; ++g) {
    const int b = g & 1;
    if (g + 1 < nstages) {
      fetch();
      load_ids(g + 2);
    }
    #pragma unroll
    for (int p = 0; p < SP; ++p) {
      const int j = jb + g * SP + p;
      if (j < jw) {
        const char *pg = lds + (b * SP + p) * L::PBYTES;
        uint4 kr[NK];
        const char *kl = pg + col * L::KPAD + grp * 16;
        #pragma unroll
        for (int c = 0; c < NK; ++c) kr[c] = *reinterpret_cast<const uint4 *>(kl + c * 64);
        if constexpr (WIDE) {
          // dim l % 32 of each 32-dim block, tokens 8 (l / 32) .. + 7
          const char *vl = pg + L::KBYTES + (lane & 31) * L::VROW + (((lane >> 5) ^ ((lane >> 3) & 1)) * 16);
          uint4 vr[D / 32];
          #pragma unroll
          for (int bk = 0; bk < D / 32; ++bk) vr[bk] = *reinterpret_cast<const uint4 *>(vl + bk * 32 * L::VROW);
          mfma_page_wide<D>(a, si, j * kBlock, kr, vr, ((ok_cur >> p) & 1) != 0, lane, w, st);
        } else {
          uint2 vr[ND];
          const char *vl = pg + L::KBYTES + col * L::VROW;
          #pragma unroll
          for (int t = 0; t < ND; ++t)
            vr[t] = *reinterpret_cast<const uint2 *>(vl + t * 16 * L::VROW + (grp ^ vswz(col + 16 * t)) * 8);
          mfma_page<D, NT>(a, si, j * kBlock, kr, vr, ((ok_cur >> p) & 1) != 0, lane, w, st);
        }
      }
    }
    if (g + 1 < nstages) {
      stage_to(b ^ 1);
      ok_cur = __builtin_amdgcn_readfirstlane(okn);
    }
    __syncthreads();
  }
}

// bf16 pools, D = 128: the same page walk with each stage fetched by gfx950's global-to-LDS loads
// (global_load_lds_dwordx4), so no VGPRs hold pages in flight.  Such a load writes 16 bytes per lane
// to consecutive LDS addresses (lane l at base + 16 l); each lane picks the global 16-byte chunk
// that belongs there.  Page layout in LDS (8 KB): K as four 1 KB blocks of 4 token rows, each row's
// 16-byte chunks placed so that a lane's score operands share one base address (below), with the 16
// rows one K read touches in different banks; V as 128 dim rows of 32 bytes (16 tokens), the two
// chunks of a row swapped where bit 2 of the dim is set (2-way bank conflicts on V reads, the least
// that 16-byte chunks allow).  Two stage buffers are separate LDS arrays, and the walk alternates
// between them with the buffer known at compile time, so the compiler sees that reads of one never
// wait for loads into the other (with a third buffer it no longer does, and waits for every load in
// flight before each page's reads).
template <int SP>
struct DmaPages {
  static constexpr int D = 128;
  static constexpr int KBYTES = kBlock * D * 2;
  static constexpr int PBYTES = 2 * KBYTES;          // K then V
  static constexpr int BYTES = SP * PBYTES;          // one stage buffer
};

// WIDE: the value products at the full rate (mfma_page_wide; st a WaveAccWide, NT = 2), with V rows
// swizzled by bit 3 of the dim so a 16-byte read of 16 consecutive dims hits 16 different bank groups.
template <int NT, int SP, bool WIDE = false, class ST>
__device__ __forceinline__ void lds_stream_pages_dma(const DecodeArgs &a, const SeqInfo &si, int kvh,
                                                     const int32_t *bt, int jb, int je, int jw,
                                                     char *buf0, char *buf1, const WaveRows<128, NT> &w,
                                                     ST &st) {
  typedef DmaPages<SP> L;
  constexpr int D = 128;
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = je - jb;
  if (n <= 0) return;
  const int nstages = (n + SP - 1) / SP;
  const char *kbase = static_cast<const char *>(a.k_cache);
  const char *vbase = static_cast<const char *>(a.v_cache);
  constexpr int64_t page_bytes = (int64_t)kBlock * D * 2;
  // this lane's chunk of the 1 KB K block (rows 4 wave .. + 3) and V block (dims 32 wave .. + 31)
  // that its wave moves for every page.  K block b holds, in 16-byte slot 16 c + 4 ((b + g) & 3) + j,
  // chunk 4 c + g of token row 4 b + j: a lane's four score operands (chunks 4 c + g of its row, c <
  // 4) are then 256 bytes apart, one base address and immediate offsets, and the 16 rows one read
  // touches sit in 16 different bank groups
  const int k_slot_g = ((lane >> 2) - wave) & 3;
  const int k_off = (4 * wave + (lane & 3)) * (D * 2) + (4 * (lane >> 4) + k_slot_g) * 16;
  const int vd = 32 * wave + (lane >> 1);
  const int v_off = vd * (kBlock * 2) + (((lane & 1) ^ ((vd >> (WIDE ? 3 : 2)) & 1)) * 16);
  // block ids of the next stage to fetch, read one stage ahead through the scalar cache (their wait
  // counts no vector loads, and it comes after the stage-end barrier, with no LDS read in flight)
  const_i32 *btc = (const_i32 *)(bt + jb);
  int nid[SP];
  auto ids_of = [&](int g) {
    #pragma unroll
    for (int p = 0; p < SP; ++p) nid[p] = btc[__builtin_amdgcn_readfirstlane(min(g * SP + p, n - 1))];
  };
  // issue the loads of the stage whose ids are in nid into buffer dst; returns bit p set when page p
  // has a valid block id
  // the page test, addresses and LDS targets are wave-uniform: kept in scalar registers, with the
  // lane's part as a 32-bit offset (a block id is an int, so comparing it with the pool size clamped
  // to int range is exact)
  const uint32_t nb32 = (uint32_t)min(a.num_blocks, (int64_t)0x7fffffff);
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t k_off32 = (uint32_t)k_off, v_off32 = (uint32_t)v_off;
  auto fetch = [&](char *dst) -> int {
    int okn = 0;
    // opaque here, so the 32-bit offsets are not widened and hoisted, and the loads take the scalar
    // page base plus a 32-bit lane offset
    uint32_t ko = k_off32, vo = v_off32;
    asm volatile("" : "+v"(ko), "+v"(vo));
    #pragma unroll
    for (int p = 0; p < SP; ++p) {
      const int bid = nid[p];
      // 1 when bid < nb32 as unsigned, in scalar arithmetic (the difference of two values below 2^32
      // is negative exactly then)
      const int okb = (int)((uint64_t)((int64_t)(uint32_t)bid - (int64_t)nb32) >> 63);
      okn |= okb << p;
      const int64_t page = ((int64_t)(bid & -okb) * a.num_kv_heads + kvh) * page_bytes;
      const char *kp = kbase + page;
      const char *vp = vbase + page;
      char *pg = dst + p * L::PBYTES;
      __builtin_amdgcn_global_load_lds(kp + ko, (__attribute__((address_space(3))) void *)(pg + swave * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(vp + vo,
                                       (__attribute__((address_space(3))) void *)(pg + L::KBYTES + swave * 1024), 16, 0, 0);
    }
    return okn;
  };
  // compute the pages of stage g from buffer src
  auto compute = [&](int g, const char *src, int ok_bits) {
    const int j0 = jb + g * SP;
    // the lane's LDS base offsets.  The half-rate page step recomputes them per stage rather than
    // keep them live across the walk: at its register budget the compiler spilled them, and each
    // reload waited on every load in flight, the next stage's included.  The full-rate step has the
    // registers to keep them (230.9 against 233.2 us on the chunked-prefill batch).
    int ln = lane;
    if constexpr (!WIDE) asm volatile("" : "+v"(ln));
    const int cl = ln & 15;
    const int gl = ln >> 4;
    const int kb = (cl >> 2) * 1024 + ((((cl >> 2) + gl) & 3) * 4 + (cl & 3)) * 16;
    const int vb = cl * (kBlock * 2) + ((gl >> 1) ^ ((cl >> 2) & 1)) * 16 + (gl & 1) * 8;
    // WIDE: dim l % 32 of each 32-dim block, tokens 8 (l / 32) .. + 7
    const int vw = (ln & 31) * (kBlock * 2) + (((ln >> 5) ^ ((ln >> 3) & 1)) * 16);
    #pragma unroll
    for (int p = 0; p < SP; ++p) {
      if (j0 + p < jw) {
        const char *pg = src + p * L::PBYTES;
        uint4 kr[NK];
        #pragma unroll
        for (int c = 0; c < NK; ++c) kr[c] = *reinterpret_cast<const uint4 *>(pg + kb + c * 256);
        if constexpr (WIDE) {
          uint4 vr[D / 32];
          #pragma unroll
          for (int b = 0; b < D / 32; ++b)
            vr[b] = *reinterpret_cast<const uint4 *>(pg + L::KBYTES + vw + b * 32 * (kBlock * 2));
          mfma_page_wide<D>(a, si, (j0 + p) * kBlock, kr, vr, ((ok_bits >> p) & 1) != 0, lane, w, st);
        } else {
          uint2 vr[ND];
          #pragma unroll
          for (int t = 0; t < ND; ++t)
            vr[t] = *reinterpret_cast<const uint2 *>(pg + L::KBYTES + vb + t * 16 * (kBlock * 2));
          mfma_page<D, NT>(a, si, (j0 + p) * kBlock, kr, vr, ((ok_bits >> p) & 1) != 0, lane, w, st);
        }
      }
    }
  };

  ids_of(0);
  int ok0 = fetch(buf0);
  if (nstages > 1) ids_of(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int g = 0; g < nstages; g += 2) {
    // even stage from buf0 while the next one lands in buf1
    int ok1 = 0;
    if (g + 1 < nstages) ok1 = fetch(buf1);
    if (g + 2 < nstages) ids_of(g + 2);
    compute(g, buf0, ok0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads into buf1 have landed
    __syncthreads();
    if (g + 1 >= nstages) break;
    // odd stage from buf1 while the next one lands in buf0
    if (g + 2 < nstages) ok0 = fetch(buf0);
    if (g + 3 < nstages) ids_of(g + 3);
    compute(g + 1, buf1, ok1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

}  // namespace pkv
