// Paged prefill / chunked prefill attention on the matrix cores (bf16, over bf16 or E4M3 pools).
//
// The same operation as decode (every new token of a sequence attends the cached tokens and the new
// tokens up to itself, through the block table), with many new tokens per sequence: a prompt, or a
// chunk of one appended to an existing context.  The lfm25-inference page pairs paged decode with
// ragged prefill over the same cache ("Runtime Design"); the inferd page lists the persistent
// paged cache and a real paged-attention kernel among its follow-up plans.
//
// With hundreds of query rows per (sequence, kv head) the products are dense enough for the matrix
// cores to be the bound, and the K/V pages are reused by every row tile.  So:
//  * one workgroup per (sequence, kv head, block of 128 rows); rows = new tokens x the G query heads
//    of the kv head, in token order; each of its 4 waves owns 32 rows (two 16-row MFMA tiles), so
//    two or three workgroups fit a CU (64 rows per wave, one workgroup per CU, measured slower);
//  * every K/V page is fetched once per workgroup, staged in LDS a few pages at a time (double-
//    buffered: the next stage's loads fly while this one is computed) and read by all four waves;
//  * a workgroup stops at the page holding its last row's last visible key (causal), and a wave
//    skips the pages past its own rows' limit;
//  * per page, each wave runs the decode's matrix-core step (scores, mask, online softmax, P.V);
//    rows end with their final output and natural-log LSE (no split: there are enough workgroups).
// Work units are laid out row block fastest (last row block first), then sequence, then kv head, and
// spread over the XCDs in contiguous ranges: the workgroups that read one (sequence, kv head)'s pages
// share an L2, and every XCD gets the same kv heads' worth of work.
#include "lds_pages.h"

namespace pkv {

// 1: the value products at the full matrix-core rate (lds_pages.h); 0: the decode's half-rate page
// step (272.0 against 252.0 us on the chunked-prefill batch over bf16 pools)
#ifndef PKV_PREFILL_WIDE
#define PKV_PREFILL_WIDE 1
#endif

constexpr int kPrefillNT = 2;                    // 16-row MFMA tiles per wave
constexpr int kPrefillRows = 4 * 16 * kPrefillNT;   // rows per workgroup

// How pages reach LDS, pages per stage, and the waves per SIMD the register allocation aims at.
//  * bf16 pools, D = 128: global-to-LDS loads (no staging registers), three-page stages (2 x 24 KB
//    of LDS per workgroup) and at most 168 VGPRs, so three workgroups share a CU: 11% faster than
//    staging through registers at two waves per SIMD.
//  * E4M3 pools: pages are widened to bf16 on the way, so they pass through registers, which hold
//    half the bytes: two-page stages (34 KB) and at most 168 VGPRs, three workgroups per CU (12%
//    faster than two).
//  * bf16 pools, D = 64: four-page stages through registers; the compiler's allocation already
//    fits three waves per SIMD.
template <int D, bool F8> struct PrefillCfg {
  static constexpr bool DMA = !F8 && D == 128;
  static constexpr bool WIDE = PKV_PREFILL_WIDE;   // value products at the full rate
  static constexpr int SP = DMA ? 3 : F8 ? 2 : 4;
  static constexpr int WAVES_PER_SIMD = DMA || F8 ? 3 : 1;   // 1: no limit beyond the workgroup size
};

// The sequence at position k when the batch is ordered by work, largest first (context length x new
// tokens; ties by index), for batches of up to 64 sequences; else sequence k.  Every wave computes it
// alone: lane t holds sequence t's key and counts the keys that sort before it.
__device__ __forceinline__ int longest_first(const DecodeArgs &a, int k, int lane) {
  const int S = a.num_seqs;
  if (S > 64) return k;
  float key = -1.f;
  if (lane < S) {
    const int ctx = max(min(a.context_lens[lane], a.max_context_len), 0);
    const int q = a.q_lens ? max(a.q_lens[lane], 1) : a.max_q_len;
    key = (float)ctx * (float)q;
  }
  int rank = 0;
  for (int t = 0; t < S; ++t) {
    const float kt = __shfl(key, t);
    rank += (kt > key || (kt == key && t < lane)) ? 1 : 0;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < S && rank == k);
  return hit ? (int)__builtin_ctzll(hit) : k;
}

template <int D, bool F8>
__global__ __launch_bounds__(256, (PrefillCfg<D, F8>::WAVES_PER_SIMD)) void prefill_mfma_kernel(DecodeArgs a) {
  typedef PrefillCfg<D, F8> Cfg;
  constexpr int SP = Cfg::SP;
  constexpr int NT = kPrefillNT;
  constexpr int WROWS = 16 * NT;             // rows per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;

  int u = xcd_unit(blockIdx.x, a.per_xcd);
  if (u >= a.units) return;
  // row blocks in descending order: under the causal limit the last ones read the most pages, and
  // dispatching them first shortens the kernel's tail (bf16 pools 445 -> 437 us, E4M3 447 -> 429 us
  // on the chunked-prefill batch)
  const int rb = a.row_tiles - 1 - u % a.row_tiles;
  u /= a.row_tiles;
  // kv head slowest: each XCD's contiguous range of units then holds whole kv heads across all the
  // sequences (with 8 kv heads, exactly one each), so the XCDs get equal work whatever the mix of
  // context lengths.  Sequence-major, each XCD got two whole sequences of the chunked-prefill batch,
  // the busiest 1.57x the mean, and the kernel waited for it (436 -> 310 us).
  const int kvh = u / a.num_seqs;
  // within the kv head, sequences in decreasing order of work: the longest workgroups start first and
  // the dispatch tail is short (a list-scheduling model of the chunked-prefill batch: makespan 1.20x
  // the ideal in index order, 1.10x longest first; measured 305 -> 297 us, E4M3 pools 303 -> 283 us)
  const int s = longest_first(a, u % a.num_seqs, lane);

  // q rows before sequence s (the workgroup sums q_lens itself: no workspace)
  SeqInfo si = load_seq(a, s);
  if (a.q_lens) {
    __shared__ int part[4];
    int acc = 0;
    for (int t = tid; t < s; t += 256) acc += max(a.q_lens[t], 0);
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    si.qbase = part[0] + part[1] + part[2] + part[3];
  }
  const int G = a.group;
  const int rows = si.qs * G;
  const int wg_row0 = rb * kPrefillRows;
  if (wg_row0 >= rows || si.ctx <= 0) return;
  const int row0 = wg_row0 + wave * WROWS;
  // the pages this workgroup reads: up to its last row's last visible key
  const int wg_last_tok = (min(rows, wg_row0 + kPrefillRows) - 1) / G;
  // wave-uniform bounds held in scalar registers, so the per-page tests against them are scalar
  const int npages = __builtin_amdgcn_readfirstlane((si.ctx - si.qs + wg_last_tok) / kBlock + 1);
  const int my_pages = __builtin_amdgcn_readfirstlane(
      row0 < rows ? (si.ctx - si.qs + (min(rows, row0 + WROWS) - 1) / G) / kBlock + 1 : 0);

  WaveRows<D, NT> w;
  load_rows<D, NT>(a, si, kvh, row0, rows, col, grp, w);
  w.first_last = __builtin_amdgcn_readfirstlane(w.first_last);
  typename std::conditional<Cfg::WIDE, WaveAccWide<D>, WaveAcc<D, NT>>::type st;
  if constexpr (Cfg::WIDE) init_acc<D>(st);
  else init_acc<D, NT>(st);

  const int32_t *bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  if constexpr (Cfg::DMA) {
    __shared__ __attribute__((aligned(16))) char buf0[DmaPages<SP>::BYTES];
    __shared__ __attribute__((aligned(16))) char buf1[DmaPages<SP>::BYTES];
    lds_stream_pages_dma<NT, SP, Cfg::WIDE>(a, si, kvh, bt, 0, npages, my_pages, buf0, buf1, w, st);
  } else {
    __shared__ __attribute__((aligned(16))) char lds[LdsPages<D, SP>::BYTES];
    lds_stream_pages<D, NT, SP, F8, Cfg::WIDE>(a, si, kvh, bt, 0, npages, my_pages, lds, w, st);
  }
  if constexpr (Cfg::WIDE) {
    if (row0 < rows) finish_wave_wide<D>(a, lane, w, st);
  } else {
    if (row0 < rows) finish_wave<D, NT>(a, 0, true, lane, w, st);
  }
}

// f8: E4M3 pools (pages widened to bf16 as they are staged).
hipError_t launch_prefill_mfma(const DecodeArgs &a, int head_dim, bool f8, hipStream_t st) {
  const dim3 grid((unsigned)(a.per_xcd * 8));
  if (head_dim == 64) {
    if (f8) prefill_mfma_kernel<64, true><<<grid, 256, 0, st>>>(a);
    else prefill_mfma_kernel<64, false><<<grid, 256, 0, st>>>(a);
  } else {
    if (f8) prefill_mfma_kernel<128, true><<<grid, 256, 0, st>>>(a);
    else prefill_mfma_kernel<128, false><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace pkv
