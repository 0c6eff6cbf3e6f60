// Paged decode attention on the matrix cores (bf16 K/V): the partition pass.
//
// Operation: GQA decode attention over K/V gathered through the block table, one key partition at a
// time, online softmax (inferd page: paged-attention reference beside the page table; lfm25-inference
// page, "Runtime Design": paged GQA/XQA decode with split-K).  A sequence that fits one partition gets
// its final output and LSE here; otherwise each partition leaves a normalized fp32 partial and its
// log2-sum-exp for the combine kernel.  The per-wave matrix-core work lives in mfma_wave.h.
//
// Two schedules:
//  * grid: one 4-wave workgroup per (kv head, partition, sequence, row tile) of a dense grid sized from
//    the host-known maxima; workgroups past a sequence's end exit at once.  The waves of a workgroup
//    take every fourth page of the partition and merge through LDS.
//  * persistent: a grid of a few workgroups per CU.  Every workgroup lists, from context_lens, the
//    pages every work item (kv head, sequence, row tile) reads as one stream, kv-head-major; each
//    wave is an independent worker that takes an equal contiguous share of that stream (each XCD
//    one eighth).  A share boundary inside a work item cuts it into pieces, merged like partitions
//    by the combine kernel, so every wave streams the same number of pages whatever the mix of
//    lengths, the page pipeline restarts only where the sequence changes, and the items that read
//    one kv head's pages (including prefix pages several sequences share) stay under one L2.
//    Fixed partitions are optional here: when asked for, pieces also end at partition boundaries.
#include "mfma_wave.h"

namespace pkv {

template <int D, int NT, int NBUF>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NW = 4;
  constexpr int ND = D / 16;
  constexpr int ROWS = 16 * NT;

  __shared__ float mrg_acc[NW][ROWS][D];
  __shared__ float mrg_m[NW][ROWS];
  __shared__ float mrg_l[NW][ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;

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

  WaveRows<D, NT> w;
  load_rows<D, NT>(a, si, kvh, row0, rows, col, grp, w);
  WaveAcc<D, NT> st;
  init_acc<D, NT>(st);

  const int tok0 = p * a.part_size;
  const int tok1 = min(si.ctx, tok0 + a.part_size);
  const int blk0 = tok0 / kBlock;
  const int nblk = (tok1 - tok0 + kBlock - 1) / kBlock;
  const int niter = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;
  const int32_t *bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  attend_pages<D, NT, NBUF>(a, si, kvh, bt, blk0 + wave, NW, niter, lane, w, st);

  // ---- per-wave state to LDS, then merge the waves
  #pragma unroll
  for (int n = 0; n < NT; ++n) {
    float l = st.lsum[n];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    #pragma unroll
    for (int t = 0; t < ND; ++t) {
      #pragma unroll
      for (int e = 0; e < 4; ++e) mrg_acc[wave][n * 16 + col][t * 16 + 4 * grp + e] = st.acc[n][t][e];
    }
    if (grp == 0) {
      mrg_m[wave][n * 16 + col] = st.m[n];
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
    for (int q = 1; q < NW; ++q) M = fmaxf(M, mrg_m[q][r]);
    float L = 0.f, O = 0.f;
    #pragma unroll
    for (int q = 0; q < NW; ++q) {
      const float sw = exp2_hw(mrg_m[q][r] - M);
      L += mrg_l[q][r] * sw;
      O += mrg_acc[q][r][d] * sw;
    }
    const bool seen = L > 0.f;
    const float o = seen ? O / L : 0.f;
    const float lse2 = seen ? M + log2_hw(L) : -INFINITY;
    const int64_t orow = (int64_t)qrow * a.num_heads + head;
    if (single) {
      static_cast<uint16_t *>(a.out)[orow * D + d] = f32_to_bf16(o);
      if (d == 0 && a.lse) a.lse[orow] = lse2 * kLn2;
    } else {
      const int64_t prow = (int64_t)p * a.total_q * a.num_heads + orow;
      a.part_o[prow * D + d] = o;
      if (d == 0) a.part_lse[prow] = lse2;
    }
  }
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  #pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// LDS tables of the persistent schedule, per sequence s: pre = stream pages of sequences < s (for
// one kv head), ctx = clamped context length, qb = first q row, rts = row tiles, qs = clamped new
// tokens.  Workgroup 0 also leaves pre in the workspace for the combine kernel.
template <int D, int NT, int NBUF, bool APPEND, bool F8>
__global__ __launch_bounds__(256) void decode_mfma_persistent_kernel(DecodeArgs a) {
  constexpr int ROWS = 16 * NT;
  constexpr int APP = 2 * AppendRows<D, F8>::MAXQ * AppendRows<D, F8>::CH;   // staging chunks per wave
  __shared__ uint4 app_lds[APPEND ? 4 : 1][APPEND ? APP : 1];
  extern __shared__ int sh[];
  const int S = a.num_seqs;
  int *pre = sh;              // [S + 1]
  int *tctx = sh + S + 1;     // [S]
  int *tqb = tctx + S;        // [S]
  int *trts = tqb + S;        // [S]
  int *tqs = trts + S;        // [S]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;

  if (wave == 0) {
    const bool publish = blockIdx.x == 0;
    int run_pages = 0, run_q = 0;
    for (int base = 0; base < S; base += 64) {
      const int s = base + lane;
      int ctx = 0, qs = 0, qraw = 0, pages = 0, rt = 1;
      if (s < S) {
        ctx = min(min(a.context_lens[s], a.max_context_len), a.max_blocks_per_seq * kBlock);
        ctx = max(ctx, 0);
        qraw = max(a.q_lens ? a.q_lens[s] : a.max_q_len, 0);
        qs = max(1, min(qraw, ctx));
        rt = (qs * G + ROWS - 1) / ROWS;
        const int nb = (ctx + kBlock - 1) / kBlock;
        pages = nb > 0 ? (nb + a.item_cost) * rt : 0;
      }
      const int inc_pages = wave_incl_scan(pages, lane);
      const int inc_q = wave_incl_scan(qraw, lane);
      if (s < S) {
        pre[s + 1] = run_pages + inc_pages;
        if (publish) a.item_pre[s + 1] = run_pages + inc_pages;
        tctx[s] = ctx;
        tqb[s] = run_q + inc_q - qraw;
        trts[s] = rt;
        tqs[s] = qs;
      }
      run_pages += __shfl(inc_pages, 63);
      run_q += __shfl(inc_q, 63);
    }
    if (lane == 0) {
      pre[0] = 0;
      if (publish) a.item_pre[0] = 0;
    }
  }
  __syncthreads();

  const int I = pre[S];                             // stream pages per kv head
  const int64_t L = (int64_t)I * a.num_kv_heads;
  const int W = a.share_waves;
  const int NW = 8 * W;
  const int N = a.cut_align;
  const int ord = (blockIdx.x & 7) * W + (blockIdx.x >> 3) * 4 + wave;
  const int64_t spill_row0 = a.spill_base + (int64_t)(blockIdx.x * 4 + wave) * ROWS;
  const int PP = a.part_size / kBlock;

  // Sequence holding stream offset r of one kv head: the last s with pre[s] <= r (never an empty
  // one).  r is wave-uniform and all lanes are active; two dependent LDS reads: lanes compare every
  // chunk's first entry (chunks of ceil(S / 64) <= 64 sequences), then the chunk's entries (pre is
  // nondecreasing, so the lanes that pass form a prefix).
  auto seq_of_wave = [&](int r) {
    int c0 = 0, len = S;
    if (S > 64) {
      len = (S + 63) >> 6;
      const int idx = lane * len;
      c0 = (__popcll(__builtin_amdgcn_ballot_w64(idx < S && pre[idx] <= r)) - 1) * len;
    }
    const int idx = c0 + lane;
    return c0 + __popcll(__builtin_amdgcn_ballot_w64(lane < len && idx < S && pre[idx] <= r)) - 1;
  };
  const int C = a.item_cost;
  // Both ends of the share at once: lane 0 cuts share ord's raw start, lane 1 share ord + 1's (the
  // wave's start-up is a chain of dependent arithmetic and LDS reads at one wave per SIMD, with HBM
  // idle).  A raw start in an item's virtual pages moves to the item's start; one on its real pages
  // moves down to a multiple of N pages from the first of them.
  int64_t kb = L;
  if (L > 0) {
    const int64_t b = share_raw(L, NW, ord + (lane & 1));
    const int64_t bc = b < L ? b : L - 1;
    const int kvh = (int)(bc / I);
    const int r = (int)(bc - (int64_t)kvh * I);
    const int s0 = seq_of_wave(__builtin_amdgcn_readlane(r, 0));
    const int s1 = seq_of_wave(__builtin_amdgcn_readlane(r, 1));
    const int s = (lane & 1) ? s1 : s0;
    const int span = (tctx[s] + kBlock - 1) / kBlock + C;
    const int off = (r - pre[s]) % span;        // stream offset in the item
    const int ro = off - C;                     // real page offset (<= 0: the item's virtual pages)
    const int rr = ro > 0 ? ro - ro % N : 0;
    if (b < L) kb = bc - off + (rr > 0 ? C + rr : 0);
  }
  const int kb_lo = (int)(uint32_t)kb, kb_hi = (int)(kb >> 32);
  int64_t k = ((int64_t)__builtin_amdgcn_readlane(kb_hi, 0) << 32) | (uint32_t)__builtin_amdgcn_readlane(kb_lo, 0);
  const int64_t k_end =
      ((int64_t)__builtin_amdgcn_readlane(kb_hi, 1) << 32) | (uint32_t)__builtin_amdgcn_readlane(kb_lo, 1);
  // The share walks its work items in stream order.  A piece that covers a whole item of a sequence
  // with one partition is final; any other piece leaves a partial: the row of its partition when it
  // starts a partition, else (only the share's first piece can start inside one) the partition row
  // of its piece index when piece slots are on and it has one, else this wave's spill rows.  The
  // piece that ends an item records the item's piece count when piece slots are on.
  while (k < k_end) {
    const int kvh = (int)(k / I);
    const int r = (int)(k - (int64_t)kvh * I);
    // LDS reads come back in vector registers; the values are wave-uniform, and saying so keeps the
    // block-table row pointer scalar (its page ids then come through the scalar cache)
    const int s = __builtin_amdgcn_readfirstlane(seq_of_wave(r));
    SeqInfo si;
    si.ctx = __builtin_amdgcn_readfirstlane(tctx[s]);
    si.qs = __builtin_amdgcn_readfirstlane(tqs[s]);
    si.qbase = __builtin_amdgcn_readfirstlane(tqb[s]);
    si.nparts = (si.ctx + a.part_size - 1) / a.part_size;
    const int nblk = (si.ctx + kBlock - 1) / kBlock;
    const int span = nblk + C;
    const int local = __builtin_amdgcn_readfirstlane(r - pre[s]);
    const int rt = local / span;
    const int off = local - rt * span;
    const int j0 = max(off - C, 0);               // k is an item start or on a real page
    k += j0 + C - off;                            // stream position of real page j0
    const int run = (int)min((int64_t)(nblk - j0), k_end - k);
    if (run <= 0) break;                          // never taken: boundaries are item starts or real pages

    const int32_t *bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    // appending: does this run reach the new tokens (the sequence's last qs positions)?
    const bool reach = APPEND && (j0 + run) * kBlock > si.ctx - si.qs;
    AppendRows<D, F8> ar;
    if (reach) append_load<D, F8>(a, si, kvh, lane, ar);
    WaveRows<D, NT> w;
    load_rows<D, NT>(a, si, kvh, rt * ROWS, si.qs * G, col, grp, w);
    WaveAcc<D, NT> st;
    init_acc<D, NT>(st);
    int kp = 0;
    stream_pages<D, NT, NBUF, F8>(
        a, si, kvh, bt_row, j0, j0 + run, PP, lane, w, st,
        [&](int part, int first, int end) {
          const bool whole = first == 0 && end == nblk && si.nparts == 1;
          // a piece that starts a partition writes its row; with piece slots there is one partition,
          // so a piece that starts inside it is the run's, and takes slot kp while there is one
          const bool at_part = first % PP == 0;
          const bool slot = !at_part && kp < a.max_pieces;
          finish_wave<D, NT>(a, slot ? kp : part, whole, lane, w, st, at_part || slot ? -1 : spill_row0);
          init_acc<D, NT>(st);
        },
        [&](int j, uint4 *kr, uint2 *vr) {
          if constexpr (APPEND) {
            if (reach) append_patch<D, F8>(j, lane, ar, app_lds[wave], kr, vr);
          }
        },
        [&] {
          // piece slots, worked out while the first pages load: the index of the run's piece in its
          // item (0 at the item's start; only a share's first run starts inside an item); the run
          // that ends the item stores its piece count, which only the merge after this kernel reads
          if (a.max_pieces > 1) {
            if (j0 > 0) {
              const int64_t pos0 = (int64_t)kvh * I + __builtin_amdgcn_readfirstlane(pre[s]) + (int64_t)rt * span;
              kp = __builtin_amdgcn_readfirstlane(piece_index(L, NW, C, pos0, ord, a.max_pieces));
            }
            if (j0 + run == nblk && lane == 0)
              a.item_cnt[((int64_t)s * a.num_kv_heads + kvh) * a.row_tiles + rt] =
                  kp < a.max_pieces ? kp + 1 : a.max_pieces + 1;
          }
        });
    if (reach && rt == 0) append_store<D, F8>(a, kvh, bt_row, j0, j0 + run, lane, ar);
    k += run;
  }
}

// Rows one launch covers per work item: 16 per N tile, at most two N tiles.
int mfma_rows_per_tile(int rows) { return rows > 16 ? 32 : 16; }

// Pages in flight per wave = depth - 1.  Depths 2..4 are built for both schedules; with fixed
// partitions the persistent schedule takes depths that divide the 4-page granule of a partition (2, 4).
// Persistent default: depth 2 (measured best with one workgroup per CU on all five workloads).
int mfma_default_depth(int head_dim, int rows_per_tile, bool persistent) { return persistent ? 2 : 3; }

// Largest batch the persistent schedule lists in LDS, and the LDS it needs.
int persistent_max_seqs() { return 4096; }
size_t persistent_lds_bytes(int num_seqs) { return (size_t)(5 * num_seqs + 1) * sizeof(int); }

template <int D, int NT, bool APPEND, bool F8>
static void launch_persistent(const DecodeArgs &a, int depth, int grid, hipStream_t st) {
  const size_t lds = persistent_lds_bytes(a.num_seqs);
  if (depth == 2) decode_mfma_persistent_kernel<D, NT, 2, APPEND, F8><<<grid, 256, lds, st>>>(a);
  else if (depth == 3) decode_mfma_persistent_kernel<D, NT, 3, APPEND, F8><<<grid, 256, lds, st>>>(a);
  else decode_mfma_persistent_kernel<D, NT, 4, APPEND, F8><<<grid, 256, lds, st>>>(a);
}

// f8: E4M3 pools (persistent schedule only).
template <int D, int NT>
static hipError_t launch_mfma_dn(const DecodeArgs &a, int depth, bool persistent, int grid, bool f8,
                                 hipStream_t st) {
  if (persistent) {
    if (f8 && a.new_k) launch_persistent<D, NT, true, true>(a, depth, grid, st);
    else if (f8) launch_persistent<D, NT, false, true>(a, depth, grid, st);
    else if (a.new_k) launch_persistent<D, NT, true, false>(a, depth, grid, st);
    else launch_persistent<D, NT, false, false>(a, depth, grid, st);
    return hipGetLastError();
  }
  switch (depth) {
    case 2: decode_mfma_kernel<D, NT, 2><<<a.per_xcd * 8, 256, 0, st>>>(a); break;
    case 4: decode_mfma_kernel<D, NT, 4><<<a.per_xcd * 8, 256, 0, st>>>(a); break;
    default: decode_mfma_kernel<D, NT, 3><<<a.per_xcd * 8, 256, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

// Workgroups of one persistent-kernel instance that fit a CU at once.
template <int D, int NT, int NBUF>
static int occupancy_of(int num_seqs) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_persistent_kernel<D, NT, NBUF, false, false>, 256,
                                                   persistent_lds_bytes(num_seqs)) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

template <int D, int NT>
static int occupancy_dn(int depth, int num_seqs) {
  return depth == 2 ? occupancy_of<D, NT, 2>(num_seqs)
                    : depth == 3 ? occupancy_of<D, NT, 3>(num_seqs) : occupancy_of<D, NT, 4>(num_seqs);
}

// Cached per (head_dim, N tiles, depth) and per LDS size class (the tables grow with the batch).
int mfma_persistent_wgs_per_cu(int head_dim, int rows_per_tile, int depth, int num_seqs) {
  static int cache[2][2][5][4];
  const int di = head_dim == 64 ? 0 : 1;
  const int ni = rows_per_tile > 16 ? 1 : 0;
  const int ci = num_seqs <= 512 ? 0 : num_seqs <= 1024 ? 1 : num_seqs <= 2048 ? 2 : 3;
  const int sz = ci == 0 ? 512 : ci == 1 ? 1024 : ci == 2 ? 2048 : 4096;
  int &slot = cache[di][ni][depth][ci];
  if (slot <= 0) {
    if (head_dim == 64)
      slot = rows_per_tile > 16 ? occupancy_dn<64, 2>(depth, sz) : occupancy_dn<64, 1>(depth, sz);
    else
      slot = rows_per_tile > 16 ? occupancy_dn<128, 2>(depth, sz) : occupancy_dn<128, 1>(depth, sz);
  }
  return slot;
}

hipError_t launch_decode_mfma(const DecodeArgs &a, int head_dim, int rows_per_tile, int depth,
                              bool persistent, int grid, bool f8, hipStream_t st) {
  if (head_dim == 64) {
    return rows_per_tile > 16 ? launch_mfma_dn<64, 2>(a, depth, persistent, grid, f8, st)
                              : launch_mfma_dn<64, 1>(a, depth, persistent, grid, f8, st);
  }
  return rows_per_tile > 16 ? launch_mfma_dn<128, 2>(a, depth, persistent, grid, f8, st)
                            : launch_mfma_dn<128, 1>(a, depth, persistent, grid, f8, st);
}

}  // namespace pkv
