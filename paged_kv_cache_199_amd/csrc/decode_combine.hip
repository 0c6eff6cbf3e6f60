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

// One wave per (sequence, new token, head); partition LSEs are in log2 units.  The LSEs of up to 64
// partitions are read at once (one per lane), their max and weight sum are wave reductions, and the
// weights are broadcast from the lane that holds them, so the partial outputs stream with several
// loads in flight instead of one dependent load per partition.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
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
  const SeqInfo si = load_seq(a, s);
  if (si.nparts <= 1 || i >= si.qs) return;
  const int row = si.qbase + i;
  if (row >= a.total_q) return;
  const int64_t stride = (int64_t)a.total_q * H;          // between partitions
  const int64_t base = (int64_t)row * H + h;

  float acc[DPL];
  #pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  float M = -INFINITY;
  for (int p = lane; p < si.nparts; p += 64) M = fmaxf(M, a.part_lse[p * stride + base]);
  M = wave_max(M);
  const float Ms = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  for (int c0 = 0; c0 < si.nparts; c0 += 64) {
    const int pl = c0 + lane;
    const float wl = pl < si.nparts ? exp2_hw(a.part_lse[pl * stride + base] - Ms) : 0.f;
    L += wl;
    const int n = min(64, si.nparts - c0);
    const float *op = a.part_o + (c0 * stride + base) * D + lane;
    int j = 0;
    for (; j + 8 <= n; j += 8) {
      float v[8][DPL];
      #pragma unroll
      for (int u = 0; u < 8; ++u) {
        #pragma unroll
        for (int k = 0; k < DPL; ++k) v[u][k] = op[(j + u) * stride * D + 64 * k];
      }
      #pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wp = __shfl(wl, j + u);
        #pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wp, v[u][k], acc[k]);
      }
    }
    for (; j < n; ++j) {
      const float wp = __shfl(wl, j);
      #pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wp, op[j * stride * D + 64 * k], acc[k]);
    }
  }
  L = wave_sum(L);
  const bool seen = L > 0.f;
  const float inv = seen ? 1.f / L : 0.f;
  #pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const float o = acc[k] * inv;
    if constexpr (BF16) {
      static_cast<uint16_t *>(a.out)[base * D + lane + 64 * k] = f32_to_bf16(o);
    } else {
      static_cast<float *>(a.out)[base * D + lane + 64 * k] = o;
    }
  }
  if (lane == 0 && a.lse) a.lse[base] = seen ? (Ms + log2_hw(L)) * kLn2 : -INFINITY;
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

hipError_t launch_combine(const DecodeArgs &a, bool bf16, int head_dim, hipStream_t st) {
  const int64_t waves = (int64_t)a.num_seqs * a.max_q_len * a.num_heads;
  const int grid = (int)((waves + 3) / 4);
  if (bf16) {
    if (head_dim == 64) combine_kernel<true, 64><<<grid, 256, 0, st>>>(a);
    else combine_kernel<true, 128><<<grid, 256, 0, st>>>(a);
  } else {
    if (head_dim == 64) combine_kernel<false, 64><<<grid, 256, 0, st>>>(a);
    else combine_kernel<false, 128><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_q_start(const int32_t *q_lens, int32_t *q_start, int n, hipStream_t st) {
  q_start_kernel<<<1, 1024, 0, st>>>(q_lens, q_start, n);
  return hipGetLastError();
}

}  // namespace pkv
