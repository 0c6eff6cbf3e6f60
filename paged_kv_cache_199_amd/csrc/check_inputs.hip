// Device-side check of the decode preconditions (include/pkv_check.h): lengths and the block ids a
// decode would read, counted and reported, never trapped on.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

#include "pkv.h"
#include "pkv_check.h"

namespace pkv {

namespace {

constexpr int kCheckBlock = 16;

// The first precondition sequence s breaks (pkv_check_reason) and its offending value; lengths and
// the table row as the caller passed them.  Every lane of the wave calls it: lanes split the table
// row, and the result is wave-uniform.
struct Finding {
  int reason;
  int value;
};

__device__ Finding check_seq(const int32_t *bt, const int32_t *ctx_lens, const int32_t *q_lens, int s,
                             int max_blocks_per_seq, int max_q_len, int max_context_len, int64_t num_blocks,
                             int lane) {
  const int ctx = ctx_lens[s];
  const int q = q_lens ? q_lens[s] : max_q_len;
  if (q < 1 || q > max_q_len) return {PKV_CHECK_Q_LEN, q};
  if (q > ctx) return {PKV_CHECK_Q_OVER_CONTEXT, ctx};
  if (ctx > max_context_len) return {PKV_CHECK_CONTEXT_LEN, ctx};
  if ((int64_t)ctx > (int64_t)max_blocks_per_seq * kCheckBlock) return {PKV_CHECK_CONTEXT_TABLE, ctx};
  // ctx >= q >= 1 and ctx <= max_blocks_per_seq * 16 here, so the row's first nb entries exist
  const int nb = (ctx + kCheckBlock - 1) / kCheckBlock;
  const int32_t *row = bt + (int64_t)s * max_blocks_per_seq;
  for (int j0 = 0; j0 < nb; j0 += 64) {
    const int j = j0 + lane;
    const int id = j < nb ? row[j] : 0;
    const bool bad = j < nb && (id < 0 || (int64_t)id >= num_blocks);
    const uint64_t m = __builtin_amdgcn_ballot_w64(bad);
    if (m) return {PKV_CHECK_BLOCK_ID, __shfl(id, __builtin_ctzll(m))};
  }
  return {PKV_CHECK_OK, 0};
}

__device__ __forceinline__ void atomic_add(int32_t *p, int v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// report = {0, INT_MAX (no sequence yet), 0, 0, 0 (q sum), 0, 0, 0}
__global__ __launch_bounds__(64) void check_init_kernel(int32_t *report) {
  const int t = threadIdx.x;
  if (t < PKV_CHECK_REPORT_INTS) report[t] = t == 1 ? INT_MAX : 0;
}

// One wave per sequence: count the sequences that break a precondition, keep the smallest index,
// and sum q_lens.
__global__ __launch_bounds__(256) void check_scan_kernel(const int32_t *bt, const int32_t *ctx_lens,
                                                          const int32_t *q_lens, int num_seqs, int max_blocks_per_seq,
                                                          int max_q_len, int max_context_len, int64_t num_blocks,
                                                          int32_t *report) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (s >= num_seqs) return;
  const Finding v = check_seq(bt, ctx_lens, q_lens, s, max_blocks_per_seq, max_q_len, max_context_len, num_blocks,
                              lane);
  if (lane == 0) {
    atomic_add(report + 4, q_lens ? q_lens[s] : max_q_len);
    if (v.reason != PKV_CHECK_OK) {
      atomic_add(report + 0, 1);
      __hip_atomic_fetch_min(report + 1, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The first bad sequence's reason and value (checked again), and the q_lens sum against total_q.
__global__ __launch_bounds__(64) void check_final_kernel(const int32_t *bt, const int32_t *ctx_lens,
                                                         const int32_t *q_lens, int max_blocks_per_seq, int total_q,
                                                         int max_q_len, int max_context_len, int64_t num_blocks,
                                                         int32_t *report) {
  const int lane = threadIdx.x;
  const int first = report[1];
  const int qsum = report[4];
  int bad = report[0];
  int reason = PKV_CHECK_OK, value = 0;
  if (first != INT_MAX) {
    const Finding v = check_seq(bt, ctx_lens, q_lens, first, max_blocks_per_seq, max_q_len, max_context_len,
                                num_blocks, lane);
    reason = v.reason;
    value = v.value;
  }
  if (qsum != total_q) {
    ++bad;
    if (first == INT_MAX) {
      reason = PKV_CHECK_Q_TOTAL;
      value = qsum;
    }
  }
  if (lane == 0) {
    report[0] = bad;
    report[1] = first == INT_MAX ? -1 : first;
    report[2] = reason;
    report[3] = value;
  }
}

}  // namespace

}  // namespace pkv

extern "C" int pkv_check_decode_inputs(const int32_t *block_tables, const int32_t *context_lens,
                                       const int32_t *q_lens, int num_seqs, int max_blocks_per_seq, int total_q,
                                       int max_q_len, int max_context_len, int64_t num_blocks, int block_size,
                                       int32_t *report, void *stream) {
  if (!report) return PKV_ERR_NULL;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PKV_ERR_NULL;
  if (block_size != pkv::kCheckBlock) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_blocks_per_seq < 1 || max_q_len < 1 || num_blocks < 0) return PKV_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  pkv::check_init_kernel<<<1, 64, 0, st>>>(report);
  if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
  if (num_seqs > 0) {
    const unsigned grid = (unsigned)((num_seqs + 3) / 4);
    pkv::check_scan_kernel<<<grid, 256, 0, st>>>(block_tables, context_lens, q_lens, num_seqs, max_blocks_per_seq,
                                                 max_q_len, max_context_len, num_blocks, report);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
  }
  pkv::check_final_kernel<<<1, 64, 0, st>>>(block_tables, context_lens, q_lens, max_blocks_per_seq, total_q,
                                            max_q_len, max_context_len, num_blocks, report);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}
