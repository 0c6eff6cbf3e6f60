// Host side of the C ABI declared in include/pkv.h: argument validation, the split-K / kernel policy,
// workspace carving and kernel launches.  Nothing here allocates, synchronizes or reads device memory.
#include "../../include/pkv.h"
#include "../../include/pkv_prefill.h"
#include "../../include/pkv_prefix.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "decode_args.h"

namespace pkv {
hipError_t launch_kv_write(const void *k, const void *v, const int64_t *slots, void *kc, void *vc,
                           int64_t num_tokens, int64_t num_blocks, int kvh_n, int head_dim, bool bf16,
                           hipStream_t st);
hipError_t launch_decode_valu(const DecodeArgs &a, bool bf16, int head_dim, int rows_per_tile,
                              hipStream_t st);
int valu_max_rows(bool bf16);
hipError_t launch_decode_mfma(const DecodeArgs &a, int head_dim, int rows_per_tile, int depth,
                              bool persistent, int grid, bool f8, hipStream_t st);
hipError_t launch_kv_write_fp8(const void *k, const void *v, const int64_t *slots, void *kc, void *vc,
                               int64_t num_tokens, int64_t num_blocks, int kvh_n, int head_dim, float k_scale,
                               float v_scale, hipStream_t st);
int mfma_rows_per_tile(int rows);
int mfma_default_depth(int head_dim, int rows_per_tile, bool persistent);
int persistent_max_seqs();
int mfma_persistent_wgs_per_cu(int head_dim, int rows_per_tile, int depth, int num_seqs);
hipError_t launch_combine(const DecodeArgs &a, bool bf16, int head_dim, const PrefixArgs *pre, hipStream_t st);
hipError_t launch_kv_append(const DecodeArgs &a, bool bf16, int head_dim, hipStream_t st);
hipError_t launch_q_start(const int32_t *q_lens, int32_t *q_start, int n, hipStream_t st);
hipError_t launch_prefix_attend(const DecodeArgs &a, const PrefixArgs &p, int head_dim, bool f8, hipStream_t st);
hipError_t launch_prefill_mfma(const DecodeArgs &a, int head_dim, bool f8, hipStream_t st);
}  // namespace pkv

namespace {

constexpr int kBlockSize = 16;
// A wave holds the page ids it visits in one register (64 lanes): a partition spans at most 64 pages
// per wave of the 4-wave workgroup, or 64 pages in all when one wave attends a whole partition.
constexpr int kMaxPartition = 64 * 4 * kBlockSize;

int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}
constexpr size_t kAlign = 256;
constexpr int64_t kMaxGrid = (int64_t)1 << 31;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

bool supported_dtype(int dtype) { return dtype == PKV_F32 || dtype == PKV_BF16 || dtype == PKV_BF16_FP8KV; }
bool valid_scale(float s) { return s == 0.f || (s > 0.f && s < 3.0e38f); }
bool supported_head_dim(int d) { return d == 64 || d == 128; }

struct Plan {
  int path;          // PKV_PATH_VALU / PKV_PATH_MFMA
  int rows_per_tile;
  int row_tiles;
  int depth;         // pages of K/V per wave in the register ring (MFMA kernel)
  int schedule;      // PKV_SCHEDULE_GRID / PKV_SCHEDULE_PERSISTENT
  int part_size;
  int num_parts;
  int grid;          // persistent schedule: workgroups (a multiple of 8)
  int item_cost;     // persistent schedule: pages of stream charged to each work item's start
  int64_t part_rows; // partial rows: num_parts * total_q * num_heads, plus the spill rows
  int64_t spill_base;
  int max_pieces;    // persistent schedule without fixed partitions: piece slots per work item (else 0)
  int64_t items;     // work items (sequences x kv heads x row tiles)
  bool need_q_start;
  size_t off_q_start, off_item_pre, off_item_cnt, off_part_lse, off_part_o, bytes;
};

int shape_status(int num_seqs, int total_q, int max_q_len, int max_context_len, int num_heads,
                 int num_kv_heads, int head_dim, int dtype, const pkv_decode_options *opts) {
  if (!supported_dtype(dtype) || !supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || total_q < 0 || max_q_len < 1 || max_context_len < 1) return PKV_ERR_SHAPE;
  if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (max_q_len > max_context_len) return PKV_ERR_SHAPE;
  if (opts) {
    const int P = opts->partition_size;
    if (P < 0 || P % kBlockSize != 0) return PKV_ERR_UNSUPPORTED;
    if (opts->path != PKV_PATH_AUTO && opts->path != PKV_PATH_VALU && opts->path != PKV_PATH_MFMA)
      return PKV_ERR_UNSUPPORTED;
    if (opts->path == PKV_PATH_MFMA && dtype == PKV_F32) return PKV_ERR_UNSUPPORTED;
    if (dtype == PKV_BF16_FP8KV && (opts->path == PKV_PATH_VALU || opts->schedule == PKV_SCHEDULE_GRID))
      return PKV_ERR_UNSUPPORTED;
    if (!valid_scale(opts->k_scale) || !valid_scale(opts->v_scale)) return PKV_ERR_UNSUPPORTED;
    if (opts->pipeline_depth != 0 && (opts->pipeline_depth < 2 || opts->pipeline_depth > 4))
      return PKV_ERR_UNSUPPORTED;
    if (opts->schedule < 0 || opts->schedule > PKV_SCHEDULE_PERSISTENT) return PKV_ERR_UNSUPPORTED;
    if (opts->workgroups_per_cu < 0) return PKV_ERR_UNSUPPORTED;
    if (opts->shared_prefix_mode < PKV_PREFIX_AUTO || opts->shared_prefix_mode > PKV_PREFIX_PER_SEQUENCE)
      return PKV_ERR_UNSUPPORTED;
  }
  return PKV_OK;
}

// Policy.  Kernel: the matrix-core kernel for bf16, the vector-ALU kernel for fp32 (or when asked).
// Rows per tile: the whole GQA group times the new tokens when it fits the kernel, else tiles.
// Schedule: persistent for the matrix-core kernel when its limits allow, else the grid.  Partition
// size: the persistent schedule balances the page stream over its waves by itself and splits a work
// item wherever a share boundary falls, so it takes no partitions of its own unless asked (a given
// size is rounded up to whole ring cycles, 64 keys); the grid schedules take the largest of
// 512/256/128/64 keys that still gives about 2048 live workgroups (8 per CU) for a mean context of
// half the maximum.  No split at all when the whole context fits one partition.
Plan make_plan(int num_seqs, int total_q, int max_q_len, int max_context_len, int num_heads,
               int num_kv_heads, int head_dim, int dtype, bool ragged_q,
               const pkv_decode_options *opts, size_t budget = SIZE_MAX) {
  Plan pl{};
  const bool bf16 = dtype != PKV_F32;
  const int G = num_heads / num_kv_heads;
  const int rows = G * max_q_len;
  const int asked = opts ? opts->path : PKV_PATH_AUTO;
  pl.path = asked == PKV_PATH_AUTO ? (bf16 ? PKV_PATH_MFMA : PKV_PATH_VALU) : asked;
  int R = 1;
  if (pl.path == PKV_PATH_MFMA) {
    R = pkv::mfma_rows_per_tile(rows);
  } else {
    const int rmax = pkv::valu_max_rows(bf16);
    while (R < rows && R < rmax) R <<= 1;
  }
  pl.rows_per_tile = R;
  pl.row_tiles = ceil_div(rows, R);
  const int asked_sched = opts ? opts->schedule : 0;
  // the stream of one kv head is counted in int
  const int64_t stream_pages = (int64_t)num_seqs * pl.row_tiles * ceil_div(max_context_len, kBlockSize);
  const bool can_persist = pl.path == PKV_PATH_MFMA && num_seqs <= pkv::persistent_max_seqs() &&
                           stream_pages * num_kv_heads < ((int64_t)1 << 31);
  pl.schedule = (asked_sched == PKV_SCHEDULE_GRID || !can_persist) ? PKV_SCHEDULE_GRID : PKV_SCHEDULE_PERSISTENT;
  // a wave that starts a work item restarts its page pipeline (new q rows, new block-table row, the
  // first pages' full latency): charging each item 4 pages of stream evens out the waves' finish
  // times.  Measured on conc32 / speculative verify / conc32 over E4M3 pools, step time for 0, 2, 4,
  // 6, 8, 12: 39.6 / 38.7 / 38.6 / 38.4 / 38.3 / 39.1 us, 123.8 / 121.0 / 120.4 / 120.9 / 120.9 /
  // 120.7 us, 34.2 / 33.2 / 32.8 / 32.7 / 32.6 / 33.7 us; long context (items of hundreds of pages)
  // stays within 0.2% up to 4 and loses 0.3-0.5% at 6-8.
  pl.item_cost = pl.schedule == PKV_SCHEDULE_PERSISTENT ? 4 : 0;
  const bool persist = pl.schedule == PKV_SCHEDULE_PERSISTENT;
  // small batches over E4M3 pools: at most 64 pages per wave at one workgroup per CU, bounded from
  // max_context_len.  A page there carries the decode's arithmetic for half the bytes, and a deeper
  // ring keeps more of them in flight per wave (below).
  const int64_t pages_bound =
      (int64_t)num_seqs * num_kv_heads * pl.row_tiles * ceil_div(max_context_len, kBlockSize);
  const bool small_f8 = persist && dtype == PKV_BF16_FP8KV && pages_bound <= 64LL * 4 * cu_count();
  pl.depth = (opts && opts->pipeline_depth) ? opts->pipeline_depth
             : small_f8                       ? 4
                                              : pkv::mfma_default_depth(head_dim, R, persist);
  int P = opts ? opts->partition_size : 0;
  const int whole = ceil_div(max_context_len, kBlockSize) * kBlockSize;
  if (persist) {
    if (P == 0 || P > whole) P = whole;
    P = ceil_div(P, 4 * kBlockSize) * 4 * kBlockSize;
  } else if (P == 0) {
    const int64_t units1 = (int64_t)num_seqs * num_kv_heads * pl.row_tiles;
    const int64_t mean_ctx = (max_context_len + 1) / 2;
    P = 64;
    for (int cand : {512, 256, 128}) {
      if (units1 * ceil_div(mean_ctx, cand) >= 2048) {
        P = cand;
        break;
      }
    }
  }
  if (!persist) {
    if (P >= whole) P = whole;
    if (P > kMaxPartition) P = kMaxPartition;
  }
  pl.part_size = P;
  pl.num_parts = ceil_div(max_context_len, P);
  // with fixed partitions, persistent share boundaries fall on ring cycles that must tile 4 pages
  if (persist && pl.num_parts > 1 && pl.depth == 3) pl.depth = 4;
  pl.grid = 0;
  pl.spill_base = -1;
  pl.part_rows = pl.num_parts > 1 ? (int64_t)pl.num_parts * total_q * num_heads : 0;
  if (persist) {
    // one workgroup per CU unless asked: fewer, longer shares measured faster than a full CU of
    // waves (less per-wave start-up and fewer cut pieces to merge) on all five workloads.  Small
    // batches over E4M3 pools ran two per CU at ring depth 2 (conc32 over E4M3 pools 32.8 -> 31.9
    // us) until the merge read piece slots; since then one per CU at depth 4 is faster there:
    // 26.5 -> 26.1 us in three interleaved repetitions (the decode 0.6 us slower, the merge over
    // 10 slots instead of 18 more than that faster).  Long context over E4M3 pools was 0.8% slower
    // at two.
    const int fits = pkv::mfma_persistent_wgs_per_cu(head_dim, R, pl.depth, num_seqs);
    const int asked_wgs = opts ? opts->workgroups_per_cu : 0;
    const int per_cu = asked_wgs > 0 ? (asked_wgs < fits ? asked_wgs : fits) : 1;
    pl.grid = cu_count() * per_cu / 8 * 8;
    if (pl.grid < 8) pl.grid = 8;
    if (pl.num_parts == 1) {
      // piece slots: the first pieces of every work item go to partition rows, so the merge reads
      // them with no search.  An item's pieces are about the waves per item, more for the longer
      // items: twice that plus two covers the configured batches' longest items (more pieces go
      // to spill rows and the general merge), at most 32; fewer when the workspace is short (below).
      pl.items = (int64_t)num_seqs * num_kv_heads * pl.row_tiles;
      const int64_t per_item = ceil_div((int64_t)pl.grid * 4, pl.items > 0 ? pl.items : 1);
      pl.max_pieces = (int)std::min<int64_t>(32, std::max<int64_t>(4, 2 * per_item + 2));
    }
  }
  pl.need_q_start = ragged_q;   // the combine kernel reads q_start too
  // rows of partials and the workspace layout for pl.max_pieces piece slots; under the persistent
  // schedule every wave of the grid owns rows_per_tile spill rows after the partition rows
  auto lay_out = [&] {
    if (persist) {
      const int64_t first_rows = pl.max_pieces > 1 ? pl.max_pieces : pl.num_parts;
      pl.spill_base = first_rows * total_q * num_heads;
      pl.part_rows = pl.spill_base + (int64_t)pl.grid * 4 * R;
    }
    size_t off = 0;
    pl.off_q_start = off;
    if (ragged_q) off = align_up(off + (size_t)(num_seqs + 1) * 4);
    pl.off_item_pre = off;
    if (persist) off = align_up(off + (size_t)(num_seqs + 1) * 4);
    pl.off_item_cnt = off;
    if (pl.max_pieces > 1) off = align_up(off + (size_t)pl.items * 4);
    pl.off_part_lse = off;
    pl.off_part_o = off;
    if (pl.part_rows > 0) {
      off = align_up(off + (size_t)pl.part_rows * 4);
      pl.off_part_o = off;
      off = align_up(off + (size_t)pl.part_rows * head_dim * 4);
    }
    pl.bytes = off;
  };
  lay_out();
  // a workspace too small for this plan: fewer piece slots, down to none (the pieces past the slots
  // go to spill rows, which the merge finds by its search); each slot costs total_q * num_heads rows
  while (pl.bytes > budget && pl.max_pieces > 1) {
    pl.max_pieces = pl.max_pieces > 2 ? pl.max_pieces - 1 : 0;
    lay_out();
  }
  return pl;
}

}  // namespace

extern "C" {

int pkv_version(void) { return (1 << 16) | 1; }

const char *pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "inconsistent sizes";
    case PKV_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, dtype, path or partition size";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small, or too few free blocks";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_SCRATCH:
      return "the call needs more than the library's static decode scratch (PKV_NOALLOC_SCRATCH_BYTES), "
             "or its device address was not found";
    default: return "unknown status";
  }
}

int pkv_kv_cache_write(const void *k, const void *v, const int64_t *slot_mapping, void *k_cache,
                       void *v_cache, int64_t num_tokens, int64_t num_blocks, int num_kv_heads,
                       int head_dim, int block_size, int dtype, void *stream) {
  if ((dtype != PKV_F32 && dtype != PKV_BF16) || !supported_head_dim(head_dim) || block_size != kBlockSize)
    return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads < 1) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_NULL;
  if (num_tokens * num_kv_heads >= kMaxGrid) return PKV_ERR_SHAPE;
  const hipError_t e = pkv::launch_kv_write(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_blocks,
                                            num_kv_heads, head_dim, dtype == PKV_BF16,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int pkv_kv_cache_write_fp8(const void *k, const void *v, const int64_t *slot_mapping, void *k_cache,
                           void *v_cache, int64_t num_tokens, int64_t num_blocks, int num_kv_heads,
                           int head_dim, int block_size, float k_scale, float v_scale, void *stream) {
  if (!supported_head_dim(head_dim) || block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (!(k_scale > 0.f && k_scale < 3.0e38f) || !(v_scale > 0.f && v_scale < 3.0e38f)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads < 1) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_NULL;
  if (num_tokens * num_kv_heads >= kMaxGrid) return PKV_ERR_SHAPE;
  const hipError_t e = pkv::launch_kv_write_fp8(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_blocks,
                                                num_kv_heads, head_dim, k_scale, v_scale,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

size_t pkv_decode_workspace_bytes(int num_seqs, int total_q, int max_q_len, int max_context_len,
                                  int num_heads, int num_kv_heads, int head_dim, int dtype,
                                  const pkv_decode_options *opts) {
  if (shape_status(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim,
                   dtype, opts) != PKV_OK)
    return 0;
  // sized for ragged q (q_lens given): the q_start table is then part of the workspace
  return make_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim,
                   dtype, true, opts)
      .bytes;
}

int pkv_decode_plan(int num_seqs, int total_q, int max_q_len, int max_context_len, int num_heads,
                    int num_kv_heads, int head_dim, int dtype, const pkv_decode_options *opts,
                    pkv_decode_plan_info *info) {
  if (!info) return PKV_ERR_NULL;
  const int st = shape_status(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                              head_dim, dtype, opts);
  if (st != PKV_OK) return st;
  const Plan pl = make_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                            head_dim, dtype, true, opts);
  info->partition_size = pl.part_size;
  info->num_partitions = pl.num_parts;
  info->path = pl.path;
  info->rows_per_tile = pl.rows_per_tile;
  info->row_tiles = pl.row_tiles;
  info->pipeline_depth = pl.depth;
  info->grid_waves = pl.grid * 4;
  info->schedule = pl.schedule;
  info->workspace_bytes = pl.bytes;
  info->item_cost = pl.item_cost;
  info->piece_slots = pl.max_pieces;
  info->min_workspace_bytes = make_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                                        head_dim, dtype, true, opts, 0)
                                  .bytes;
  return PKV_OK;
}

}  // extern "C"

namespace {

// Shared body of pkv_paged_attn_decode and pkv_paged_attn_decode_append (new_k / new_v NULL: no append),
// and the per-sequence pass of the read-once decode (pre: its prefix pass, merged in the combine).
int decode_impl(const void *q, const void *new_k, const void *new_v, const void *k_cache, const void *v_cache,
                const int32_t *block_tables, const int32_t *context_lens, const int32_t *q_lens, void *out,
                float *lse, int num_seqs, int max_blocks_per_seq, int total_q, int max_q_len,
                int max_context_len, int64_t num_blocks, int num_heads, int num_kv_heads, int head_dim,
                int block_size, float scale, int dtype, const pkv_decode_options *opts, void *workspace,
                size_t workspace_bytes, void *stream, const pkv::PrefixArgs *pre = nullptr) {
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  const int st = shape_status(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                              head_dim, dtype, opts);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || num_blocks < 1) return PKV_ERR_SHAPE;
  if (!q_lens && (int64_t)num_seqs * max_q_len != total_q) return PKV_ERR_SHAPE;
  if (q_lens && total_q < num_seqs) return PKV_ERR_SHAPE;

  const bool bf16 = dtype != PKV_F32;       // the dtype of q and out
  const bool f8 = dtype == PKV_BF16_FP8KV;
  // a workspace short of the full plan's bytes gets the plan with as many piece slots as it holds
  const Plan pl = make_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                            head_dim, dtype, q_lens != nullptr, opts, workspace ? workspace_bytes : 0);
  if (pl.bytes > 0 && (!workspace || workspace_bytes < pl.bytes)) return PKV_ERR_WORKSPACE;
  const int64_t units = (int64_t)num_kv_heads * pl.num_parts * num_seqs * pl.row_tiles;
  if (units + 8 >= kMaxGrid || (int64_t)num_seqs * max_q_len * num_heads / 4 + 1 >= kMaxGrid)
    return PKV_ERR_SHAPE;

  char *ws = static_cast<char *>(workspace);
  pkv::DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.q_lens = q_lens;
  a.q_start = pl.need_q_start ? reinterpret_cast<const int32_t *>(ws + pl.off_q_start) : nullptr;
  a.out = out;
  a.lse = lse;
  a.part_lse = pl.part_rows > 0 ? reinterpret_cast<float *>(ws + pl.off_part_lse) : nullptr;
  a.part_o = pl.part_rows > 0 ? reinterpret_cast<float *>(ws + pl.off_part_o) : nullptr;
  const bool persist = pl.schedule == PKV_SCHEDULE_PERSISTENT;
  // E4M3 pools: the matrix-core persistent schedule only; an append in the same call only where that
  // kernel does it itself (up to 8 new tokens per sequence)
  if (f8 && (pl.path != PKV_PATH_MFMA || !persist || (new_k && max_q_len > 8))) return PKV_ERR_UNSUPPORTED;
  a.item_pre = persist ? reinterpret_cast<int32_t *>(ws + pl.off_item_pre) : nullptr;
  a.spill_base = pl.spill_base;
  a.share_waves = pl.grid / 8 * 4;
  // share boundaries must start ring cycles only where a partition end could fall inside a run
  a.cut_align = pl.num_parts > 1 ? pl.depth : 1;
  a.item_cost = pl.item_cost;
  a.rows_per_tile = pl.rows_per_tile;
  a.max_pieces = pl.max_pieces;
  a.item_cnt = pl.max_pieces > 1 ? reinterpret_cast<int32_t *>(ws + pl.off_item_cnt) : nullptr;
  // the persistent matrix-core kernel appends in its own pass (up to 8 new tokens per sequence);
  // every other launch appends with a small kernel first
  const bool appending = new_k != nullptr;
  const bool fused_append = appending && persist && pl.path == PKV_PATH_MFMA && max_q_len <= 8;
  a.new_k = new_k;
  a.new_v = new_v;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.max_context_len = max_context_len;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.v_scale = 1.f;
  a.k_scale = 1.f;
  if (f8) {
    // the pools' scales factor out of the products: K's into the scores, V's into the epilogue
    const float ks = opts && opts->k_scale > 0.f ? opts->k_scale : 1.f;
    a.scale_log2 *= ks;
    a.k_scale = ks;
    a.v_scale = opts && opts->v_scale > 0.f ? opts->v_scale : 1.f;
  }
  a.part_size = pl.part_size;
  a.num_parts = pl.num_parts;
  a.row_tiles = pl.row_tiles;
  a.units = (int)units;
  a.per_xcd = ceil_div(units, 8);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pl.need_q_start) {
    if (pkv::launch_q_start(q_lens, reinterpret_cast<int32_t *>(ws + pl.off_q_start), num_seqs, s) !=
        hipSuccess)
      return PKV_ERR_LAUNCH;
  }
  if (appending && !fused_append) {
    if (pkv::launch_kv_append(a, bf16, head_dim, s) != hipSuccess) return PKV_ERR_LAUNCH;
  }
  if (!fused_append) {
    a.new_k = nullptr;
    a.new_v = nullptr;
  }
  if (opts && opts->event_main_begin &&
      hipEventRecord(static_cast<hipEvent_t>(opts->event_main_begin), s) != hipSuccess)
    return PKV_ERR_LAUNCH;
  const hipError_t le =
      pl.path == PKV_PATH_MFMA
          ? pkv::launch_decode_mfma(a, head_dim, pl.rows_per_tile, pl.depth, persist, pl.grid, f8, s)
          : pkv::launch_decode_valu(a, bf16, head_dim, pl.rows_per_tile, s);
  if (le != hipSuccess) return PKV_ERR_LAUNCH;
  if (opts && opts->event_main_end &&
      hipEventRecord(static_cast<hipEvent_t>(opts->event_main_end), s) != hipSuccess)
    return PKV_ERR_LAUNCH;
  if (pl.num_parts > 1 || persist || pre) {
    if (pkv::launch_combine(a, bf16, head_dim, pre, s) != hipSuccess) return PKV_ERR_LAUNCH;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *block_tables, const int32_t *context_lens,
                          const int32_t *q_lens, void *out, float *lse, int num_seqs,
                          int max_blocks_per_seq, int total_q, int max_q_len, int max_context_len,
                          int64_t num_blocks, int num_heads, int num_kv_heads, int head_dim,
                          int block_size, float scale, int dtype, const pkv_decode_options *opts,
                          void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl(q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse,
                     num_seqs, max_blocks_per_seq, total_q, max_q_len, max_context_len, num_blocks, num_heads,
                     num_kv_heads, head_dim, block_size, scale, dtype, opts, workspace, workspace_bytes,
                     stream);
}

}  // extern "C"

// Static decode scratch of pkv_paged_attn_decode_noalloc: one copy per GPU, owned by the library until
// the process ends.  In host code `scratch` names a host-side stand-in, not device memory: its device
// address on the current GPU comes from hipGetSymbolAddress, taken once per device and kept.
static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, or nullptr.
void *scratch_on_current_device() {
  static std::mutex mu;
  static void *addr[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int pkv_paged_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *q_lens, void *out, float *lse, int num_seqs,
                                  int max_blocks_per_seq, int total_q, int max_q_len, int max_context_len,
                                  int64_t num_blocks, int num_heads, int num_kv_heads, int head_dim,
                                  int block_size, float scale, int dtype, const pkv_decode_options *opts,
                                  void *stream) {
  // the decode's own validation first, so a bad call fails the same way as pkv_paged_attn_decode
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  const int st = shape_status(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                              head_dim, dtype, opts);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  // the plan decode_impl makes for a workspace of the scratch's size
  const Plan pl = make_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim,
                            dtype, q_lens != nullptr, opts, PKV_NOALLOC_SCRATCH_BYTES);
  if (pl.bytes > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  void *ws = scratch_on_current_device();
  if (!ws) return PKV_ERR_SCRATCH;
  return decode_impl(q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse,
                     num_seqs, max_blocks_per_seq, total_q, max_q_len, max_context_len, num_blocks, num_heads,
                     num_kv_heads, head_dim, block_size, scale, dtype, opts, ws, PKV_NOALLOC_SCRATCH_BYTES,
                     stream);
}

int pkv_paged_attn_decode_append(const void *q, const void *new_k, const void *new_v, void *k_cache,
                                 void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                                 const int32_t *q_lens, void *out, float *lse, int num_seqs,
                                 int max_blocks_per_seq, int total_q, int max_q_len, int max_context_len,
                                 int64_t num_blocks, int num_heads, int num_kv_heads, int head_dim,
                                 int block_size, float scale, int dtype, const pkv_decode_options *opts,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  if (num_seqs > 0 && (!new_k || !new_v)) return PKV_ERR_NULL;
  return decode_impl(q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse, num_seqs,
                     max_blocks_per_seq, total_q, max_q_len, max_context_len, num_blocks, num_heads,
                     num_kv_heads, head_dim, block_size, scale, dtype, opts, workspace, workspace_bytes,
                     stream);
}

}  // extern "C"

namespace {

// Read-once shared-prefix decode: workspace carving and the chunking of the prefix pass.
// Bytes the read-once pass must save before it pays: over groups of 16..64 sequences sharing
// 1024..4096 tokens (GQA 4, D 128) the per-sequence / read-once time ratio is 0.91-1.01 at 240-252
// MiB saved and 1.18-1.30 at about 500 MiB (break-even near 250-340 MiB), because the per-sequence
// decode reads the shared pages from the Infinity Cache after the first sequence.
constexpr int64_t kReadOnceBytes = 320ll << 20;
struct PrefixPlan {
  int rows_max, row_tiles, chunk_pages, chunks, sfx_stride;
  int64_t items;
  size_t off_skip, off_sfx_ctx, off_table, off_q_start, off_sfx_lse, off_pre_lse, off_pre_o, off_decode, bytes;
  size_t decode_bytes;
};

int prefix_status(int num_seqs, int total_q, int max_q_len, int max_context_len, int num_heads, int num_kv_heads,
                  int head_dim, int dtype, int num_groups, int max_group_size, int max_prefix_len,
                  const pkv_decode_options *opts) {
  const int st = shape_status(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim,
                              dtype, opts);
  if (st != PKV_OK) return st;
  if (dtype == PKV_F32 || (opts && opts->path == PKV_PATH_VALU)) return PKV_ERR_UNSUPPORTED;
  if (num_groups < 0 || max_prefix_len < 0 || (num_groups > 0 && max_group_size < 1)) return PKV_ERR_SHAPE;
  if (max_prefix_len % kBlockSize != 0) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// The prefix pass: one wave per (group, kv head, chunk, row tile of 32 rows).  Every row tile reads
// its chunk's pages again (from cache when the tiles run together), and every chunk leaves fp32
// partial rows that the merge reads back.  Chunks are cut for about four waves per CU, but no
// smaller than 4 pages per row tile, so a chunk's partials (rows x D x 4 bytes, written and read)
// stay within the bytes of its K/V pages; at most 64 (the merge holds a row's chunk LSEs in one
// wave's lanes).  Measured on 64 sequences x 4096 shared tokens: 8 chunks of 32 pages took 31 us
// for the pass and 6 us for the merge, 32 chunks of 8 pages 37 us and 14 us.
PrefixPlan make_prefix_plan(int num_seqs, int total_q, int max_q_len, int max_context_len, int num_heads,
                            int num_kv_heads, int head_dim, int dtype, int num_groups, int max_group_size,
                            int max_prefix_len, const pkv_decode_options *opts) {
  PrefixPlan pp{};
  const int G = num_heads / num_kv_heads;
  const int groups = num_groups > 0 ? num_groups : 0;
  const int64_t rows = (int64_t)(groups > 0 ? max_group_size : 0) * max_q_len * G;
  pp.rows_max = (int)rows;
  pp.row_tiles = ceil_div(rows, pkv::kPrefixRows);
  const int pages = max_prefix_len / kBlockSize;
  const int64_t base = (int64_t)groups * num_kv_heads * pp.row_tiles;
  int chunks = 1;
  if (base > 0 && pages > 0 && dtype == PKV_BF16_FP8KV) {
    const int64_t want = ceil_div(4LL * cu_count(), base);
    const int most = pages / (4 * pp.row_tiles) > 1 ? pages / (4 * pp.row_tiles) : 1;
    chunks = (int)(want < 1 ? 1 : (want > most ? most : want));
  } else if (base > 0 && pages > 0) {
    // bf16: a workgroup per (chunk, four row tiles); about one workgroup per CU, chunks of at least
    // one 4-page LDS stage.  Measured on 64 sequences behind a 4096-token prefix, step time for 0.5,
    // 1, 2 and 4 workgroups per CU: 74.4, 66.4, 68.2 and 84.8 us (fewer, larger chunks leave fewer
    // partials for the merge to read)
    const int64_t wgs = (int64_t)groups * num_kv_heads * ceil_div(pp.row_tiles, 4);
    const int64_t want = ceil_div((int64_t)cu_count(), wgs);
    const int most = pages / 4 > 1 ? pages / 4 : 1;
    chunks = (int)(want < 1 ? 1 : (want > most ? most : want));
  }
  if (chunks > 64) chunks = 64;
  pp.chunk_pages = pages > 0 ? ceil_div(pages, chunks) : 1;
  pp.chunks = pages > 0 ? ceil_div(pages, pp.chunk_pages) : 0;
  pp.items = base * pp.chunks;
  pp.sfx_stride = ceil_div(max_context_len, kBlockSize);
  size_t off = 0;
  pp.off_skip = off;
  off = align_up(off + (size_t)num_seqs * 4);
  pp.off_sfx_ctx = off;
  off = align_up(off + (size_t)num_seqs * 4);
  pp.off_table = off;
  off = align_up(off + (size_t)num_seqs * pp.sfx_stride * 4);
  pp.off_q_start = off;
  off = align_up(off + (size_t)(num_seqs + 1) * 4);
  pp.off_sfx_lse = off;
  off = align_up(off + (size_t)total_q * num_heads * 4);
  pp.off_pre_lse = off;
  off = align_up(off + (size_t)pp.items * pkv::kPrefixRows * 4);
  pp.off_pre_o = off;
  off = align_up(off + (size_t)pp.items * pkv::kPrefixRows * head_dim * 4);
  pp.off_decode = off;
  pp.decode_bytes = make_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim,
                              dtype, true, opts)
                        .bytes;
  pp.bytes = off + pp.decode_bytes;
  return pp;
}

}  // namespace

extern "C" {

size_t pkv_decode_shared_prefix_workspace_bytes(int num_seqs, int total_q, int max_q_len, int max_context_len,
                                                int num_heads, int num_kv_heads, int head_dim, int dtype,
                                                int num_groups, int max_group_size, int max_prefix_len,
                                                const pkv_decode_options *opts) {
  if (prefix_status(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim, dtype,
                    num_groups, max_group_size, max_prefix_len, opts) != PKV_OK)
    return 0;
  return make_prefix_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim, dtype,
                          num_groups, max_group_size, max_prefix_len, opts)
      .bytes;
}

int pkv_paged_attn_decode_shared_prefix(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *block_tables, const int32_t *context_lens,
                                        const int32_t *q_lens, void *out, float *lse, int num_seqs,
                                        int max_blocks_per_seq, int total_q, int max_q_len, int max_context_len,
                                        int64_t num_blocks, int num_heads, int num_kv_heads, int head_dim,
                                        int block_size, float scale, int dtype, const int32_t *group_starts,
                                        const int32_t *prefix_lens, const int32_t *prefix_blocks,
                                        int num_groups, int max_group_size,
                                        int max_prefix_len, const pkv_decode_options *opts, void *workspace,
                                        size_t workspace_bytes, void *stream) {
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  const int st = prefix_status(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim,
                               dtype, num_groups, max_group_size, max_prefix_len, opts);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (num_groups > 0 && (!group_starts || !prefix_lens || (max_prefix_len > 0 && !prefix_blocks)))
    return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || num_blocks < 1) return PKV_ERR_SHAPE;
  if (!q_lens && (int64_t)num_seqs * max_q_len != total_q) return PKV_ERR_SHAPE;
  if (q_lens && total_q < num_seqs) return PKV_ERR_SHAPE;
  const PrefixPlan pp = make_prefix_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                                         head_dim, dtype, num_groups, max_group_size, max_prefix_len, opts);
  if (!workspace || workspace_bytes < pp.bytes) return PKV_ERR_WORKSPACE;
  // Policy: the shared pass costs two launches more than the per-sequence decode (8 us or more); it
  // pays when the K/V bytes it saves (every member past the first reading the whole prefix) are
  // large enough that even their cache-served reads take longer than that.
  const int mode = opts ? opts->shared_prefix_mode : PKV_PREFIX_AUTO;
  const int64_t saved = (int64_t)(num_groups > 0 ? num_groups : 0) * (max_group_size > 1 ? max_group_size - 1 : 0) *
                        max_prefix_len * num_kv_heads * head_dim * 2 * (dtype == PKV_BF16_FP8KV ? 1 : 2);
  if (mode == PKV_PREFIX_PER_SEQUENCE || (mode == PKV_PREFIX_AUTO && saved < kReadOnceBytes))
    return decode_impl(q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse,
                       num_seqs, max_blocks_per_seq, total_q, max_q_len, max_context_len, num_blocks, num_heads,
                       num_kv_heads, head_dim, block_size, scale, dtype, opts, static_cast<char *>(workspace) +
                       pp.off_decode, pp.decode_bytes, stream);
  if (pp.items + 8 >= kMaxGrid || (int64_t)num_seqs * max_q_len * num_heads + 8 >= kMaxGrid) return PKV_ERR_SHAPE;

  char *ws = static_cast<char *>(workspace);
  pkv::DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.q_lens = q_lens;
  a.out = out;
  a.lse = lse;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.max_context_len = max_context_len;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.v_scale = 1.f;
  if (dtype == PKV_BF16_FP8KV) {
    a.scale_log2 *= opts && opts->k_scale > 0.f ? opts->k_scale : 1.f;
    a.v_scale = opts && opts->v_scale > 0.f ? opts->v_scale : 1.f;
  }
  a.part_size = max_context_len;   // load_seq's partition count is not used here
  a.num_parts = 1;

  pkv::PrefixArgs p{};
  p.group_starts = group_starts;
  p.prefix_lens = prefix_lens;
  p.prefix_blocks = prefix_blocks;
  p.num_groups = num_groups;
  p.max_group_size = max_group_size;
  p.max_prefix_len = max_prefix_len;
  p.rows_max = pp.rows_max;
  p.row_tiles = pp.row_tiles;
  p.chunk_pages = pp.chunk_pages;
  p.chunks = pp.chunks;
  p.skip = reinterpret_cast<int32_t *>(ws + pp.off_skip);
  p.sfx_ctx = reinterpret_cast<int32_t *>(ws + pp.off_sfx_ctx);
  p.sfx_table = reinterpret_cast<int32_t *>(ws + pp.off_table);
  p.sfx_stride = pp.sfx_stride;
  p.q_start = q_lens ? reinterpret_cast<const int32_t *>(ws + pp.off_q_start) : nullptr;
  p.sfx_lse = reinterpret_cast<float *>(ws + pp.off_sfx_lse);
  p.pre_lse = reinterpret_cast<float *>(ws + pp.off_pre_lse);
  p.pre_o = reinterpret_cast<float *>(ws + pp.off_pre_o);
  a.q_start = p.q_start;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_lens && pkv::launch_q_start(q_lens, reinterpret_cast<int32_t *>(ws + pp.off_q_start), num_seqs, s) !=
                    hipSuccess)
    return PKV_ERR_LAUNCH;
  // the shared pass, with the suffix tables built by extra workgroups of the same launch
  if (pkv::launch_prefix_attend(a, p, head_dim, dtype == PKV_BF16_FP8KV, s) != hipSuccess) return PKV_ERR_LAUNCH;
  // every sequence's own keys: the ordinary decode over the suffix tables; its combine merges the
  // prefix chunks in (the merge reads the suffix LSE, so one is kept when the caller wants none)
  return decode_impl(q, nullptr, nullptr, k_cache, v_cache, p.sfx_table, p.sfx_ctx, q_lens, out,
                     lse ? lse : p.sfx_lse, num_seqs, pp.sfx_stride, total_q, max_q_len, max_context_len, num_blocks,
                     num_heads, num_kv_heads, head_dim, block_size, scale, dtype, opts, ws + pp.off_decode,
                     pp.decode_bytes, stream, &p);
}

}  // extern "C"

extern "C" {

int pkv_paged_attn_prefill(const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,
                           const int32_t *context_lens, const int32_t *q_lens, void *out, float *lse, int num_seqs,
                           int max_blocks_per_seq, int total_q, int max_q_len, int max_context_len,
                           int64_t num_blocks, int num_heads, int num_kv_heads, int head_dim, int block_size,
                           float scale, int dtype, const pkv_decode_options *opts, void *stream) {
  if (block_size != kBlockSize || (dtype != PKV_BF16 && dtype != PKV_BF16_FP8KV)) return PKV_ERR_UNSUPPORTED;
  if (opts && (!valid_scale(opts->k_scale) || !valid_scale(opts->v_scale))) return PKV_ERR_UNSUPPORTED;
  const int st = shape_status(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim,
                              dtype, nullptr);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || num_blocks < 1) return PKV_ERR_SHAPE;
  if (!q_lens && (int64_t)num_seqs * max_q_len != total_q) return PKV_ERR_SHAPE;
  if (q_lens && total_q < num_seqs) return PKV_ERR_SHAPE;
  const int G = num_heads / num_kv_heads;
  const int64_t row_blocks = ceil_div((int64_t)max_q_len * G, 128);   // rows per prefill workgroup
  const int64_t units = (int64_t)num_seqs * num_kv_heads * row_blocks;
  if (units + 8 >= kMaxGrid) return PKV_ERR_SHAPE;

  pkv::DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.q_lens = q_lens;
  a.out = out;
  a.lse = lse;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.max_context_len = max_context_len;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = G;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.v_scale = 1.f;
  a.k_scale = 1.f;
  const bool f8 = dtype == PKV_BF16_FP8KV;
  if (f8) {
    // the pools' scales factor out of the products: K's into the scores, V's into the epilogue
    a.k_scale = opts && opts->k_scale > 0.f ? opts->k_scale : 1.f;
    a.scale_log2 *= a.k_scale;
    a.v_scale = opts && opts->v_scale > 0.f ? opts->v_scale : 1.f;
  }
  a.part_size = max_context_len;
  a.num_parts = 1;
  a.row_tiles = (int)row_blocks;
  a.units = (int)units;
  a.per_xcd = ceil_div(units, 8);
  return pkv::launch_prefill_mfma(a, head_dim, f8, static_cast<hipStream_t>(stream)) == hipSuccess ? PKV_OK
                                                                                                    : PKV_ERR_LAUNCH;
}

}  // extern "C"
