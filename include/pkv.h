/*
 * pkv.h — C ABI of the paged-KV decode-attention library (libpkv.so), written for AMD CDNA4 (gfx950).
 *
 * What the library computes
 * -------------------------
 * The inferd page describes a paged KV cache as a block allocator plus a page table and keeps a plain
 * paged-attention reference next to it (repository tree; its results table shows the paged path equal
 * to the unpaged one).  The lfm25-inference page ("Runtime Design") runs paged grouped-query (GQA/XQA)
 * decode attention with a split-K reduction, without per-step allocation, over engine-owned KV pages
 * of 16 tokens ("Run Inference": page size 16; page size is a startup policy).  This library is that
 * hot path: the slot-mapped append of new K/V rows into their pages, and decode attention of 1..few
 * new query tokens per sequence over K/V gathered through the block table.
 *
 * For sequence s with context length ctx_s (which COUNTS its q_s new tokens, the last q_s positions),
 * query row i in [0, q_s) and query head h:
 *     kv head  = h / (num_heads / num_kv_heads)
 *     visible  = key positions 0 .. ctx_s - q_s + i            (causal among the new tokens)
 *     out      = softmax_t(scale * <q, K[t]>) . V               (fp32 accumulation)
 *     lse      = ln sum_t exp(scale * <q, K[t]>)                (natural log, fp32)
 *
 * Memory layout (all arrays dense, row-major, device memory owned by the caller):
 *     q, out         [total_q, num_heads, head_dim]        rows packed sequence after sequence
 *     k_cache        [num_blocks, num_kv_heads, block_size, head_dim]   (token rows inside a block)
 *     v_cache        [num_blocks, num_kv_heads, head_dim, block_size]   (dim rows inside a block)
 *     block_tables   int32 [num_seqs, max_blocks_per_seq]  logical block j of sequence s -> physical id
 *     context_lens   int32 [num_seqs]
 *     q_lens         int32 [num_seqs]  or NULL: every sequence has max_q_len new tokens
 *     lse            float [total_q, num_heads]  or NULL
 *     slot_mapping   int64 [num_tokens]  slot = physical_block * block_size + offset; < 0 skips the row
 * Logical token t of sequence s sits in block block_tables[s][t / block_size] at offset t % block_size.
 *
 * Element types: PKV_F32 (q, caches, out all fp32), PKV_BF16 (all bf16) or PKV_BF16_FP8KV (bf16 q
 * and out, E4M3 pools; see below).  head_dim is 64 or 128,
 * block_size is 16.
 *
 * Calls only enqueue work on `stream` (a hipStream_t; NULL = the default stream).  They never allocate,
 * never synchronize and never read device memory on the host.  Host-side validation happens before
 * any launch; a non-zero return means nothing was enqueued (except PKV_ERR_LAUNCH, which reports a
 * failed launch).  Device data is trusted to satisfy the preconditions listed per call; the kernels
 * stay memory-safe when it does not (out-of-range block ids, slots and lengths are skipped or
 * clamped) but the results are then unspecified.  Calls that share output or workspace buffers must
 * not overlap on different streams.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,       /* sizes are inconsistent (e.g. num_heads % num_kv_heads != 0) */
  PKV_ERR_UNSUPPORTED = -3, /* head_dim, block_size, dtype or partition size outside what is built */
  PKV_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than pkv_decode_workspace_bytes(); in
                               pkv_blocks.h: the block pool has too few free blocks */
  PKV_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch */
  PKV_ERR_SCRATCH = -6      /* pkv_paged_attn_decode_noalloc: the call needs more scratch than the
                               library's static scratch holds (PKV_NOALLOC_SCRATCH_BYTES), or its
                               address could not be found on this device */
} pkv_status;

/* PKV_BF16_FP8KV: q, out and appended rows bf16; the K and V pools hold 8-bit E4M3 codes (sign, 4-bit
 * exponent with bias 7, 3-bit mantissa, no infinities, one NaN pattern per sign, largest finite
 * value 448) standing for code * k_scale and code * v_scale (pkv_decode_options; the scales of the
 * pools, 0 meaning 1).  Half the cache bytes of bf16 (lfm25-inference, "Current Scope and
 * Limitations": FP8 KV storage is the step after its BF16 KV cache).  Decode only on the
 * matrix-core persistent schedule. */
typedef enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1, PKV_BF16_FP8KV = 2 } pkv_dtype;

/* Kernel family for the partition pass.  AUTO lets the library choose. */
typedef enum pkv_path { PKV_PATH_AUTO = 0, PKV_PATH_VALU = 1, PKV_PATH_MFMA = 2 } pkv_path;

/* How partition work maps onto the GPU (matrix-core kernel).  GRID: one workgroup per (kv head,
 * partition, sequence, row tile) of a grid sized from the host maxima.  PERSISTENT: a few workgroups
 * per CU; every wave takes an equal share (to within the ring depth) of the K/V pages all work items
 * read, listed from context_lens, so a long sequence is split wherever a share ends and its pieces
 * are merged like partitions (num_seqs <= 4096, ring depth 2 or 4; partitions are optional here).
 * AUTO lets the library choose. */
typedef enum pkv_schedule {
  PKV_SCHEDULE_AUTO = 0, PKV_SCHEDULE_GRID = 1, PKV_SCHEDULE_PERSISTENT = 2
} pkv_schedule;

/* Optional tuning / instrumentation for pkv_paged_attn_decode.  Pass NULL for defaults; a zeroed
 * struct also means defaults. */
typedef struct pkv_decode_options {
  int partition_size;       /* keys per split-K partition, a multiple of block_size; 0 = policy
                               (the persistent schedule then uses none); the grid schedules clamp
                               values above 4096; the persistent schedule rounds up to a multiple of
                               64 */
  int path;                 /* pkv_path */
  int pipeline_depth;       /* MFMA kernel: pages of K/V held per wave (2..4); 0 = policy */
  int schedule;             /* pkv_schedule */
  void *event_main_begin;   /* hipEvent_t recorded on `stream` right before the partition kernel */
  void *event_main_end;     /* hipEvent_t recorded right after it (before the combine kernel) */
  int workgroups_per_cu;    /* persistent schedule: resident workgroups per CU, at most what fits
                               (0 = policy) */
  float k_scale;            /* PKV_BF16_FP8KV: the K pool's scale (0 = 1); ignored otherwise */
  float v_scale;            /* PKV_BF16_FP8KV: the V pool's scale (0 = 1); ignored otherwise */
  int shared_prefix_mode;   /* pkv_paged_attn_decode_shared_prefix only (pkv_prefix.h): a
                               pkv_shared_prefix_mode */
} pkv_decode_options;

typedef enum {
  PKV_PREFIX_AUTO = 0,          /* read shared prefixes once when the bytes that saves are large */
  PKV_PREFIX_READ_ONCE = 1,     /* always attend each group's shared prefix once for the group */
  PKV_PREFIX_PER_SEQUENCE = 2   /* every sequence reads its own pages (pkv_paged_attn_decode) */
} pkv_shared_prefix_mode;

/*
 * Slot-mapped KV append (lfm25-inference, "Runtime Design": engine-owned KV pages; inferd follow-up
 * plan: the block allocator feeding live decode).  For every t in [0, num_tokens) with
 * slot_mapping[t] >= 0:
 *     k_cache[slot / B][h][slot % B][:] = k[t][h][:]      v_cache[slot / B][h][:][slot % B] = v[t][h][:]
 * for all kv heads h.  k, v: [num_tokens, num_kv_heads, head_dim] of `dtype`.  Bits are copied
 * unchanged.  Slots >= num_blocks * block_size are skipped.  Preconditions: non-negative slots are
 * unique (duplicates race); writing into a block several sequences share is the caller's
 * copy-on-write decision.  num_tokens == 0 is a no-op.
 */
int pkv_kv_cache_write(const void *k, const void *v, const int64_t *slot_mapping,
                       void *k_cache, void *v_cache,
                       int64_t num_tokens, int64_t num_blocks,
                       int num_kv_heads, int head_dim, int block_size,
                       int dtype, void *stream);

/*
 * Slot-mapped append into E4M3 pools (PKV_BF16_FP8KV): as pkv_kv_cache_write, but k / v are bf16 and
 * each element is stored as the E4M3 code nearest to x / scale (x widened to fp32, the division
 * correctly rounded in fp32), ties to the even code, magnitudes beyond 448 saturating to 448, NaN to
 * the NaN code of its sign.  k_scale / v_scale > 0.  k_cache [num_blocks, KVH, block_size, head_dim]
 * and v_cache [num_blocks, KVH, head_dim, block_size] of uint8 codes.
 */
int pkv_kv_cache_write_fp8(const void *k, const void *v, const int64_t *slot_mapping,
                           void *k_cache, void *v_cache,
                           int64_t num_tokens, int64_t num_blocks,
                           int num_kv_heads, int head_dim, int block_size,
                           float k_scale, float v_scale, void *stream);

/*
 * Workspace query.  The lfm25-inference page ("Runtime Design") runs its decode without allocating per
 * step, with temporary device memory taken from bounded, reused pools; here the caller owns that
 * memory and this call says how much one decode call needs, so a serving loop sizes it once and
 * reuses it for every step.
 * Bytes of device workspace pkv_paged_attn_decode needs for these sizes and options with its full
 * plan (0 is possible: a single-partition grid launch with uniform q needs none).  The split-K
 * partials take ceil(max_context_len / P) * total_q * num_heads * (head_dim + 1) * 4 bytes; the
 * persistent schedule adds (num_seqs + 1) * 4 bytes and rows_per_tile * (head_dim + 1) * 4 bytes per
 * wave of its grid, and without fixed partitions it keeps piece slots: the first pieces its split
 * cuts from each work item get total_q * num_heads * (head_dim + 1) * 4 bytes each, up to 32 slots
 * (plan_info.piece_slots), plus 4 bytes per work item.  The value depends on the device's CU count.
 * A smaller workspace of at least plan_info.min_workspace_bytes also serves (fewer slots, below).
 */
size_t pkv_decode_workspace_bytes(int num_seqs, int total_q, int max_q_len, int max_context_len,
                                  int num_heads, int num_kv_heads, int head_dim, int dtype,
                                  const pkv_decode_options *opts);

/* What the library will launch for these sizes and options. */
typedef struct pkv_decode_plan_info {
  int partition_size;      /* keys per partition */
  int num_partitions;      /* ceil(max_context_len / partition_size) */
  int path;                /* PKV_PATH_VALU or PKV_PATH_MFMA */
  int rows_per_tile;       /* query rows (heads x new tokens of one kv head) per workgroup */
  int row_tiles;           /* workgroups per (sequence, kv head, partition) */
  int pipeline_depth;      /* MFMA kernel register ring depth */
  int schedule;            /* PKV_SCHEDULE_GRID or PKV_SCHEDULE_PERSISTENT */
  int grid_waves;          /* persistent schedule: waves of its grid on the current device; else 0 */
  size_t workspace_bytes;  /* same value as pkv_decode_workspace_bytes() */
  int item_cost;           /* persistent schedule: stream pages charged to each (sequence, kv head,
                              row tile) work item's start when the page stream is cut into equal
                              shares; else 0 */
  int piece_slots;         /* persistent schedule without fixed partitions: pieces of each work item
                              whose partials sit at fixed rows (the merge reads them with no search);
                              0 = none (every piece past the first in spill rows) */
  size_t min_workspace_bytes;  /* the smallest workspace the call accepts: the plan with no piece
                                  slots (equal to workspace_bytes when the plan has none); added in
                                  ABI 1.1 */
} pkv_decode_plan_info;

/* Fills *info; returns PKV_OK or a negative pkv_status on bad sizes / options. */
int pkv_decode_plan(int num_seqs, int total_q, int max_q_len, int max_context_len, int num_heads,
                    int num_kv_heads, int head_dim, int dtype, const pkv_decode_options *opts,
                    pkv_decode_plan_info *info);

/*
 * Paged decode attention (definition at the top of this file), with a split-K pass over key
 * partitions merged through their log-sum-exp (lfm25-inference, "Runtime Design"): partitions of P
 * tokens, and under the persistent schedule also the pieces its page-balanced split cuts.
 * Preconditions on device data: 1 <= q_lens[s] <= context_lens[s] <= max_context_len,
 * context_lens[s] <= max_blocks_per_seq * block_size, block ids in [0, num_blocks), and
 * sum(q_lens) == total_q (q_lens == NULL: total_q == num_seqs * max_q_len).
 * `workspace` holds pkv_decode_workspace_bytes() bytes for the full plan (may be NULL when that is 0);
 * its contents on entry do not matter.  A workspace_bytes below that but at least
 * plan_info.min_workspace_bytes runs the same kernels with as many piece slots as fit (the results
 * agree within rounding: the merge sums the same partials, found by a search instead of at fixed
 * rows); below the minimum the call returns PKV_ERR_WORKSPACE.
 * `scale` multiplies the raw dot products (usually 1/sqrt(head_dim)).
 */
int pkv_paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *block_tables, const int32_t *context_lens,
                          const int32_t *q_lens, void *out, float *lse,
                          int num_seqs, int max_blocks_per_seq, int total_q, int max_q_len,
                          int max_context_len, int64_t num_blocks,
                          int num_heads, int num_kv_heads, int head_dim, int block_size,
                          float scale, int dtype, const pkv_decode_options *opts,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step with its append: the new tokens' K/V rows are written into their cache slots and
 * attended in the same call (the step a serving engine runs once per generated token; inferd
 * follow-up plan: the block allocator feeding live decode).  new_k / new_v: [total_q, num_kv_heads,
 * head_dim] of `dtype`, packed like q (row qbase_s + i is new token i of sequence s).  Token i of
 * sequence s goes to position p = context_lens[s] - q_lens[s] + i, i.e. block
 * block_tables[s][p / block_size], offset p % block_size (its slot is block * block_size + offset,
 * the slot_mapping a caller of pkv_kv_cache_write would pass).  The result equals
 * pkv_kv_cache_write with those slots followed by pkv_paged_attn_decode, bit for bit.  The matrix-core
 * persistent schedule does both in one pass for up to 8 new tokens per sequence; other launches run
 * a small append kernel first.  PKV_BF16_FP8KV: new_k / new_v are bf16 and are stored as E4M3 codes
 * (quantized as pkv_kv_cache_write_fp8 does, with the options' scales); the result equals
 * pkv_kv_cache_write_fp8 followed by pkv_paged_attn_decode, bit for bit; up to 8 new tokens per
 * sequence (PKV_ERR_UNSUPPORTED above).  Extra precondition: no other sequence of the batch reads the new
 * tokens' slots (a block shared by several sequences is copied before it is appended to).  Other
 * arguments, preconditions and errors as pkv_paged_attn_decode; new_k / new_v NULL -> PKV_ERR_NULL.
 */
int pkv_paged_attn_decode_append(const void *q, const void *new_k, const void *new_v,
                                 void *k_cache, void *v_cache,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 const int32_t *q_lens, void *out, float *lse,
                                 int num_seqs, int max_blocks_per_seq, int total_q, int max_q_len,
                                 int max_context_len, int64_t num_blocks,
                                 int num_heads, int num_kv_heads, int head_dim, int block_size,
                                 float scale, int dtype, const pkv_decode_options *opts,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): pkv_paged_attn_decode without a workspace argument.  The split-K partials, spill
 * rows and tables the decode keeps in its workspace go to a static device array of the library
 * instead, PKV_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU the library runs on, held until the process
 * ends.  Nothing is allocated: no hipMalloc / hipFree and no allocating library routine.  The call
 * is pkv_paged_attn_decode with a workspace of PKV_NOALLOC_SCRATCH_BYTES bytes: the full plan when it
 * fits (then the results are the same bits as with a workspace of pkv_decode_workspace_bytes()),
 * else the plan with as many piece slots as fit; a call whose plan needs more scratch than that
 * even without slots (plan_info.min_workspace_bytes larger; e.g. fixed partitions over very long
 * batches) returns PKV_ERR_SCRATCH and enqueues nothing.  Every call on one GPU shares that GPU's
 * array, so calls that overlap on one GPU (different streams, or host threads) race: serialize
 * them.  The decode needs nothing in the scratch to start at zero.  Arguments, preconditions, results
 * and the other errors are those of pkv_paged_attn_decode with that workspace, bit for bit.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pkv_paged_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *q_lens, void *out, float *lse,
                                  int num_seqs, int max_blocks_per_seq, int total_q, int max_q_len,
                                  int max_context_len, int64_t num_blocks,
                                  int num_heads, int num_kv_heads, int head_dim, int block_size,
                                  float scale, int dtype, const pkv_decode_options *opts, void *stream);

/* Human-readable text for a pkv_status value (static storage): the error side of the boundary, which,
 * like the lfm25-inference page's runtime ("Runtime Design": an engine that owns its pages and
 * memory), reports a refused call to its caller instead of allocating or failing on the device. */
const char *pkv_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
