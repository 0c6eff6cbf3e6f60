/*
 * pkv_check.h — checking the decode calls' device-side preconditions without attending.
 *
 * pkv_paged_attn_decode and its variants trust the lengths and block tables they are given: the
 * kernels stay memory-safe when those break the preconditions (out-of-range block ids are read as
 * empty pages, lengths are clamped), but the results are then unspecified.  A serving engine that owns
 * its pages (lfm25-inference, "Runtime Design": KV pages managed by the engine, temporary memory in
 * bounded pools) builds these arrays itself; this call lets it, or a test, confirm on the device that
 * a batch satisfies them before it decodes.  It never traps or aborts on bad data: it counts and
 * reports.
 */
#ifndef PKV_CHECK_H
#define PKV_CHECK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Why a sequence (or the batch) breaks the preconditions, in the order they are tested. */
typedef enum pkv_check_reason {
  PKV_CHECK_OK = 0,
  PKV_CHECK_Q_LEN = 1,           /* q_lens[s] < 1 or > max_q_len (value: q_lens[s]) */
  PKV_CHECK_Q_OVER_CONTEXT = 2,  /* q_lens[s] > context_lens[s] (value: context_lens[s]) */
  PKV_CHECK_CONTEXT_LEN = 3,     /* context_lens[s] > max_context_len (value: context_lens[s]) */
  PKV_CHECK_CONTEXT_TABLE = 4,   /* context_lens[s] > max_blocks_per_seq * block_size (value: context_lens[s]) */
  PKV_CHECK_BLOCK_ID = 5,        /* a block id among the sequence's first ceil(context_lens[s] / block_size)
                                    table entries outside [0, num_blocks) (value: the first such id) */
  PKV_CHECK_Q_TOTAL = 6          /* sum of q_lens != total_q (value: the sum, when no sequence broke a
                                    precondition of its own) */
} pkv_check_reason;

/* Ints of the report (int32, device memory owned by the caller). */
#define PKV_CHECK_REPORT_INTS 8

/*
 * Checks, for every sequence s, the preconditions pkv_paged_attn_decode lists on device data:
 * 1 <= q_lens[s] <= max_q_len, q_lens[s] <= context_lens[s] <= max_context_len,
 * context_lens[s] <= max_blocks_per_seq * block_size, and every block id among its first
 * ceil(context_lens[s] / block_size) table entries in [0, num_blocks) (entries past those are not
 * read by the decode and are not checked); and sum(q_lens) == total_q.  q_lens == NULL: every
 * sequence has max_q_len new tokens.
 *
 * report: int32[PKV_CHECK_REPORT_INTS] of device memory, written by the call (its contents on entry
 * do not matter):
 *     report[0]  sequences that break a precondition, plus 1 when the q_lens sum is wrong
 *     report[1]  the first such sequence, or -1
 *     report[2]  its pkv_check_reason (the first one tested that fails; PKV_CHECK_Q_TOTAL when only
 *                the sum is wrong; PKV_CHECK_OK when nothing is)
 *     report[3]  the offending value named under that reason (0 when nothing is wrong)
 *     report[4]  the q_lens sum as read
 *     report[5..7] reserved (written as 0)
 * Three small launches on `stream`; the caller reads the report after synchronizing it.  Calls that
 * share a report must not overlap.  Returns PKV_OK, or before any launch: PKV_ERR_NULL (block_tables,
 * context_lens or report NULL with num_seqs > 0; report NULL), PKV_ERR_SHAPE (num_seqs < 0,
 * max_blocks_per_seq < 1, max_q_len < 1, num_blocks < 0), PKV_ERR_UNSUPPORTED (block_size != 16);
 * PKV_ERR_LAUNCH if a launch fails.
 */
int pkv_check_decode_inputs(const int32_t *block_tables, const int32_t *context_lens, const int32_t *q_lens,
                            int num_seqs, int max_blocks_per_seq, int total_q, int max_q_len,
                            int max_context_len, int64_t num_blocks, int block_size, int32_t *report,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_CHECK_H */
