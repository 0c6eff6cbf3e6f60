/*
 * pkv_prefill.h — paged attention for many new tokens per sequence: prompt prefill and chunked
 * prefill over the paged KV cache.
 *
 * The operation is the one pkv_paged_attn_decode computes (definition in pkv.h): new token i of
 * sequence s (query row q_start_s + i) attends key positions 0 .. context_lens[s] - q_lens[s] + i of
 * its block table, the cached tokens and the new tokens up to itself.  The lfm25-inference page runs
 * ragged prefill and paged decode over one engine-owned cache ("Runtime Design"); inferd's
 * follow-up plans list the persistent paged cache feeding the model.  The new tokens' K/V must
 * already sit in the cache (pkv_kv_cache_write with their slots) before the call.
 *
 * This entry point is laid out for hundreds of query rows per (sequence, kv head): each K/V page is
 * fetched once per 128 rows and the matrix cores do the products.  For one or a few new tokens per
 * sequence pkv_paged_attn_decode is the faster call; both give the same result up to rounding order.
 */
#ifndef PKV_PREFILL_H
#define PKV_PREFILL_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Arguments, layouts and preconditions as pkv_paged_attn_decode (q_lens NULL: every sequence has
 * max_q_len new tokens); no workspace.  dtype: PKV_BF16, or PKV_BF16_FP8KV (E4M3 pools, their scales
 * in opts->k_scale / v_scale; opts may be NULL, and its other fields are ignored here).  Writes out
 * [total_q, H, D] and, when lse is not NULL, lse [total_q, H] (natural log).  Errors:
 * PKV_ERR_UNSUPPORTED for another dtype, head_dim or block_size or a bad scale; PKV_ERR_SHAPE /
 * PKV_ERR_NULL as pkv_paged_attn_decode; PKV_ERR_LAUNCH.  Enqueued on `stream`; nothing is allocated
 * or synchronized.
 */
int pkv_paged_attn_prefill(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens, const int32_t *q_lens,
                           void *out, float *lse, int num_seqs, int max_blocks_per_seq, int total_q,
                           int max_q_len, int max_context_len, int64_t num_blocks, int num_heads,
                           int num_kv_heads, int head_dim, int block_size, float scale, int dtype,
                           const pkv_decode_options *opts, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PREFILL_H */
