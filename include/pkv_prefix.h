/*
 * pkv_prefix.h — paged decode attention that reads each shared prompt prefix once per batch.
 *
 * Background in the pages: lfm25-inference reuses the KV blocks of a common prefix across requests
 * through a radix tree ("Runtime Design"; "Performance & Scalability Evidence": prefix-cache
 * speedup), and splits long-context decode into key partitions merged by their log-sum-exp
 * ("Runtime Design").  inferd lists prefix sharing among its follow-up plans.  Softmax attention
 * over a key set equals the log-sum-exp merge of attention over any partition of that set, so when
 * the sequences of a group hold the same physical blocks for their first tokens, those keys can be
 * attended once for every query row of the group (one matrix-core pass, the group's rows stacked),
 * and merged with each sequence's attention over its own remaining keys.
 *
 * The result is the attention of pkv_paged_attn_decode (definition in pkv.h) for every row, up to
 * floating-point rounding order: the arguments shared with pkv_paged_attn_decode mean the same and
 * carry the same preconditions.
 */
#ifndef PKV_PREFIX_H
#define PKV_PREFIX_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Workspace of pkv_paged_attn_decode_shared_prefix for these sizes and bounds (0 on bad sizes).
 * Sized for ragged q (q_lens given).
 */
size_t pkv_decode_shared_prefix_workspace_bytes(int num_seqs, int total_q, int max_q_len, int max_context_len,
                                                int num_heads, int num_kv_heads, int head_dim, int dtype,
                                                int num_groups, int max_group_size, int max_prefix_len,
                                                const pkv_decode_options *opts);

/*
 * Groups (device arrays, int32):
 *   group_starts [num_groups + 1]: group g is sequences group_starts[g] .. group_starts[g + 1] - 1
 *     (non-decreasing; sequences outside every group have no shared prefix);
 *   prefix_lens [num_groups]: tokens that group g shares, a multiple of 16;
 *   prefix_blocks [num_groups, max_prefix_len / 16]: row g holds the physical ids of group g's shared
 *     blocks (its first prefix_lens[g] / 16 entries are read).
 * Precondition: for every member s, block_tables[s][j] == prefix_blocks[g][j] for j < P_s / 16 (P_s
 * below); a member need not hold the whole prefix.
 * Host-known bounds: max_group_size >= every group's size, max_prefix_len >= every prefix_lens[g]
 * (a multiple of 16).  Members past max_group_size and prefix tokens past max_prefix_len are treated
 * as unshared (still attended, by the per-sequence pass).
 * Sequence s of group g attends the shared pass over its first P_s = min(prefix_lens[g], the whole
 * pages before its new tokens) keys, and the per-sequence pass over the rest.  Pass NULL arrays and
 * num_groups = 0 for a batch without shared prefixes.
 * dtype: PKV_BF16 or PKV_BF16_FP8KV (the matrix-core kernels); path PKV_PATH_VALU is unsupported.
 * Writes out and lse (lse may be NULL).  Errors as pkv_paged_attn_decode, plus PKV_ERR_UNSUPPORTED
 * for a max_prefix_len that is not a multiple of 16, and PKV_ERR_SHAPE for negative counts or
 * num_groups > 0 with max_group_size < 1; PKV_ERR_NULL for a missing group array when num_groups > 0.
 */
int pkv_paged_attn_decode_shared_prefix(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *block_tables, const int32_t *context_lens,
                                        const int32_t *q_lens, void *out, float *lse,
                                        int num_seqs, int max_blocks_per_seq, int total_q, int max_q_len,
                                        int max_context_len, int64_t num_blocks,
                                        int num_heads, int num_kv_heads, int head_dim, int block_size,
                                        float scale, int dtype,
                                        const int32_t *group_starts, const int32_t *prefix_lens,
                                        const int32_t *prefix_blocks, int num_groups, int max_group_size,
                                        int max_prefix_len,
                                        const pkv_decode_options *opts,
                                        void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PREFIX_H */
