/*
 * pkv_blocks.h — the host-side data structures that feed the decode path of libpkv.so: a pool of
 * reference-counted KV blocks, per-sequence block tables that hand out slots for new tokens (with
 * copy-on-write for blocks several sequences share), a radix index that lets a new request reuse
 * the blocks of a cached token prefix, and a GPU kernel that copies whole blocks.
 *
 * What the pages describe: the inferd page keeps a block allocator next to a page table
 * (repository layout, core/paged_cache) and plans to wire it into live decode (follow-up plans:
 * persistent paged runtime KV cache, prefix sharing); the lfm25-inference page lets the engine, not
 * the requests, own the KV pages ("Runtime Design") and reuses KV blocks across conversation turns
 * through a radix tree ("Runtime Design": radix tree multi-turn prefix caching; "Performance &
 * Scalability Evidence": prefix-cache speedup).
 *
 * Blocks hold block_size (16) tokens of every kv head, in the pool layout of pkv.h.  Block ids are
 * int32 in [0, num_blocks).  A block's reference count is the number of holders (sequences and the
 * radix index); a block returns to the free list when its count reaches zero.
 *
 * Threading: the objects are not thread-safe; one owner (the engine's scheduler thread) calls them.
 * Errors: functions return 0 / a count, or a negative pkv_status (pkv.h): PKV_ERR_NULL for a NULL
 * handle or output, PKV_ERR_SHAPE for bad sizes or ids, PKV_ERR_WORKSPACE when the pool has too
 * few free blocks (nothing is changed then).
 */
#ifndef PKV_BLOCKS_H
#define PKV_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_pool pkv_block_pool;
typedef struct pkv_seq pkv_seq;
typedef struct pkv_radix pkv_radix;

/* ---- block pool ---- */
pkv_block_pool *pkv_block_pool_create(int32_t num_blocks);
void pkv_block_pool_destroy(pkv_block_pool *pool);
int32_t pkv_block_pool_free_count(const pkv_block_pool *pool);
/* reference count of block id (0 when free), or a negative status */
int32_t pkv_block_refcount(const pkv_block_pool *pool, int32_t id);

/* ---- sequences ---- */
/* An empty sequence (no tokens, no blocks) drawing from pool. */
pkv_seq *pkv_seq_create(pkv_block_pool *pool);
/* Releases the sequence's blocks and frees the handle. */
void pkv_seq_destroy(pkv_seq *seq);
int64_t pkv_seq_length(const pkv_seq *seq);
int32_t pkv_seq_num_blocks(const pkv_seq *seq);
/* Copies the sequence's block table (logical block j -> physical id) into row[0 .. min(n, max)). */
int32_t pkv_seq_block_table(const pkv_seq *seq, int32_t *row, int32_t max);
/*
 * Make room for n_tokens new tokens at the end of the sequence and report where they go:
 * slots[i] = block * block_size + offset of token length + i (the slot_mapping of
 * pkv_kv_cache_write).  New blocks come from the pool.  When the last, partly filled block is shared
 * with another holder, the sequence first takes a private copy of it: a new block replaces it in
 * the table, and (copy_src[k], copy_dst[k]) records that its contents must be copied (see
 * pkv_copy_blocks) before the new tokens are written; *n_copies says how many such pairs (0 or 1).
 * All-or-nothing: PKV_ERR_WORKSPACE if the pool cannot supply the blocks.
 */
int32_t pkv_seq_append(pkv_seq *seq, int32_t n_tokens, int64_t *slots, int32_t *copy_src, int32_t *copy_dst,
                       int32_t *n_copies);
/*
 * One decode step's appends in one call: pkv_seq_append for seqs[0], seqs[1], ... in that order,
 * n_tokens[i] tokens each (0 allowed).  slots receives every sequence's slots back to back (the
 * slot_mapping of the step, Σ n_tokens entries); copy_src / copy_dst (room for n_seqs pairs) receive
 * the copies the step needs, *n_copies their number.  The sequences must be distinct handles
 * (PKV_ERR_SHAPE otherwise).  All-or-nothing: the blocks the whole step needs are counted first,
 * and PKV_ERR_WORKSPACE leaves every sequence unchanged.  Returns Σ n_tokens.
 */
int64_t pkv_seqs_append(pkv_seq *const *seqs, int32_t n_seqs, const int32_t *n_tokens, int64_t *slots,
                        int32_t *copy_src, int32_t *copy_dst, int32_t *n_copies);
/* A new sequence sharing all of seq's blocks (each block's count goes up by one). */
pkv_seq *pkv_seq_fork(const pkv_seq *seq);
/*
 * Start an empty sequence on a cached prefix: its first n_blocks blocks are blocks[0 .. n_blocks),
 * full (n_blocks * block_size tokens); each gains a reference.
 */
int32_t pkv_seq_adopt_prefix(pkv_seq *seq, const int32_t *blocks, int32_t n_blocks);

/* ---- radix prefix index ---- */
/* An index over token-id prefixes in whole blocks, holding references to the blocks it caches. */
pkv_radix *pkv_radix_create(pkv_block_pool *pool);
/* Releases every cached block and frees the index. */
void pkv_radix_destroy(pkv_radix *index);
/*
 * Longest cached prefix of tokens[0 .. n) in whole blocks: writes its blocks to blocks[0 .. r) and
 * returns r (tokens matched = r * block_size).  Marks the matched path as used now (LRU).
 */
int32_t pkv_radix_match(pkv_radix *index, const int32_t *tokens, int64_t n, int32_t *blocks, int32_t max_blocks);
/*
 * Cache the blocks that hold tokens[0 .. n) (n / block_size whole blocks; a partial last block is
 * not cached): blocks[j] holds tokens [j * block_size, (j + 1) * block_size).  Blocks already cached
 * for the same tokens are kept; new ones gain a reference.  Returns the number of blocks newly cached.
 */
int32_t pkv_radix_insert(pkv_radix *index, const int32_t *tokens, int64_t n, const int32_t *blocks);
/*
 * Free up to n_blocks blocks that only the index holds, least recently used leaves first.  Returns
 * how many blocks went back to the pool.
 */
int32_t pkv_radix_evict(pkv_radix *index, int32_t n_blocks);
int32_t pkv_radix_cached_blocks(const pkv_radix *index);

/* ---- device ---- */
/*
 * Copy whole blocks on the GPU: for k < n, block dst[k] of both pools becomes a copy of block
 * src[k] (every kv head, every slot).  Pools in the layout of pkv.h with elem_bytes 4 (fp32), 2 (bf16)
 * or 1 (E4M3 codes); src/dst device arrays of n int32 ids in [0, num_blocks) (others are skipped).
 * dst ids must be distinct and must not appear in src.  Pools start on a 16-byte boundary
 * (PKV_ERR_UNSUPPORTED otherwise).  Enqueued on `stream`; n == 0 enqueues nothing.
 */
int pkv_copy_blocks(void *k_cache, void *v_cache, const int32_t *src, const int32_t *dst, int32_t n,
                    int64_t num_blocks, int num_kv_heads, int head_dim, int elem_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCKS_H */
