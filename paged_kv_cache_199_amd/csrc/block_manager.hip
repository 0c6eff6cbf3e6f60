// Host-side KV block management (include/pkv_blocks.h) and the GPU block copy behind copy-on-write.
//
// The inferd page pairs a block allocator with a page table and plans to wire it into live decode
// (repository layout, core/paged_cache; follow-up plans).  The lfm25-inference page lets the engine
// own the KV pages and reuses them across conversation turns through a radix tree ("Runtime
// Design").  Here: reference-counted blocks, per-sequence tables that hand out slots (taking a
// private copy of a shared, partly filled last block before writing into it), and a radix index
// over 16-token chunks whose leaves are evicted least recently used first.
#include "pkv.h"
#include "pkv_blocks.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cstdint>
#include <map>
#include <memory>
#include <vector>

namespace {
constexpr int kBS = 16;   // tokens per block
}

struct pkv_block_pool {
  std::vector<int32_t> ref;        // holders per block
  std::vector<int32_t> free_ids;   // a stack; the lowest ids come out first

  explicit pkv_block_pool(int32_t n) : ref(n, 0) {
    free_ids.reserve(n);
    for (int32_t i = n - 1; i >= 0; --i) free_ids.push_back(i);
  }
  int32_t alloc() {
    const int32_t id = free_ids.back();
    free_ids.pop_back();
    ref[id] = 1;
    return id;
  }
  void retain(int32_t id) { ++ref[id]; }
  void release(int32_t id) {
    if (--ref[id] == 0) free_ids.push_back(id);
  }
  bool valid(int32_t id) const { return id >= 0 && id < (int32_t)ref.size(); }
};

struct pkv_seq {
  pkv_block_pool *pool;
  std::vector<int32_t> blocks;
  int64_t len = 0;
};

namespace {
typedef std::array<int32_t, kBS> Chunk;

struct RadixNode {
  RadixNode *parent = nullptr;
  Chunk key{};
  int32_t block = -1;
  uint64_t last_used = 0;
  std::map<Chunk, std::unique_ptr<RadixNode>> children;
};
}  // namespace

struct pkv_radix {
  pkv_block_pool *pool;
  RadixNode root;
  uint64_t tick = 0;
  int32_t cached = 0;
};

extern "C" {

pkv_block_pool *pkv_block_pool_create(int32_t num_blocks) {
  if (num_blocks < 0) return nullptr;
  return new pkv_block_pool(num_blocks);
}

void pkv_block_pool_destroy(pkv_block_pool *pool) { delete pool; }

int32_t pkv_block_pool_free_count(const pkv_block_pool *pool) {
  return pool ? (int32_t)pool->free_ids.size() : PKV_ERR_NULL;
}

int32_t pkv_block_refcount(const pkv_block_pool *pool, int32_t id) {
  if (!pool) return PKV_ERR_NULL;
  if (!pool->valid(id)) return PKV_ERR_SHAPE;
  return pool->ref[id];
}

pkv_seq *pkv_seq_create(pkv_block_pool *pool) {
  if (!pool) return nullptr;
  pkv_seq *s = new pkv_seq;
  s->pool = pool;
  return s;
}

void pkv_seq_destroy(pkv_seq *seq) {
  if (!seq) return;
  for (int32_t b : seq->blocks) seq->pool->release(b);
  delete seq;
}

int64_t pkv_seq_length(const pkv_seq *seq) { return seq ? seq->len : PKV_ERR_NULL; }

int32_t pkv_seq_num_blocks(const pkv_seq *seq) { return seq ? (int32_t)seq->blocks.size() : PKV_ERR_NULL; }

int32_t pkv_seq_block_table(const pkv_seq *seq, int32_t *row, int32_t max) {
  if (!seq || (!row && max > 0)) return PKV_ERR_NULL;
  const int32_t n = std::min<int32_t>(max, (int32_t)seq->blocks.size());
  for (int32_t j = 0; j < n; ++j) row[j] = seq->blocks[j];
  return n;
}

int32_t pkv_seq_append(pkv_seq *seq, int32_t n_tokens, int64_t *slots, int32_t *copy_src, int32_t *copy_dst,
                       int32_t *n_copies) {
  if (!seq || !n_copies || (n_tokens > 0 && !slots)) return PKV_ERR_NULL;
  if (n_tokens < 0) return PKV_ERR_SHAPE;
  *n_copies = 0;
  if (n_tokens == 0) return 0;
  pkv_block_pool *pool = seq->pool;
  const int64_t new_len = seq->len + n_tokens;
  const int64_t need_total = (new_len + kBS - 1) / kBS;
  const int32_t fresh = (int32_t)(need_total - (int64_t)seq->blocks.size());
  // writing into a partly filled last block that another holder still reads: copy it first
  const bool cow = seq->len % kBS != 0 && pool->ref[seq->blocks.back()] > 1;
  if (cow && (!copy_src || !copy_dst)) return PKV_ERR_NULL;
  if ((int64_t)pool->free_ids.size() < fresh + (cow ? 1 : 0)) return PKV_ERR_WORKSPACE;
  if (cow) {
    const int32_t old = seq->blocks.back();
    const int32_t mine = pool->alloc();
    copy_src[0] = old;
    copy_dst[0] = mine;
    *n_copies = 1;
    pool->release(old);
    seq->blocks.back() = mine;
  }
  for (int32_t k = 0; k < fresh; ++k) seq->blocks.push_back(pool->alloc());
  for (int32_t i = 0; i < n_tokens; ++i) {
    const int64_t pos = seq->len + i;
    slots[i] = (int64_t)seq->blocks[pos / kBS] * kBS + pos % kBS;
  }
  seq->len = new_len;
  return n_tokens;
}

int64_t pkv_seqs_append(pkv_seq *const *seqs, int32_t n_seqs, const int32_t *n_tokens, int64_t *slots,
                        int32_t *copy_src, int32_t *copy_dst, int32_t *n_copies) {
  if (!n_copies || (n_seqs > 0 && (!seqs || !n_tokens || !copy_src || !copy_dst))) return PKV_ERR_NULL;
  if (n_seqs < 0) return PKV_ERR_SHAPE;
  *n_copies = 0;
  if (n_seqs == 0) return 0;
  pkv_block_pool *pool = nullptr;
  int64_t total = 0;
  std::vector<pkv_seq *> order(seqs, seqs + n_seqs);
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (!seqs[i]) return PKV_ERR_NULL;
    if (n_tokens[i] < 0 || (pool && seqs[i]->pool != pool)) return PKV_ERR_SHAPE;
    pool = seqs[i]->pool;
    total += n_tokens[i];
  }
  std::sort(order.begin(), order.end());
  if (std::adjacent_find(order.begin(), order.end()) != order.end()) return PKV_ERR_SHAPE;
  if (total > 0 && !slots) return PKV_ERR_NULL;
  // count the step's blocks first; an earlier sequence's copy can leave a later sharer sole owner
  std::map<int32_t, int32_t> dropped;
  int64_t need = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const pkv_seq *s = seqs[i];
    if (n_tokens[i] == 0) continue;
    need += (s->len + n_tokens[i] + kBS - 1) / kBS - (int64_t)s->blocks.size();
    if (s->len % kBS != 0) {
      const int32_t last = s->blocks.back();
      if (pool->ref[last] - dropped[last] > 1) {
        ++need;
        ++dropped[last];
      }
    }
  }
  if (need > (int64_t)pool->free_ids.size()) return PKV_ERR_WORKSPACE;
  int64_t off = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    int32_t nc = 0;
    const int32_t r = pkv_seq_append(seqs[i], n_tokens[i], slots + off, copy_src + *n_copies,
                                     copy_dst + *n_copies, &nc);
    if (r < 0) return r;   // not reached: the count above covers every block
    off += n_tokens[i];
    *n_copies += nc;
  }
  return total;
}

pkv_seq *pkv_seq_fork(const pkv_seq *seq) {
  if (!seq) return nullptr;
  pkv_seq *s = new pkv_seq(*seq);
  for (int32_t b : s->blocks) s->pool->retain(b);
  return s;
}

int32_t pkv_seq_adopt_prefix(pkv_seq *seq, const int32_t *blocks, int32_t n_blocks) {
  if (!seq || (n_blocks > 0 && !blocks)) return PKV_ERR_NULL;
  if (n_blocks < 0 || seq->len != 0 || !seq->blocks.empty()) return PKV_ERR_SHAPE;
  for (int32_t j = 0; j < n_blocks; ++j)
    if (!seq->pool->valid(blocks[j]) || seq->pool->ref[blocks[j]] <= 0) return PKV_ERR_SHAPE;
  for (int32_t j = 0; j < n_blocks; ++j) {
    seq->pool->retain(blocks[j]);
    seq->blocks.push_back(blocks[j]);
  }
  seq->len = (int64_t)n_blocks * kBS;
  return n_blocks;
}

pkv_radix *pkv_radix_create(pkv_block_pool *pool) {
  if (!pool) return nullptr;
  pkv_radix *r = new pkv_radix;
  r->pool = pool;
  return r;
}

static void radix_release_all(pkv_radix *r, RadixNode *node) {
  for (auto &kv : node->children) {
    radix_release_all(r, kv.second.get());
    r->pool->release(kv.second->block);
  }
  node->children.clear();
}

void pkv_radix_destroy(pkv_radix *index) {
  if (!index) return;
  radix_release_all(index, &index->root);
  delete index;
}

static Chunk chunk_at(const int32_t *tokens, int64_t j) {
  Chunk c;
  std::copy(tokens + j * kBS, tokens + (j + 1) * kBS, c.begin());
  return c;
}

int32_t pkv_radix_match(pkv_radix *index, const int32_t *tokens, int64_t n, int32_t *blocks, int32_t max_blocks) {
  if (!index || (n > 0 && !tokens) || (max_blocks > 0 && !blocks)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  const uint64_t now = ++index->tick;
  RadixNode *node = &index->root;
  int32_t r = 0;
  for (int64_t j = 0; j < n / kBS && r < max_blocks; ++j) {
    auto it = node->children.find(chunk_at(tokens, j));
    if (it == node->children.end()) break;
    node = it->second.get();
    node->last_used = now;
    blocks[r++] = node->block;
  }
  return r;
}

int32_t pkv_radix_insert(pkv_radix *index, const int32_t *tokens, int64_t n, const int32_t *blocks) {
  if (!index || (n >= kBS && (!tokens || !blocks))) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  for (int64_t j = 0; j < n / kBS; ++j)
    if (!index->pool->valid(blocks[j]) || index->pool->ref[blocks[j]] <= 0) return PKV_ERR_SHAPE;
  const uint64_t now = ++index->tick;
  RadixNode *node = &index->root;
  int32_t added = 0;
  for (int64_t j = 0; j < n / kBS; ++j) {
    const Chunk key = chunk_at(tokens, j);
    auto it = node->children.find(key);
    if (it == node->children.end()) {
      std::unique_ptr<RadixNode> child(new RadixNode);
      child->parent = node;
      child->key = key;
      child->block = blocks[j];
      index->pool->retain(blocks[j]);
      ++added;
      ++index->cached;
      it = node->children.emplace(key, std::move(child)).first;
    }
    node = it->second.get();
    node->last_used = now;
  }
  return added;
}

static void collect_evictable(const pkv_radix *r, RadixNode *node, std::vector<RadixNode *> &out) {
  for (auto &kv : node->children) {
    RadixNode *c = kv.second.get();
    if (!c->children.empty())
      collect_evictable(r, c, out);
    else if (r->pool->ref[c->block] == 1)   // a leaf only the index holds
      out.push_back(c);
  }
}

int32_t pkv_radix_evict(pkv_radix *index, int32_t n_blocks) {
  if (!index) return PKV_ERR_NULL;
  std::vector<RadixNode *> heap;
  collect_evictable(index, &index->root, heap);
  // oldest first; a parent whose last child goes joins the candidates at its own age
  const auto newer = [](const RadixNode *x, const RadixNode *y) { return x->last_used > y->last_used; };
  std::make_heap(heap.begin(), heap.end(), newer);
  int32_t freed = 0;
  while (freed < n_blocks && !heap.empty()) {
    std::pop_heap(heap.begin(), heap.end(), newer);
    RadixNode *leaf = heap.back();
    heap.pop_back();
    RadixNode *parent = leaf->parent;
    index->pool->release(leaf->block);
    ++freed;
    --index->cached;
    parent->children.erase(leaf->key);   // frees the node
    if (parent != &index->root && parent->children.empty() && index->pool->ref[parent->block] == 1) {
      heap.push_back(parent);
      std::push_heap(heap.begin(), heap.end(), newer);
    }
  }
  return freed;
}

int32_t pkv_radix_cached_blocks(const pkv_radix *index) { return index ? index->cached : PKV_ERR_NULL; }

}  // extern "C"

namespace pkv {

// One workgroup per (pair, pool): the block's pages of every kv head are one contiguous run of
// bytes in each pool, copied with 16-byte moves.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char *k_cache, char *v_cache, const int32_t *src,
                                                          const int32_t *dst, int32_t n, int64_t num_blocks,
                                                          int64_t block_bytes) {
  const int32_t pair = blockIdx.x >> 1;
  if (pair >= n) return;
  const int64_t s = src[pair];
  const int64_t d = dst[pair];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks || s == d) return;
  char *pool = (blockIdx.x & 1) ? v_cache : k_cache;
  const uint4 *from = reinterpret_cast<const uint4 *>(pool + s * block_bytes);
  uint4 *to = reinterpret_cast<uint4 *>(pool + d * block_bytes);
  for (int64_t i = threadIdx.x; i < block_bytes / 16; i += 256) to[i] = from[i];
}

}  // namespace pkv

extern "C" int pkv_copy_blocks(void *k_cache, void *v_cache, const int32_t *src, const int32_t *dst, int32_t n,
                               int64_t num_blocks, int num_kv_heads, int head_dim, int elem_bytes, void *stream) {
  if (n < 0 || num_blocks < 0 || num_kv_heads < 1 || head_dim < 1) return PKV_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return PKV_ERR_UNSUPPORTED;
  if (n == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src || !dst) return PKV_ERR_NULL;
  // 16-byte moves: pools must start on a 16-byte boundary (a block is 16 * KVH * D elements, so
  // every block then does too)
  if (reinterpret_cast<uintptr_t>(k_cache) % 16 || reinterpret_cast<uintptr_t>(v_cache) % 16)
    return PKV_ERR_UNSUPPORTED;
  const int64_t block_bytes = (int64_t)num_kv_heads * kBS * head_dim * elem_bytes;
  pkv::copy_blocks_kernel<<<2 * n, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<char *>(k_cache), static_cast<char *>(v_cache), src, dst, n, num_blocks, block_bytes);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}
