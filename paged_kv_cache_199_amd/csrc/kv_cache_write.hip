// Slot-mapped KV append: new K/V rows go to the page slots the engine assigned to them.
// (lfm25-inference, "Runtime Design": KV pages belong to the engine; inferd follow-up plan: the
// block allocator feeding live decode.)  Bits are moved unchanged, so the write is exact.
//
// One 64-thread workgroup per (new token, kv head).  K pages are token-major: the row is one
// contiguous run, copied with 16-byte moves.  V pages are dim-major: element d of the row lands at
// stride block_size, one element per lane.  The source rows are read together with the slot (they
// do not depend on it), so the kernel waits for memory once before it stores.
#include "decode_args.h"
#include "device_common.h"
#include "e4m3.h"

namespace pkv {

template <int E, int D>
__global__ __launch_bounds__(64) void kv_write_kernel(const void *__restrict__ k, const void *__restrict__ v,
                                                      const int64_t *__restrict__ slots,
                                                      void *__restrict__ kc, void *__restrict__ vc,
                                                      int64_t num_slots, int kvh_n) {
  using elem_t = typename std::conditional<E == 2, uint16_t, uint32_t>::type;
  constexpr int ROWB = D * E;
  const int64_t row = blockIdx.x;            // token * kvh_n + head
  const int64_t t = row / kvh_n;
  const int h = (int)(row - t * kvh_n);
  static_assert(ROWB / 16 <= 64 && D % 64 == 0, "one 16-byte K chunk per lane, D / 64 V elements per lane");
  constexpr int VPL = D / 64;
  const int lane = threadIdx.x;
  const int64_t slot = slots[t];
  const char *ks = static_cast<const char *>(k) + row * ROWB;
  const bool kl = lane < ROWB / 16;
  const uint4 kchunk = kl ? *reinterpret_cast<const uint4 *>(ks + lane * 16) : make_uint4(0, 0, 0, 0);
  const elem_t *vs = static_cast<const elem_t *>(v) + row * D;
  elem_t vv[VPL];
  #pragma unroll
  for (int e = 0; e < VPL; ++e) vv[e] = vs[lane + 64 * e];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / kBlock;
  const int off = (int)(slot - blk * kBlock);
  const int64_t page = blk * kvh_n + h;
  char *kd = static_cast<char *>(kc) + (page * kBlock + off) * ROWB;
  if (kl) *reinterpret_cast<uint4 *>(kd + lane * 16) = kchunk;
  elem_t *vd = static_cast<elem_t *>(vc) + page * D * kBlock + off;
  #pragma unroll
  for (int e = 0; e < VPL; ++e) vd[(lane + 64 * e) * kBlock] = vv[e];
}

// Append for the decode paths that do not fold it into the attention pass: new token i of sequence s
// (row qbase + i of k / v, packed like q) goes to position ctx - q_s + i, the page found through the
// block table.  One 64-thread workgroup per (sequence, new token, kv head).
template <int E, int D>
__global__ __launch_bounds__(64) void kv_append_kernel(DecodeArgs a) {
  using elem_t = typename std::conditional<E == 2, uint16_t, uint32_t>::type;
  constexpr int ROWB = D * E;
  constexpr int VPL = D / 64;
  const int KVH = a.num_kv_heads;
  const int64_t u = blockIdx.x;
  const int h = (int)(u % KVH);
  const int64_t t = u / KVH;
  const int i = (int)(t % a.max_q_len);
  const int s = (int)(t / a.max_q_len);
  const SeqInfo si = load_seq(a, s);
  if (i >= si.qs || si.ctx <= 0) return;
  const int row_q = si.qbase + i;
  if (row_q >= a.total_q) return;
  const int pos = si.ctx - si.qs + i;
  const int64_t bid = a.block_tables[(int64_t)s * a.max_blocks_per_seq + pos / kBlock];
  if (bid < 0 || bid >= a.num_blocks) return;
  const int lane = threadIdx.x;
  const int64_t row = (int64_t)row_q * KVH + h;
  const int64_t page = bid * KVH + h;
  const int off = pos % kBlock;
  const char *ks = static_cast<const char *>(a.new_k) + row * ROWB;
  if (lane < ROWB / 16)
    *reinterpret_cast<uint4 *>(static_cast<char *>(const_cast<void *>(a.k_cache)) + (page * kBlock + off) * ROWB +
                               lane * 16) = *reinterpret_cast<const uint4 *>(ks + lane * 16);
  const elem_t *vs = static_cast<const elem_t *>(a.new_v) + row * D;
  elem_t *vd = static_cast<elem_t *>(const_cast<void *>(a.v_cache)) + page * D * kBlock + off;
  #pragma unroll
  for (int e = 0; e < VPL; ++e) vd[(lane + 64 * e) * kBlock] = vs[lane + 64 * e];
}

hipError_t launch_kv_append(const DecodeArgs &a, bool bf16, int head_dim, hipStream_t st) {
  const int64_t grid = (int64_t)a.num_seqs * a.max_q_len * a.num_kv_heads;
  if (bf16) {
    if (head_dim == 64) kv_append_kernel<2, 64><<<grid, 64, 0, st>>>(a);
    else kv_append_kernel<2, 128><<<grid, 64, 0, st>>>(a);
  } else {
    if (head_dim == 64) kv_append_kernel<4, 64><<<grid, 64, 0, st>>>(a);
    else kv_append_kernel<4, 128><<<grid, 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

// Slot-mapped append into E4M3 pools: bf16 rows in, one code per element out (x / scale in fp32).
template <int D>
__global__ __launch_bounds__(64) void kv_write_fp8_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                                          const int64_t *__restrict__ slots, uint8_t *__restrict__ kc,
                                                          uint8_t *__restrict__ vc, int64_t num_slots, int kvh_n,
                                                          float k_scale, float v_scale) {
  constexpr int PER = D / 64;
  const int64_t row = blockIdx.x;            // token * kvh_n + head
  const int64_t t = row / kvh_n;
  const int h = (int)(row - t * kvh_n);
  const int lane = threadIdx.x;
  const int64_t slot = slots[t];
  uint32_t kq[PER], vq[PER];
  #pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = lane + 64 * e;
    kq[e] = e4m3_code(__uint_as_float((uint32_t)k[row * D + d] << 16) / k_scale);
    vq[e] = e4m3_code(__uint_as_float((uint32_t)v[row * D + d] << 16) / v_scale);
  }
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / kBlock;
  const int off = (int)(slot - blk * kBlock);
  const int64_t page = blk * kvh_n + h;
  #pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = lane + 64 * e;
    kc[(page * kBlock + off) * D + d] = (uint8_t)kq[e];
    vc[(page * D + d) * kBlock + off] = (uint8_t)vq[e];
  }
}

hipError_t launch_kv_write_fp8(const void *k, const void *v, const int64_t *slots, void *kc, void *vc,
                               int64_t num_tokens, int64_t num_blocks, int kvh_n, int head_dim, float k_scale,
                               float v_scale, hipStream_t st) {
  const int64_t grid = num_tokens * kvh_n;
  const int64_t nslots = num_blocks * kBlock;
  const uint16_t *ks = static_cast<const uint16_t *>(k);
  const uint16_t *vs = static_cast<const uint16_t *>(v);
  uint8_t *kd = static_cast<uint8_t *>(kc);
  uint8_t *vd = static_cast<uint8_t *>(vc);
  if (head_dim == 64) kv_write_fp8_kernel<64><<<grid, 64, 0, st>>>(ks, vs, slots, kd, vd, nslots, kvh_n, k_scale, v_scale);
  else kv_write_fp8_kernel<128><<<grid, 64, 0, st>>>(ks, vs, slots, kd, vd, nslots, kvh_n, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_write(const void *k, const void *v, const int64_t *slots, void *kc, void *vc,
                           int64_t num_tokens, int64_t num_blocks, int kvh_n, int head_dim, bool bf16,
                           hipStream_t st) {
  const int64_t grid = num_tokens * kvh_n;
  const int64_t nslots = num_blocks * kBlock;
  if (bf16) {
    if (head_dim == 64) kv_write_kernel<2, 64><<<grid, 64, 0, st>>>(k, v, slots, kc, vc, nslots, kvh_n);
    else kv_write_kernel<2, 128><<<grid, 64, 0, st>>>(k, v, slots, kc, vc, nslots, kvh_n);
  } else {
    if (head_dim == 64) kv_write_kernel<4, 64><<<grid, 64, 0, st>>>(k, v, slots, kc, vc, nslots, kvh_n);
    else kv_write_kernel<4, 128><<<grid, 64, 0, st>>>(k, v, slots, kc, vc, nslots, kvh_n);
  }
  return hipGetLastError();
}

}  // namespace pkv
