// Page-stream probe (include/pkv_probe.h): the matrix-core decode kernel's K/V page loads with the
// attention arithmetic taken out, to measure what the memory system delivers for a page pattern.
#include "pkv.h"
#include "pkv_probe.h"

#include <type_traits>

#include "device_common.h"

namespace pkv {

typedef const __attribute__((address_space(4))) int32_t const_i32_probe;

// F8: 1-byte E4M3 pools, loaded with the decode kernel's E4M3 shapes (half the bytes per lane).
template <int D, int NBUF, bool F8>
__global__ __launch_bounds__(256) void page_stream_kernel(const char *__restrict__ K, const char *__restrict__ V,
                                                          int64_t pool_pages, const int32_t *__restrict__ list,
                                                          const int32_t *__restrict__ offs, int num_waves,
                                                          uint32_t *sink) {
  constexpr int EB = F8 ? 1 : 2;             // bytes per cache element
  constexpr int ROWB = D * EB;
  constexpr int NK = D / 32;
  constexpr int ND = D / 16;
  typedef typename std::conditional<F8, uint2, uint4>::type KR;      // 8 elements of a K row
  typedef typename std::conditional<F8, uint4, uint2>::type VR;      // 4 tokens of a V dim (E4M3: a dim row)
  constexpr int NV = F8 ? ND / 4 : ND;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= num_waves) return;
  const int b0 = offs[w];
  const int n = offs[w + 1] - b0;
  if (n <= 0) return;
  const const_i32_probe *ids = (const const_i32_probe *)(list + b0);   // read through the scalar cache
  const int last = n - 1;
  const int64_t page_bytes = (int64_t)kBlock * ROWB;
  auto id_of = [&](int j) -> int64_t {
    const int64_t id = ids[__builtin_amdgcn_readfirstlane(min(j, last))];
    return id >= 0 && id < pool_pages ? id : 0;
  };
  uint32_t acc = 0;
  KR kb[NBUF][NK];
  VR vb[NBUF][NV];
  auto issue = [&](int64_t id, KR *kr, VR *vr) {
    const char *kp = K + id * page_bytes + col * ROWB + grp * 8 * EB;
    #pragma unroll
    for (int c = 0; c < NK; ++c) kr[c] = *reinterpret_cast<const KR *>(kp + c * 32 * EB);
    if constexpr (F8) {
      // E4M3 pages: whole 16-token dim rows, lane (col, grp) reading row 64 h + 16 grp + col
      const char *vp = V + id * page_bytes + (16 * grp + col) * kBlock * EB;
      #pragma unroll
      for (int h = 0; h < NV; ++h) vr[h] = *reinterpret_cast<const VR *>(vp + h * 64 * kBlock * EB);
    } else {
      const char *vp = V + id * page_bytes + (col * kBlock + 4 * grp) * EB;
      #pragma unroll
      for (int t = 0; t < ND; ++t) vr[t] = *reinterpret_cast<const VR *>(vp + t * 16 * kBlock * EB);
    }
  };
  auto use = [&](const KR *kr, const VR *vr) {
    #pragma unroll
    for (int c = 0; c < NK; ++c) acc += kr[c].x ^ kr[c].y;
    #pragma unroll
    for (int t = 0; t < NV; ++t) acc += reinterpret_cast<const uint32_t *>(&vr[t])[0];
  };
  int64_t sid[NBUF];
  #pragma unroll
  for (int j = 0; j < NBUF - 1; ++j) issue(id_of(j), kb[j], vb[j]);
  #pragma unroll
  for (int b = 0; b < NBUF; ++b) sid[b] = id_of(NBUF - 1 + b);
  int j0 = 0;
  for (; j0 + NBUF <= n; j0 += NBUF) {
    #pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int bn = (b + NBUF - 1) % NBUF;
      issue(sid[b], kb[bn], vb[bn]);
      sid[b] = id_of(j0 + b + 2 * NBUF - 1);
      use(kb[b], vb[b]);
    }
  }
  #pragma unroll
  for (int b = 0; b < NBUF - 1; ++b)
    if (j0 + b < n) use(kb[b], vb[b]);
  if (acc == 0x5a5a5a5au) sink[0] = acc;   // practically never true; keeps the loads
}

}  // namespace pkv

extern "C" int pkv_probe_page_stream(const void *k_pool, const void *v_pool, int64_t pool_pages, int head_dim,
                                     int elem_bytes, const int32_t *page_index, const int32_t *wave_offsets,
                                     int num_waves, uint32_t *sink, void *stream) {
  if (!k_pool || !v_pool || !page_index || !wave_offsets || !sink) return PKV_ERR_NULL;
  if ((head_dim != 64 && head_dim != 128) || (elem_bytes != 1 && elem_bytes != 2)) return PKV_ERR_UNSUPPORTED;
  if (num_waves < 0 || pool_pages < 1) return PKV_ERR_SHAPE;
  if (num_waves == 0) return PKV_OK;
  const int grid = (num_waves + 3) / 4;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char *K = static_cast<const char *>(k_pool);
  const char *V = static_cast<const char *>(v_pool);
  if (head_dim == 64 && elem_bytes == 2)
    pkv::page_stream_kernel<64, 3, false><<<grid, 256, 0, st>>>(K, V, pool_pages, page_index, wave_offsets, num_waves, sink);
  else if (head_dim == 64)
    pkv::page_stream_kernel<64, 3, true><<<grid, 256, 0, st>>>(K, V, pool_pages, page_index, wave_offsets, num_waves, sink);
  else if (elem_bytes == 2)
    pkv::page_stream_kernel<128, 3, false><<<grid, 256, 0, st>>>(K, V, pool_pages, page_index, wave_offsets, num_waves, sink);
  else
    pkv::page_stream_kernel<128, 3, true><<<grid, 256, 0, st>>>(K, V, pool_pages, page_index, wave_offsets, num_waves, sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}
