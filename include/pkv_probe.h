/*
 * pkv_probe.h — the benchmark's measurement helper, built as its own library (libpkv_probe.so, not
 * part of libpkv.so): how fast the memory system streams a given list of KV pages with the exact load
 * shapes the decode kernels use, with no arithmetic on the data.  The benchmark runs it on the decode
 * workload's own pages to report a memory ceiling for that access pattern next to the HBM datasheet
 * peak.  It computes nothing of the attention method.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Stream pages: wave w (of num_waves, 4 per 256-thread workgroup, workgroup i on XCD i % 8) reads
 * K page page_index[j] and V page page_index[j] for j in [wave_offsets[w], wave_offsets[w + 1]),
 * keeping a ring of 3 pages in flight, exactly as the matrix-core decode kernel loads a 16-token
 * page of one kv head.  Page p starts at k_pool + p * page_bytes (and v_pool + p * page_bytes);
 * page_bytes = 16 * head_dim * elem_bytes: elem_bytes 2 for bf16 pools, 1 for E4M3 pools (loaded
 * with the decode kernel's E4M3 shapes); head_dim is 64 or 128.  Each pool must hold pool_pages
 * pages.  Indexes outside [0, pool_pages) are read as page 0.  A value derived from the data goes to
 * *sink so the loads are not optimised away.  Device pointers; enqueued on `stream`; returns 0 or a
 * negative pkv_status (PKV_ERR_UNSUPPORTED for another head_dim or elem_bytes).
 */
int pkv_probe_page_stream(const void *k_pool, const void *v_pool, int64_t pool_pages, int head_dim,
                          int elem_bytes, const int32_t *page_index, const int32_t *wave_offsets,
                          int num_waves, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
