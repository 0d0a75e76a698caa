/*
 * gbsa_probe.h -- measurement probes beside libgbsa (libgbsa_probe.so): the achievable HBM
 * bandwidth of the KV gather pattern of block-sparse paged attention on this GPU, and of a
 * plain contiguous read, so that a kernel's roofline fraction can be read against what the
 * memory system delivers for the same access pattern, not only against the datasheet.
 *
 * The gather pattern is the one the GenericBlockSparseAttention article's paged KV cache
 * imposes ("parameters" section: PA_BBND key/value, one KV head's slice of a 128-token page
 * being 128 rows strided by N2 * D elements): every selected block is read once from key and
 * once from value. Nothing is computed; the loaded words only feed a never-taken store.
 *
 * All pointers are device pointers owned by the caller; work is enqueued on `stream`. The
 * probes never allocate or synchronise. Return value: 0, or a hipError_t code (launch
 * failure), or -1 for an invalid argument (checked before any launch).
 */
#ifndef GBSA_PROBE_H_
#define GBSA_PROBE_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `num_slices` block slices from key and from value: slice s is 128 rows of `row_bytes`
 * bytes (256: one 16-bit head row of D = 128; 128: fp8) starting `slice_offsets[s]` bytes
 * into key (and into value), rows `row_stride` bytes apart. One 256-thread workgroup per
 * slice, 16-byte non-temporal loads. The caller guarantees every slice lies inside both
 * tensors. sink: device buffer of at least num_slices * 4096 bytes (written only if the XOR
 * of all words equals a fixed improbable value).
 */
int gbsa_probe_gather(const void* key, const void* value, const int64_t* slice_offsets,
                      int32_t num_slices, int32_t row_bytes, int64_t row_stride, void* sink,
                      hipStream_t stream);

/*
 * Read `bytes` (a multiple of 16) contiguous bytes of `src` with 16-byte non-temporal loads
 * over `grid` 256-thread workgroups. sink: at least grid * 4096 bytes.
 */
int gbsa_probe_stream(const void* src, int64_t bytes, int32_t grid, void* sink,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GBSA_PROBE_H_ */
