// Measurement probes (libgbsa_probe.so): HBM read bandwidth of the paged-KV gather pattern
// and of a contiguous read. See include/gbsa_probe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gbsa_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kNever = 0x9e3779b9u;  // the XOR of the loaded words is not expected to hit it

__device__ __forceinline__ void sink_if(u32x4 acc, u32x4* sink) {
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == kNever) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

// One workgroup per slice: 128 rows x ROW bytes from key and from value.
template <int ROW>
__global__ __launch_bounds__(256) void gather_kernel(const unsigned char* k, const unsigned char* v,
                                                     const int64_t* off, int64_t stride,
                                                     u32x4* sink) {
    constexpr int lanes_per_row = ROW / 16;
    constexpr int rows_per_pass = 256 / lanes_per_row;
    const int64_t base = off[blockIdx.x];
    const int row = threadIdx.x / lanes_per_row, col = (threadIdx.x % lanes_per_row) * 16;
    u32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 128 / rows_per_pass; ++i) {
        const int64_t o = base + (int64_t)(row + i * rows_per_pass) * stride + col;
        acc ^= __builtin_nontemporal_load((const u32x4*)(k + o));
        acc ^= __builtin_nontemporal_load((const u32x4*)(v + o));
    }
    sink_if(acc, sink);
}

__global__ __launch_bounds__(256) void stream_kernel(const u32x4* src, int64_t n, u32x4* sink) {
    u32x4 acc = {0, 0, 0, 0};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        acc ^= __builtin_nontemporal_load(src + i);
    sink_if(acc, sink);
}

}  // namespace

extern "C" {

int gbsa_probe_gather(const void* key, const void* value, const int64_t* slice_offsets,
                      int32_t num_slices, int32_t row_bytes, int64_t row_stride, void* sink,
                      hipStream_t stream) {
    if (key == nullptr || value == nullptr || slice_offsets == nullptr || sink == nullptr ||
        num_slices <= 0 || row_stride < row_bytes || (row_bytes != 256 && row_bytes != 128))
        return -1;
    const unsigned char* k = (const unsigned char*)key;
    const unsigned char* v = (const unsigned char*)value;
    if (row_bytes == 256)
        hipLaunchKernelGGL(gather_kernel<256>, dim3(num_slices), dim3(256), 0, stream, k, v,
                           slice_offsets, row_stride, (u32x4*)sink);
    else
        hipLaunchKernelGGL(gather_kernel<128>, dim3(num_slices), dim3(256), 0, stream, k, v,
                           slice_offsets, row_stride, (u32x4*)sink);
    return (int)hipGetLastError();
}

int gbsa_probe_stream(const void* src, int64_t bytes, int32_t grid, void* sink,
                      hipStream_t stream) {
    if (src == nullptr || sink == nullptr || bytes <= 0 || bytes % 16 != 0 || grid <= 0)
        return -1;
    hipLaunchKernelGGL(stream_kernel, dim3(grid), dim3(256), 0, stream, (const u32x4*)src,
                       bytes / 16, (u32x4*)sink);
    return (int)hipGetLastError();
}

}  // extern "C"
