// gbsa_validate: an opt-in check of the tensor values the forward calls take on trust
// (GenericBlockSparseAttention article, "general constraints": the host stage reads no tensor
// values, the caller guarantees them). One 1024-thread workgroup; speed is secondary.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gbsa.h"
#include "launch_lds.hpp"
#include "gbsa_internal.hpp"

namespace gbsa {
namespace {

constexpr int kThreads = 1024;

// Exclusive prefix of one value per thread over the workgroup (Hillis-Steele in LDS); also
// returns the total. Every thread of the block must call it.
__device__ int block_prefix(int v, int* buf, int* total) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {
        const int add = tid >= d ? buf[tid - d] : 0;
        __syncthreads();
        buf[tid] += add;
        __syncthreads();
    }
    const int incl = buf[tid];
    *total = buf[kThreads - 1];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(kThreads) void validate_kernel(ValArgs a) {
    extern __shared__ int qbase[];  // [B + 1]: first q-block of each sequence
    __shared__ int scan[kThreads];
    __shared__ int flags;
    const int tid = threadIdx.x;
    if (tid == 0) flags = 0;
    __syncthreads();
    int f = 0;

    // sequence lengths and the q-block prefix (in chunks of one value per thread)
    int carry = 0;
    for (int b0 = 0; b0 < a.B; b0 += kThreads) {
        const int b = b0 + tid;
        int nq = 0;
        if (b < a.B) {
            const int64_t c0 = a.cu[b], c1 = a.cu[b + 1];
            if (c0 < 0 || c1 < c0 || c1 > a.total_q) f |= GBSA_BAD_CU_SEQLENS_Q;
            const int64_t st = c1 > c0 ? c1 - c0 : 0;
            nq = (int)((st + a.X - 1) / a.X);
            int64_t sq = st;
            if (a.squ != nullptr) {
                if (a.squ[b] < 0 || a.squ[b] > st) f |= GBSA_BAD_SEQUSED_Q;
                sq = a.squ[b] < 0 ? 0 : (a.squ[b] > st ? st : a.squ[b]);
            }
            // KV side: storage and visible length
            int64_t kst;
            if (a.cu_kv != nullptr) {
                const int64_t k0 = a.cu_kv[b], k1 = a.cu_kv[b + 1];
                if (k0 < 0 || k1 < k0 || k1 > a.kv_rows) f |= GBSA_BAD_CU_SEQLENS_KV;
                kst = k1 > k0 ? k1 - k0 : 0;
            } else {
                kst = (int64_t)a.maxb * 128;
            }
            int64_t kl = kst;
            if (a.skv != nullptr) {
                if (a.skv[b] < 0 || a.skv[b] > kst) f |= GBSA_BAD_KV_LENGTH;
                kl = a.skv[b] < 0 ? 0 : (a.skv[b] > kst ? kst : a.skv[b]);
            }
            if (a.umask != nullptr && (sq > a.um_rows || kl > a.um_cols))
                f |= GBSA_BAD_MASK_EXTENT;
            if ((a.max_sq > 0 && st > a.max_sq) || (a.max_skv > 0 && kl > a.max_skv))
                f |= GBSA_BAD_MAX_SEQLEN;
        }
        int tot;
        const int ex = block_prefix(nq, scan, &tot);
        if (b < a.B) qbase[b] = carry + ex;
        carry += tot;
    }
    if (tid == 0) {
        qbase[a.B] = carry;
        if (carry != a.tqb) f |= GBSA_BAD_CU_SEQLENS_Q;  // the q-blocks the selections describe
    }
    __syncthreads();

    // visible KV length of sequence b (clamped as the kernels do)
    auto kv_len = [&](int b) -> int64_t {
        int64_t kst = (int64_t)a.maxb * 128;
        if (a.cu_kv != nullptr) {
            const int64_t k0 = a.cu_kv[b], k1 = a.cu_kv[b + 1];
            kst = k1 > k0 ? k1 - k0 : 0;
        }
        if (a.skv == nullptr) return kst;
        const int64_t s = a.skv[b];
        return s < 0 ? 0 : (a.cu_kv != nullptr && s > kst ? kst : s);
    };

    // page table entries of every visible block (paged key/value)
    if (a.table != nullptr) {
        const int64_t n = (int64_t)a.B * a.maxb;
        for (int64_t i = tid; i < n; i += kThreads) {
            const int b = (int)(i / a.maxb), j = (int)(i % a.maxb);
            if ((int64_t)j * 128 < kv_len(b)) {
                const int page = a.table[i];
                if (page < 0 || page >= a.num_pages) f |= GBSA_BAD_BLOCK_TABLE;
            }
        }
    }

    // counts and selected indices of every (KV head, q-block)
    const int64_t nu = (int64_t)a.N2 * a.tqb;
    for (int64_t i = tid; i < nu; i += kThreads) {
        const int g = (int)(i % a.tqb);
        const int c = a.cnt[i];
        if (c < 0 || c > a.topK) f |= GBSA_BAD_COUNT;
        // sequence of q-block g: the last b with qbase[b] <= g
        int lo = 0, hi = a.B;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (qbase[mid] <= g) lo = mid;
            else hi = mid;
        }
        if (g >= qbase[a.B]) continue;  // past the last sequence's q-blocks
        const int64_t nblk = (kv_len(lo) + 127) / 128;
        const int cc = c < 0 ? 0 : (c > a.topK ? a.topK : c);
        const int32_t* sel = a.idx + i * a.topK;
        for (int s = 0; s < cc; ++s) {
            const int j = sel[s];
            if (j >= 0 && j >= nblk) f |= GBSA_BAD_SELECTION;
        }
    }
    if (f) atomicOr(&flags, f);
    __syncthreads();
    if (tid == 0 && flags) atomicOr(a.out, flags);
}

}  // namespace

hipError_t launch_validate(const ValArgs& a, hipStream_t s) {
    const size_t lds = sizeof(int) * ((size_t)a.B + 1);
    static std::atomic<int> granted[kMaxDevices];
    const hipError_t e = ensure_dynamic_lds((const void*)validate_kernel, granted, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace gbsa
