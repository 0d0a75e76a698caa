// Split-KV merge, fused into the main kernels.
//
// When the task split cuts a unit's KV slots across workers, every worker holding a piece
// stores its unnormalised partial result (O, running max m, running sum l) in the workspace
// and then arrives on the unit's counter; the last workgroup to arrive merges all pieces in
// worker order and writes the output. FlashAttention article (ai6s.net), "three steps":
// partial softmax results over disjoint key sets merge exactly after rescaling by the running
// maxima: m* = max m_i, l* = sum l_i 2^(m_i - m*), O = sum O_i 2^(m_i - m*) / l*,
// LSE = (m* + log2 l*) ln 2 (m in the log2 domain). The order is fixed, so the result does not
// depend on which workgroup merges (GBSA article, "general constraints": deterministic).
//
// Piece slots: a worker that starts a unit without finishing it stores the piece in slot
// 2w+1; a worker that continues a unit started by an earlier worker stores it in slot 2w.
#pragma once

#include "device_common.hpp"

namespace gbsa {

// The worker whose range contains the start (u, 0) of unit u, searching back from w.
__device__ __forceinline__ int unit_starter(const int32_t* meta, int w, int u) {
    int ww = w;
    while (true) {
        const Bound b = read_bound(meta, ww);
        if (b.u < u || (b.u == u && b.s == 0)) return ww;
        --ww;
    }
}

// Advance from worker *ww to the next worker that holds a piece of unit u (its range starts
// strictly inside u and is not empty). Returns false when u ends within *ww.
__device__ __forceinline__ bool next_piece(const int32_t* meta, int u, int* ww, int* slot) {
    while (true) {
        const Bound nb = read_bound(meta, *ww + 1);  // end of *ww = start of *ww + 1
        if (!(nb.u == u && nb.s > 0)) return false;
        ++*ww;
        const Bound ne = read_bound(meta, *ww + 1);
        if (bound_less(nb, ne)) {
            *slot = 2 * *ww;
            return true;
        }
    }
}

__device__ __forceinline__ int count_pieces(const int32_t* meta, int w_a, int u) {
    int n = 1, ww = w_a, slot = 0;
    while (next_piece(meta, u, &ww, &slot)) ++n;
    return n;
}

// Arrive on counter `idx` after this workgroup's piece is stored; true for the last arrival.
// Called by every thread of the workgroup. The last arrival resets the counter to zero.
__device__ __forceinline__ bool piece_arrive(const FwdArgs& a, int idx, int npieces, int* flag) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = atomicAdd(&a.ws_arrive[idx], 1);
        const int last = (old == npieces - 1) ? 1 : 0;
        if (last) a.ws_arrive[idx] = 0;
        *flag = last;
    }
    __syncthreads();
    const bool last = *flag != 0;
    if (last) __threadfence();
    return last;
}

__device__ __forceinline__ float ld_cg(const float* p) {
    return __builtin_nontemporal_load(p);
}

// Merge rows [r0, r1) of split unit u (pieces starting at worker w_a) and write the output.
// Workgroup-wide; each thread takes (row, 32 head-dim values) items.
template <int OUT>
__device__ void merge_rows(const FwdArgs& a, int w_a, int u, int r0, int r1, int b, int n2,
                           int t0, int64_t row0, int sq) {
    const int items = (r1 - r0) * 4;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int r = r0 + (it >> 2);
        const int dq = (it & 3) * 32;
        const int t = t0 + r / a.G;
        if (t >= sq) continue;
        const int h = n2 * a.G + r % a.G;
        float mstar = kNegInf;
        {
            int ww = w_a, slot = 2 * w_a + 1;
            do {
                mstar = fmaxf(mstar, ld_cg(a.ws_m + (int64_t)slot * a.M + r));
            } while (next_piece(a.meta, u, &ww, &slot));
        }
        const float muse = (mstar == kNegInf) ? 0.f : mstar;
        float acc[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] = 0.f;
        float lsum = 0.f;
        {
            int ww = w_a, slot = 2 * w_a + 1;
            do {
                const float f = fast_exp2(ld_cg(a.ws_m + (int64_t)slot * a.M + r) - muse);
                lsum += f * ld_cg(a.ws_l + (int64_t)slot * a.M + r);
                const f32x4* po = (const f32x4*)(a.ws_o + ((int64_t)slot * a.M + r) * 128 + dq);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const f32x4 x = __builtin_nontemporal_load(po + e);
                    acc[4 * e] += f * x[0];
                    acc[4 * e + 1] += f * x[1];
                    acc[4 * e + 2] += f * x[2];
                    acc[4 * e + 3] += f * x[3];
                }
            } while (next_piece(a.meta, u, &ww, &slot));
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const int64_t orow = (row0 + t) * a.N1 + h;
        uint16_t* op = (uint16_t*)a.out + orow * 128 + dq;
#pragma unroll
        for (int e = 0; e < 32; e += 8) {
            *(u32x4*)(op + e) = (u32x4){pack2<OUT>(acc[e] * inv, acc[e + 1] * inv),
                                        pack2<OUT>(acc[e + 2] * inv, acc[e + 3] * inv),
                                        pack2<OUT>(acc[e + 4] * inv, acc[e + 5] * inv),
                                        pack2<OUT>(acc[e + 6] * inv, acc[e + 7] * inv)};
        }
        if (a.return_lse && dq == 0)
            a.lse[orow] = lsum > 0.f ? (mstar + __log2f(lsum)) * kLn2 : kNegInf;
    }
}

}  // namespace gbsa
