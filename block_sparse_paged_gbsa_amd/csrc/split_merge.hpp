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
// The pieces of a unit are held by consecutive workers: its starter, then every later worker
// whose (non-empty) range begins inside the unit.
//
// Visibility without cache maintenance: the L2 is per XCD and the pieces of a unit may run on
// different XCDs. The partial results are stored and loaded with agent-scope coherent accesses
// (cache policy sc1: the store is written through to the memory side, the load does not return
// a line another XCD may have changed), each wave waits for its stores to complete before the
// workgroup barrier that precedes the arrival atomic, and the merging workgroup reads the
// pieces only after its atomic has returned. A device-scope fence instead would write back and
// invalidate the whole L2 of the XCD in every arriving workgroup (measured: it made a decode
// whose 512 units were all split four times slower).
#pragma once

#include "device_common.hpp"

namespace gbsa {

constexpr int kAgentScope = 16;  // buffer cache policy bits: sc1
// LDS ints a kernel lends to the merge once its stages are free: the slot list and two words.
constexpr int kPieceListInts = kMaxWorkers + 3;
constexpr int kPieceListBytes = kPieceListInts * 4;

// Partial O of slot `slot`: M rows of 128 floats; byte offset (row * 128 + d) * 4.
__device__ __forceinline__ rsrc_t ws_o_rsrc(const FwdArgs& a, int slot) {
    return make_rsrc(a.ws_o + (int64_t)slot * a.M * 128, a.M * 128 * 4);
}
__device__ __forceinline__ void ws_put4(rsrc_t r, int byte_off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0,
                                           kAgentScope);
}
__device__ __forceinline__ f32x4 ws_get4(rsrc_t r, int byte_off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0,
                                                                           kAgentScope));
}
__device__ __forceinline__ void ws_put1(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ws_get1(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wave-wide: the worker whose range contains the start (u, 0) of unit u, at or before w
// (64 candidates per step).
__device__ __forceinline__ int unit_starter(const int32_t* meta, int w, int u) {
    // boundaries are ordered: the last worker at or before w whose start is <= (u, 0)
    int lo = 0, hi = w;  // invariant: start(lo) <= (u, 0); answer in [lo, hi]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const Bound b = read_bound(meta, mid);
        if (b.u < u || (b.u == u && b.s == 0)) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Wave-wide: writes the slots of unit u's pieces (starter w_a first, then worker order) to
// list and returns their number.
__device__ __forceinline__ int list_pieces(const FwdArgs& a, int w_a, int u, int* list) {
    const int lane = threadIdx.x & 63;
    if (lane == 0) list[0] = 2 * w_a + 1;
    int n = 1;
    for (int base = w_a + 1; base < a.P; base += 64) {
        const int ww = base + lane;
        bool inside = false, held = false;
        if (ww < a.P) {
            const Bound nb = read_bound(a.meta, ww);  // start of worker ww
            inside = nb.u == u && nb.s > 0;
            held = inside && bound_less(nb, read_bound(a.meta, ww + 1));
        }
        const uint64_t in = __ballot(inside);
        const int run = (~in == 0) ? 64 : __builtin_ctzll(~in);  // workers inside u, from base
        const uint64_t pm = __ballot(held) & (run == 64 ? ~0ull : ((1ull << run) - 1));
        if ((pm >> lane) & 1) {
            const int below = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(pm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)pm, 0));
            list[n + below] = 2 * ww;
        }
        n += __builtin_popcountll(pm);
        if (run < 64) break;
    }
    return n;
}

// Whole workgroup, after it stored its piece of unit u (row subtile st of nst) with ws_put*.
// Lists the unit's pieces in `list` (kPieceListInts LDS ints, free for the merge) and arrives
// on the subtile's counter. Returns the number of pieces in the last-arriving workgroup (which
// then merges), 0 in the others. The last arrival resets the counter to zero.
__device__ __forceinline__ int piece_arrive(const FwdArgs& a, int w, int u, int st, int nst,
                                            int* list) {
    wait_stores();
    __syncthreads();
    if (threadIdx.x < 64) {
        const int w_a = unit_starter(a.meta, w, u);
        const int np = list_pieces(a, w_a, u, list);
        if (threadIdx.x == 0) {
            int32_t* ctr = a.ws_arrive + (int64_t)w_a * nst + st;
            const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            const bool last = old == np - 1;
            if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            list[kMaxWorkers + 1] = last ? np : 0;
        }
    }
    __syncthreads();
    return list[kMaxWorkers + 1];
}

// Merge rows [r0, r1) of a split unit from its np pieces (slots in list) and write the output.
// Workgroup-wide; each thread takes (row, 4 head-dim values) items. Pieces are read four at a
// time and combined in list order.
template <int OUT>
__device__ void merge_rows(const FwdArgs& a, const int* list, int np, int r0, int r1, int n2,
                           int t0, int64_t row0, int sq) {
    const int items = (r1 - r0) * 32;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int r = r0 + (it >> 5);
        const int d = (it & 31) * 4;
        const int t = t0 + r / a.G;
        if (t >= sq) continue;
        const int h = n2 * a.G + r % a.G;
        float mstar = kNegInf;
        for (int i = 0; i < np; i += 4) {
            float mi[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                mi[k] = (i + k < np) ? ws_get1(a.ws_m + (int64_t)list[i + k] * a.M + r) : kNegInf;
#pragma unroll
            for (int k = 0; k < 4; ++k) mstar = fmaxf(mstar, mi[k]);
        }
        const float muse = (mstar == kNegInf) ? 0.f : mstar;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
        for (int i = 0; i < np; i += 4) {
            const int nk = min(4, np - i);
            float mi[4], li[4];
            f32x4 x[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (k < nk) {
                    const int slot = list[i + k];
                    mi[k] = ws_get1(a.ws_m + (int64_t)slot * a.M + r);
                    li[k] = ws_get1(a.ws_l + (int64_t)slot * a.M + r);
                    x[k] = ws_get4(ws_o_rsrc(a, slot), (r * 128 + d) * 4);
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (k < nk) {
                    const float f = fast_exp2(mi[k] - muse);
                    lsum += f * li[k];
                    acc[0] += f * x[k][0];
                    acc[1] += f * x[k][1];
                    acc[2] += f * x[k][2];
                    acc[3] += f * x[k][3];
                }
            }
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const int64_t orow = (row0 + t) * a.N1 + h;
        uint16_t* op = (uint16_t*)a.out + orow * 128 + d;
        *(u32x2*)op = (u32x2){pack2<OUT>(acc[0] * inv, acc[1] * inv),
                              pack2<OUT>(acc[2] * inv, acc[3] * inv)};
        if (a.return_lse && d == 0)
            a.lse[orow] = lsum > 0.f ? (mstar + __log2f(lsum)) * kLn2 : kNegInf;
    }
}

}  // namespace gbsa
