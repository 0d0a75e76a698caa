// Split-KV combine: merges the partial results of units whose KV slots were cut across
// workers by the task split, then writes the normalised output and LSE.
//
// FlashAttention article (ai6s.net), "three steps": partial softmax results over disjoint
// key sets merge exactly by rescaling with the running maxima: with pieces (O_i, m_i, l_i)
// in the log2 domain, m* = max m_i, l* = sum l_i 2^(m_i - m*), O = sum O_i 2^(m_i - m*) / l*,
// LSE = (m* + log2 l*) ln 2. Pieces are merged in worker order, so the result is
// deterministic (GBSA article, "general constraints": deterministic by default).
//
// Piece slots: a worker that starts a unit but does not finish it stores that piece in slot
// 2w+1; a worker that continues a unit started earlier stores it in slot 2w.
#include "device_common.hpp"

namespace gbsa {
namespace {

constexpr int kRowsPerBlock = 64;  // 4 threads per row, 32 head-dim values each

// Advance from worker *ww to the next worker that holds a piece of unit u (its range starts
// strictly inside u and is not empty). Returns false when the unit ends within *ww.
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

template <int OUT>
__global__ __launch_bounds__(256) void combine_kernel(FwdArgs a) {
    const int w = blockIdx.x;
    if (!header_ok(a)) return;
    const Bound b0 = read_bound(a.meta, w), b1 = read_bound(a.meta, w + 1);
    // Worker w starts a split unit iff its range ends strictly inside unit b1.u and that
    // unit begins inside the range.
    if (b1.s == 0) return;
    if (!(b0.u < b1.u || (b0.u == b1.u && b0.s == 0))) return;
    const int u = b1.u;
    const PieceDesc desc = a.ws_desc[2 * w + 1];

    int64_t row0;
    int storage, sq;
    batch_lengths(a, desc.b, &row0, &storage, &sq);
    const int t0 = desc.gl * a.X;
    const int rows_exist = min(a.X, storage - t0) * a.G;

    const int r = blockIdx.y * kRowsPerBlock + (threadIdx.x >> 2);
    const int dq = (threadIdx.x & 3) * 32;
    if (r >= rows_exist) return;
    const int t = t0 + r / a.G;
    if (t >= sq) return;
    const int h = desc.n2 * a.G + r % a.G;

    // pass 1: global max over the pieces
    float mstar = kNegInf;
    {
        int ww = w, slot = 2 * w + 1;
        do {
            mstar = fmaxf(mstar, a.ws_m[(int64_t)slot * a.M + r]);
        } while (next_piece(a.meta, u, &ww, &slot));
    }
    const float muse = (mstar == kNegInf) ? 0.f : mstar;
    float acc[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] = 0.f;
    float lsum = 0.f;
    {
        int ww = w, slot = 2 * w + 1;
        do {
            const float f = fast_exp2(a.ws_m[(int64_t)slot * a.M + r] - muse);
            lsum += f * a.ws_l[(int64_t)slot * a.M + r];
            const float* po = a.ws_o + ((int64_t)slot * a.M + r) * 128 + dq;
#pragma unroll
            for (int e = 0; e < 32; e += 4) {
                const f32x4 x = *(const f32x4*)(po + e);
                acc[e] += f * x[0];
                acc[e + 1] += f * x[1];
                acc[e + 2] += f * x[2];
                acc[e + 3] += f * x[3];
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

}  // namespace

hipError_t launch_combine(const FwdArgs& a, int out_dtype, hipStream_t s) {
    const dim3 grid(a.P, (a.M + kRowsPerBlock - 1) / kRowsPerBlock);
    if (out_dtype == kF16)
        hipLaunchKernelGGL((combine_kernel<kF16>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((combine_kernel<kBF16>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace gbsa
