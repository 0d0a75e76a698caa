// Main kernel for units with at most 16 query rows (packed-GQA tile M = blockShapeX * G <= 16),
// the decode shape. These units are bound by the bytes of the gathered KV pages, so the
// design goal is many page loads in flight per compute unit:
//  * one workgroup of 4 waves per worker; the task's KV slots are dealt round-robin to the
//    waves, each wave keeping its own online-softmax state for the (<= 16) query columns;
//  * K goes straight from HBM into MFMA A-operand registers (S^T = K Q^T, 16x16x32);
//  * V is loaded with full-row coalescing, staged through a wave-private LDS buffer and read
//    back with the gfx950 transpose read as the A operand of O^T = V^T P^T;
//  * at the end of a task the four wave states are merged through LDS (fixed order).
// GenericBlockSparseAttention article (cf-1.com), "sparse attention mechanism" and
// "implementation architecture"; FlashAttention article (ai6s.net), "three steps".
#include "device_common.hpp"

namespace gbsa {
namespace {

constexpr int kNW = 4;
constexpr int kVPitch = 288;            // bytes per staged V row (bf16/f16)
constexpr int kStageRows = 64;          // V rows staged per half page
constexpr int kStageBytes = kStageRows * kVPitch;
constexpr int kMergeFloats = 16 * 128 + 32;  // per wave: O^T tile + m + l

template <int DT, int OUT>
__global__ __launch_bounds__(256) void fwd_decode_kernel(FwdArgs a) {
    constexpr int kLdsBytes = (kNW * kStageBytes > kNW * kMergeFloats * 4)
                                  ? kNW * kStageBytes
                                  : kNW * kMergeFloats * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
    __shared__ int scratch[2 * 256 + 8];
    constexpr int PT = (DT == kF16) ? kF16 : kBF16;  // PV operand type
    constexpr int esz = (DT == kFP8) ? 1 : 2;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int w = xcd_remap(blockIdx.x, gridDim.x);

    if (!header_ok(a)) {
        if (tid == 0) atomicOr(a.ws_status, 1);
        return;
    }
    const Bound b0 = read_bound(a.meta, w), b1 = read_bound(a.meta, w + 1);
    const int U = a.meta[3];
    if (!bound_less(b0, b1) || b0.u >= U) return;
    UnitIter it = locate_unit(a, b0.u, scratch);
    if (it.b < 0) return;

    unsigned char* stage = smem + wave * kStageBytes;
    const int64_t rs = (int64_t)a.N2 * 128 * esz;  // bytes between tokens of a page

    for (int u = b0.u;; ++u) {
        const int sa = (u == b0.u) ? b0.s : 0;
        if (u >= U || u > b1.u || (u == b1.u && sa >= b1.s)) break;
        const int g = it.qbase + it.gl;
        int cnt = 0;
        if (g < a.tqb) cnt = min(max(a.cnt[(int64_t)it.n2 * a.tqb + g], 0), a.topK);
        const int se = (u == b1.u) ? b1.s : cnt;
        const bool complete = (sa == 0) && (se == cnt);
        const int t0 = it.gl * a.X;
        const int rows_exist = min(a.X, it.storage - t0) * a.G;
        const int skv = a.skv[it.b];
        const int off = skv - it.sq;

        // Q as the B operand: column = query row (lane & 15), k = head dim.
        const bool exists = lrow < rows_exist;
        const int t = t0 + (exists ? lrow / a.G : 0);
        const int h = it.n2 * a.G + (exists ? lrow % a.G : 0);
        const bool rvalid = exists && t < it.sq;
        float cs = a.scale_log2;
        if constexpr (DT == kFP8) cs *= a.qs[h] * a.ks[it.n2];
        const int64_t qoff = ((it.row0 + t) * a.N1 + h) * 128;
        u32x4 qf[4];
        u32x2 q8[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int d = kk * 32 + lgrp * 8;
            if constexpr (DT == kFP8) {
                q8[kk] = exists ? *(const u32x2*)((const uint8_t*)a.q + qoff + d) : (u32x2){0, 0};
            } else {
                qf[kk] = exists ? *(const u32x4*)((const uint16_t*)a.q + qoff + d)
                                : (u32x4){0, 0, 0, 0};
            }
        }
        const int t_lo = t0, t_hi = t0 + (rows_exist - 1) / a.G;

        float mrun = kNegInf, lrun = 0.f;
        f32x4 o[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};

        const int32_t* sel = a.idx + ((int64_t)it.n2 * a.tqb + g) * a.topK;
        for (int s = sa + wave; s < se; s += kNW) {
            const int j = sel[s];
            if (j < 0) continue;
            const int64_t p0 = (int64_t)j * 128;
            const int cls = block_class(a, p0, skv, off, t_lo, t_hi);
            if (cls == 0) continue;
            const int page = a.table[(int64_t)it.b * a.maxb + j];
            const int64_t pbase = ((int64_t)page * a.kv_stride + (int64_t)it.n2 * 128) * esz;
            const unsigned char* kg = (const unsigned char*)a.k + pbase;
            const unsigned char* vg = (const unsigned char*)a.v + pbase;

            // ---- issue all loads of the page ------------------------------------------
            u32x4 kf[8][4];
            u32x2 k8[8][4];
            u32x4 vr[32];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const unsigned char* kp = kg + (tt * 16 + lrow) * rs + (kk * 32 + lgrp * 8) * esz;
                    if constexpr (DT == kFP8) k8[tt][kk] = load_nt((const u32x2*)kp);
                    else kf[tt][kk] = load_nt((const u32x4*)kp);
                }
            if constexpr (DT == kFP8) {
                // 128 B rows: 8 lanes per row, 16 rows per load
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    vr[q] = load_nt((const u32x4*)(vg + (q * 8 + (lane >> 3)) * rs + (lane & 7) * 16));
            } else {
                // 256 B rows: 16 lanes per row, 4 rows per load
#pragma unroll
                for (int q = 0; q < 32; ++q)
                    vr[q] = load_nt((const u32x4*)(vg + (q * 4 + lgrp) * rs + lrow * 16));
            }

            // ---- S^T = K Q^T ---------------------------------------------------------
            f32x4 sacc[8];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    if constexpr (DT == kFP8) acc = mfma_16x16x32_fp8(k8[tt][kk], q8[kk], acc);
                    else acc = mfma_16x16x32<DT>(kf[tt][kk], qf[kk], acc);
                }
                sacc[tt] = acc;
            }
            if (cls == 2) {
                const int64_t d = (int64_t)t + off;
#pragma unroll
                for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t p = p0 + tt * 16 + lgrp * 4 + i;
                        if (!key_visible(a, p, skv, d)) sacc[tt][i] = kNegInf;
                    }
            }
            // ---- online softmax ------------------------------------------------------
            float mx = kNegInf;
#pragma unroll
            for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[tt][i]);
            mx = wave_max_cols(mx);
            const float mnew = fmaxf(mrun, mx == kNegInf ? kNegInf : mx * cs);
            const float muse = (mnew == kNegInf) ? 0.f : mnew;
            const float alpha = fast_exp2(mrun - muse);
            mrun = mnew;
            uint32_t pk[8][2];
            float ls = 0.f;
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                float pv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[i] = fast_exp2(__builtin_fmaf(sacc[tt][i], cs, -muse));
                    ls += pv[i];
                }
                pk[tt][0] = pack2<PT>(pv[0], pv[1]);
                pk[tt][1] = pack2<PT>(pv[2], pv[3]);
            }
            lrun = lrun * alpha + ls;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;

            // ---- O^T += V^T P^T, V staged 64 rows at a time --------------------------
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if constexpr (DT == kFP8) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const u32x4 vx = vr[half * 8 + q];
                        const u32x2 c0 = fp8x4_to_bf16x4(vx[0]), c1 = fp8x4_to_bf16x4(vx[1]);
                        const u32x2 c2 = fp8x4_to_bf16x4(vx[2]), c3 = fp8x4_to_bf16x4(vx[3]);
                        const u32x4 lo = (u32x4){c0[0], c0[1], c1[0], c1[1]};
                        const u32x4 hi = (u32x4){c2[0], c2[1], c3[0], c3[1]};
                        u32x4* vd = (u32x4*)(stage + (q * 8 + (lane >> 3)) * kVPitch + (lane & 7) * 32);
                        vd[0] = lo;
                        vd[1] = hi;
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        *(u32x4*)(stage + (q * 4 + lgrp) * kVPitch + lrow * 16) = vr[half * 16 + q];
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int kc2 = 0; kc2 < 2; ++kc2) {
                    const int kc = half * 2 + kc2;
                    const u32x4 pb = (u32x4){pk[2 * kc][0], pk[2 * kc][1], pk[2 * kc + 1][0],
                                             pk[2 * kc + 1][1]};
                    const unsigned char* vrow =
                        stage + (kc2 * 32 + lgrp * 4 + (lrow >> 2)) * kVPitch + (lane & 3) * 8;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        const u32x2 v0 = lds_read_tr16(vrow + dt * 32);
                        const u32x2 v1 = lds_read_tr16(vrow + 16 * kVPitch + dt * 32);
                        o[dt] = mfma_16x16x32<PT>((u32x4){v0[0], v0[1], v1[0], v1[1]}, pb, o[dt]);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }

        // ---- merge the four wave states (fixed order) ----------------------------------
        lrun = wave_sum_cols(lrun);
        __syncthreads();  // staging buffers are reused for the merge
        float* mg = (float*)smem + wave * kMergeFloats;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            *(f32x4*)(mg + lrow * 128 + dt * 16 + lgrp * 4) = o[dt];
        if (lgrp == 0) {
            mg[16 * 128 + lrow] = mrun;
            mg[16 * 128 + 16 + lrow] = lrun;
        }
        __syncthreads();
        {
            // thread -> (column c, 8 consecutive head-dim values)
            const int c = tid & 15, d0 = (tid >> 4) * 8;
            float mw[kNW], mstar = kNegInf;
#pragma unroll
            for (int v = 0; v < kNW; ++v) {
                mw[v] = ((float*)smem)[v * kMergeFloats + 16 * 128 + c];
                mstar = fmaxf(mstar, mw[v]);
            }
            const float muse = (mstar == kNegInf) ? 0.f : mstar;
            float lsum = 0.f, acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
            for (int v = 0; v < kNW; ++v) {
                const float* src = (float*)smem + v * kMergeFloats;
                const float f = fast_exp2(mw[v] - muse);
                lsum += f * src[16 * 128 + 16 + c];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += f * src[c * 128 + d0 + e];
            }
            const bool cexists = c < rows_exist;
            const int ct = t0 + (cexists ? c / a.G : 0);
            const int ch = it.n2 * a.G + (cexists ? c % a.G : 0);
            const float vscale = (DT == kFP8) ? a.vs[it.n2] : 1.f;
            if (cexists && ct < it.sq) {
                if (complete) {
                    const float inv = lsum > 0.f ? vscale / lsum : 0.f;
                    const int64_t orow = (it.row0 + ct) * a.N1 + ch;
                    uint16_t* op = (uint16_t*)a.out + orow * 128 + d0;
                    *(u32x4*)op = (u32x4){pack2<OUT>(acc[0] * inv, acc[1] * inv),
                                          pack2<OUT>(acc[2] * inv, acc[3] * inv),
                                          pack2<OUT>(acc[4] * inv, acc[5] * inv),
                                          pack2<OUT>(acc[6] * inv, acc[7] * inv)};
                    if (a.return_lse && d0 == 0)
                        a.lse[orow] = lsum > 0.f ? (mstar + __log2f(lsum)) * kLn2 : kNegInf;
                } else {
                    const int slot = 2 * w + (sa > 0 ? 0 : 1);
                    float* po = a.ws_o + ((int64_t)slot * a.M + c) * 128 + d0;
                    *(f32x4*)po = (f32x4){acc[0], acc[1], acc[2], acc[3]} * vscale;
                    *(f32x4*)(po + 4) = (f32x4){acc[4], acc[5], acc[6], acc[7]} * vscale;
                    if (d0 == 0) {
                        a.ws_m[(int64_t)slot * a.M + c] = mstar;
                        a.ws_l[(int64_t)slot * a.M + c] = lsum;
                    }
                }
            }
            if (!complete && tid == 0)
                a.ws_desc[2 * w + (sa > 0 ? 0 : 1)] = PieceDesc{it.b, it.n2, it.gl, g};
        }
        __syncthreads();
        advance_unit(a, it);
    }
}

template <int DT, int OUT>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((fwd_decode_kernel<DT, OUT>), dim3(a.P), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const FwdArgs& a, int dtype, int out_dtype, hipStream_t s) {
    if (dtype == kF16) return launch_t<kF16, kF16>(a, s);
    if (dtype == kBF16) return launch_t<kBF16, kBF16>(a, s);
    if (out_dtype == kF16) return launch_t<kFP8, kF16>(a, s);
    return launch_t<kFP8, kBF16>(a, s);
}

}  // namespace gbsa
