// Main kernel for units with many query rows (packed-GQA tile M = blockShapeX * G > 16).
//
// GenericBlockSparseAttention article (cf-1.com): "sparse attention mechanism" (only the
// selected KV blocks take part in QK^T, softmax and PV), "implementation architecture"
// (gemm for QK/PV, epilogue with online softmax, rescale and write-out). FlashAttention
// article (ai6s.net), "three steps": blockwise loads, online softmax with rescale, blockwise
// weighted sum, exact.
//
// One workgroup = (worker w, row subtile st). The worker's task range comes from the
// metadata; for each task (unit, slots [a, e)) the workgroup keeps R = NW * NQ * 16 query
// rows in registers and streams the selected KV pages through LDS. Each wave owns NQ
// 16-row tiles and computes S^T = K Q^T so that the 16x16 MFMA result already has the
// layout PV needs as its B operand (P^T); V^T is read from LDS with the gfx950 transpose
// read. Running max / sum live in registers, in the log2 domain.
#include "split_merge.hpp"

namespace gbsa {
namespace {

constexpr int kVPitch = 288;  // bytes per V row in LDS (256 + 32: conflict-free tr reads)

template <int DT>
struct KLds {
    static constexpr int pitch = (DT == kFP8) ? 136 : 272;  // bytes per K row in LDS
};

template <int DT, int OUT, int NW, int NQ>
__global__ __launch_bounds__(NW * 64) void fwd_prefill_kernel(FwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int R = NW * NQ * 16;
    constexpr int KP = KLds<DT>::pitch;
    __shared__ __attribute__((aligned(16))) unsigned char smem[128 * KP + 128 * kVPitch];
    __shared__ int flag[1];
    unsigned char* Ks = smem;
    unsigned char* Vs = smem + 128 * KP;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform for the compiler
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int w = lin / a.nst, st = lin - (lin / a.nst) * a.nst;

    if (!header_ok(a)) {
        if (tid == 0) atomicOr(a.ws_status, 1);
        return;
    }
    const Bound b0 = read_bound(a.meta, w), b1 = read_bound(a.meta, w + 1);
    const int U = a.meta[3];
    if (!bound_less(b0, b1) || b0.u >= U) return;

    UnitIter it = locate_unit(a, b0.u);
    if (it.b < 0) return;

    const int esz = (DT == kFP8) ? 1 : 2;
    const int64_t kv_row = (int64_t)a.N2 * 128;  // elements between tokens of a page
    const int lrow = lane & 15, lgrp = lane >> 4;

    for (int u = b0.u;; ++u) {
        const int sa = (u == b0.u) ? b0.s : 0;
        if (u >= U || u > b1.u || (u == b1.u && sa >= b1.s)) break;
        const int g = it.qbase + it.gl;
        int cnt = 0;
        if (g < a.tqb) cnt = min(max(a.cnt[(int64_t)it.n2 * a.tqb + g], 0), a.topK);
        const int se = (u == b1.u) ? b1.s : cnt;
        const bool complete = (sa == 0) && (se == cnt);

        const int t0 = it.gl * a.X;  // batch-local first row of the q-block
        const int rows_exist = min(a.X, it.storage - t0) * a.G;
        const int row_base = st * R;
        if (row_base < rows_exist) {
            const int skv = a.skv[it.b];
            const int off = skv - it.sq;
            // ---- Q tile (B operand of S^T = K Q^T) and per-column state -------------
            u32x4 qf[NQ][4];
            u32x2 q8[NQ][4];
            float colscale[NQ];
            int trow[NQ];
            bool rvalid[NQ];
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq) {
                const int r = row_base + wave * NQ * 16 + nq * 16 + lrow;
                const bool exists = r < rows_exist;
                const int t = t0 + (exists ? r / a.G : 0);
                const int h = it.n2 * a.G + (exists ? r % a.G : 0);
                trow[nq] = t;
                rvalid[nq] = exists && t < it.sq;
                float cs = a.scale_log2;
                if (DT == kFP8) cs *= a.qs[h] * a.ks[it.n2];
                colscale[nq] = cs;
                const int64_t qoff = ((it.row0 + t) * a.N1 + h) * 128;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int d = kk * 32 + lgrp * 8;
                    if (DT == kFP8) {
                        const uint8_t* qp = (const uint8_t*)a.q + qoff + d;
                        q8[nq][kk] = exists ? *(const u32x2*)qp : (u32x2){0, 0};
                    } else {
                        const uint16_t* qp = (const uint16_t*)a.q + qoff + d;
                        qf[nq][kk] = exists ? *(const u32x4*)qp : (u32x4){0, 0, 0, 0};
                    }
                }
            }
            float mrun[NQ], lrun[NQ];
            f32x4 o[8][NQ];
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq) {
                mrun[nq] = kNegInf;
                lrun[nq] = 0.f;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[dt][nq] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
            // rows of this workgroup, for block classification
            const int t_lo = t0 + row_base / a.G;
            const int t_hi = t0 + (min(row_base + R, rows_exist) - 1) / a.G;

            const int32_t* sel = a.idx + ((int64_t)it.n2 * a.tqb + g) * a.topK;
            for (int s = sa; s < se; ++s) {
                const int j = sel[s];
                if (j < 0) continue;
                const int64_t p0 = (int64_t)j * 128;
                const int cls = block_class(a, p0, skv, off, t_lo, t_hi);
                if (cls == 0) continue;
                const int page = a.table[(int64_t)it.b * a.maxb + j];
                const int64_t pbase = ((int64_t)page * a.kv_stride + (int64_t)it.n2 * 128) * esz;
                const unsigned char* kg = (const unsigned char*)a.k + pbase;
                const unsigned char* vg = (const unsigned char*)a.v + pbase;
                const int64_t rs = kv_row * esz;  // bytes between tokens

                __syncthreads();  // previous page fully consumed
                if (DT == kFP8) {
                    // K: 128 rows x 128 B; V: 128 rows x 128 B -> widened to bf16 in LDS
#pragma unroll
                    for (int i = 0; i < 1024 / NT; ++i) {
                        const int c = tid + i * NT, row = c >> 3, col = c & 7;
                        const u32x4 kx = *(const u32x4*)(kg + row * rs + col * 16);
                        u32x2* kd = (u32x2*)(Ks + row * KP + col * 16);
                        kd[0] = (u32x2){kx[0], kx[1]};
                        kd[1] = (u32x2){kx[2], kx[3]};
                        const u32x4 vx = *(const u32x4*)(vg + row * rs + col * 16);
                        const u32x2 c0 = fp8x4_to_bf16x4(vx[0]), c1 = fp8x4_to_bf16x4(vx[1]);
                        const u32x2 c2 = fp8x4_to_bf16x4(vx[2]), c3 = fp8x4_to_bf16x4(vx[3]);
                        const u32x4 lo = (u32x4){c0[0], c0[1], c1[0], c1[1]};
                        const u32x4 hi = (u32x4){c2[0], c2[1], c3[0], c3[1]};
                        u32x4* vd = (u32x4*)(Vs + row * kVPitch + col * 32);
                        vd[0] = lo;
                        vd[1] = hi;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 2048 / NT; ++i) {
                        const int c = tid + i * NT, row = c >> 4, col = c & 15;
                        const u32x4 kx = *(const u32x4*)(kg + row * rs + col * 16);
                        const u32x4 vx = *(const u32x4*)(vg + row * rs + col * 16);
                        *(u32x4*)(Ks + row * KP + col * 16) = kx;
                        *(u32x4*)(Vs + row * kVPitch + col * 16) = vx;
                    }
                }
                __syncthreads();

                // ---- S^T = K Q^T : 8 token tiles x NQ query tiles --------------------
                f32x4 sacc[8][NQ];
#pragma unroll
                for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                    for (int nq = 0; nq < NQ; ++nq) sacc[tt][nq] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                    for (int tt = 0; tt < 8; ++tt) {
                        const unsigned char* kp =
                            Ks + (tt * 16 + lrow) * KP + (kk * 32 + lgrp * 8) * esz;
                        if (DT == kFP8) {
                            const u32x2 ka = *(const u32x2*)kp;
#pragma unroll
                            for (int nq = 0; nq < NQ; ++nq)
                                sacc[tt][nq] = mfma_16x16x32_fp8(ka, q8[nq][kk], sacc[tt][nq]);
                        } else {
                            const u32x4 ka = *(const u32x4*)kp;
#pragma unroll
                            for (int nq = 0; nq < NQ; ++nq)
                                sacc[tt][nq] = mfma_16x16x32<DT == kFP8 ? kBF16 : DT>(
                                    ka, qf[nq][kk], sacc[tt][nq]);
                        }
                    }
                }
                // ---- mask ------------------------------------------------------------
                if (cls == 2) {
#pragma unroll
                    for (int nq = 0; nq < NQ; ++nq) {
                        const int64_t d = (int64_t)trow[nq] + off;
#pragma unroll
                        for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int64_t p = p0 + tt * 16 + lgrp * 4 + i;
                                if (!key_visible(a, p, skv, d)) sacc[tt][nq][i] = kNegInf;
                            }
                    }
                }
                // ---- online softmax (log2 domain) --------------------------------------
                uint32_t pk[8][NQ][2];
#pragma unroll
                for (int nq = 0; nq < NQ; ++nq) {
                    float mx = kNegInf;
#pragma unroll
                    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[tt][nq][i]);
                    mx = wave_max_cols(mx);
                    const float cs = colscale[nq];
                    const float mnew = fmaxf(mrun[nq], mx == kNegInf ? kNegInf : mx * cs);
                    const float muse = (mnew == kNegInf) ? 0.f : mnew;
                    const float alpha = fast_exp2(mrun[nq] - muse);
                    mrun[nq] = mnew;
                    float ls = 0.f;
#pragma unroll
                    for (int tt = 0; tt < 8; ++tt) {
                        float pv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            pv[i] = fast_exp2(__builtin_fmaf(sacc[tt][nq][i], cs, -muse));
                            ls += pv[i];
                        }
                        constexpr int PT = (DT == kF16) ? kF16 : kBF16;
                        pk[tt][nq][0] = pack2<PT>(pv[0], pv[1]);
                        pk[tt][nq][1] = pack2<PT>(pv[2], pv[3]);
                    }
                    lrun[nq] = lrun[nq] * alpha + ls;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) o[dt][nq] *= alpha;
                }
                // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    u32x4 pb[NQ];
#pragma unroll
                    for (int nq = 0; nq < NQ; ++nq)
                        pb[nq] = (u32x4){pk[2 * kc][nq][0], pk[2 * kc][nq][1],
                                         pk[2 * kc + 1][nq][0], pk[2 * kc + 1][nq][1]};
                    const unsigned char* vrow =
                        Vs + (kc * 32 + lgrp * 4 + (lrow >> 2)) * kVPitch + (lane & 3) * 8;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        const u32x2 v0 = lds_read_tr16(vrow + dt * 32);
                        const u32x2 v1 = lds_read_tr16(vrow + 16 * kVPitch + dt * 32);
                        const u32x4 va = (u32x4){v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
                        for (int nq = 0; nq < NQ; ++nq) {
                            constexpr int PT = (DT == kF16) ? kF16 : kBF16;
                            o[dt][nq] = mfma_16x16x32<PT>(va, pb[nq], o[dt][nq]);
                        }
                    }
                }
            }

            // ---- epilogue: normalised output + LSE, or a split-KV partial --------------
            const float vscale = (DT == kFP8) ? a.vs[it.n2] : 1.f;
            const int slot = 2 * w + (sa > 0 ? 0 : 1);
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq) {
                const float ltot = wave_sum_cols(lrun[nq]);
                const int r = row_base + wave * NQ * 16 + nq * 16 + lrow;
                if (!rvalid[nq]) continue;
                if (complete) {
                    const float inv = ltot > 0.f ? vscale / ltot : 0.f;
                    const int t = trow[nq];
                    const int h = it.n2 * a.G + r % a.G;
                    const int64_t orow = ((it.row0 + t) * a.N1 + h);
                    uint16_t* op = (uint16_t*)a.out + orow * 128;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        const int d = dt * 16 + lgrp * 4;
                        const u32x2 pr = (u32x2){pack2<OUT>(o[dt][nq][0] * inv, o[dt][nq][1] * inv),
                                                 pack2<OUT>(o[dt][nq][2] * inv, o[dt][nq][3] * inv)};
                        *(u32x2*)(op + d) = pr;
                    }
                    if (a.return_lse && lgrp == 0)
                        a.lse[orow] = ltot > 0.f ? (mrun[nq] + __log2f(ltot)) * kLn2 : kNegInf;
                } else {
                    float* po = a.ws_o + ((int64_t)slot * a.M + r) * 128;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        const int d = dt * 16 + lgrp * 4;
                        *(f32x4*)(po + d) = o[dt][nq] * vscale;
                    }
                    if (lgrp == 0) {
                        a.ws_m[(int64_t)slot * a.M + r] = mrun[nq];
                        a.ws_l[(int64_t)slot * a.M + r] = ltot;
                    }
                }
            }
            if (!complete) {
                const int w_a = unit_starter(a.meta, w, u);
                const int np = count_pieces(a.meta, w_a, u);
                if (piece_arrive(a, w_a * a.nst + st, np, flag))
                    merge_rows<OUT>(a, w_a, u, row_base, min(row_base + R, rows_exist), it.b,
                                    it.n2, t0, it.row0, it.sq);
                __syncthreads();
            }
        }
        advance_unit(a, it);
    }
}

template <int DT, int OUT>
hipError_t launch_t(const FwdArgs& a, int rows, hipStream_t s) {
    const int grid = a.P * a.nst;
    if (rows == 256) {
        hipLaunchKernelGGL((fwd_prefill_kernel<DT, OUT, 8, 2>), dim3(grid), dim3(512), 0, s, a);
    } else {
        hipLaunchKernelGGL((fwd_prefill_kernel<DT, OUT, 4, 2>), dim3(grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, int dtype, int out_dtype, int rows, hipStream_t s) {
    if (dtype == kF16) return launch_t<kF16, kF16>(a, rows, s);
    if (dtype == kBF16) return launch_t<kBF16, kBF16>(a, rows, s);
    if (out_dtype == kF16) return launch_t<kFP8, kF16>(a, rows, s);
    return launch_t<kFP8, kBF16>(a, rows, s);
}

}  // namespace gbsa
