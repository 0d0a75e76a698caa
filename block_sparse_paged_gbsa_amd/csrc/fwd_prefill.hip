// Main kernels for units with many query rows (packed-GQA tile M = blockShapeX * G > 16).
//
// GenericBlockSparseAttention article (cf-1.com): "sparse attention mechanism" (only the
// selected KV blocks take part in QK^T, softmax and PV), "implementation architecture"
// (gemm for QK/PV, epilogue with online softmax, rescale and write-out). FlashAttention
// article (ai6s.net), "three steps": blockwise loads, online softmax with rescale, blockwise
// weighted sum, exact.
//
// One workgroup = (worker w, row subtile st) of 8 waves. Throughout, S^T = K Q^T is computed so
// that the MFMA result is already P^T in the B-operand layout of O^T = V^T P^T, and V^T is read
// with the gfx950 transpose read. Split units are merged in kernel by the last arriving
// workgroup (split_merge.hpp). Three kernels by unit size:
//  * fwd_prefill_pp32d_kernel (more than 256 rows, 16-bit key/value), fwd_prefill_pp32_kernel
//    (more than 256 rows, fp8), both on 256-row subtiles, and fwd_prefill_ks32_kernel (65-256
//    rows, 128-row subtiles): two wave groups alternate MFMA and softmax items on the same SIMDs
//    over half pages (schedules described with each), on 32x32 MFMA tiles; pp32d moves K and V
//    into LDS by DMA, the others through registers;
//  * fwd_prefill_kernel (17-64 rows): all waves in phase, 16 rows each, whole pages through a
//    double-buffered LDS stage with one barrier per page, each page's keys split over 2
//    (33-64 rows) or 4 (17-32 rows) wave groups that hold the same rows, 16x16 MFMA tiles.
#include <stdint.h>

#include <atomic>

#include "split_merge.hpp"

namespace gbsa {
namespace {

// Bytes per V row in LDS (16-bit values). 320 = 256 + 64 shifts successive rows by 16 banks,
// so the eight rows of a transposing V read cover every bank equally often (LDS bank-conflict
// counter 0 on the bf16 prefill, against 13 % of the time with K's 304).
constexpr int kVPitch = 320;

template <int DT>
struct KLds {
    // bytes per K row in LDS: 304 = 256 + 48 gives the 16-byte fragment reads of 32 rows
    // distinct banks (measured fastest with the 32x32 tiles)
    static constexpr int pitch = (DT == kFP8) ? 144 : 304;
};

template <int DT>
struct PageStage {
    static constexpr int k_bytes = 128 * KLds<DT>::pitch;
    static constexpr int bytes = k_bytes + 128 * kVPitch;
};

// Per-thread share of one K or V page slice while it travels HBM/L2 -> registers -> LDS.
template <int DT, int NT, int ROWS = 128>
struct PageRegs {
    static constexpr int n16 = ROWS * ((DT == kFP8) ? 8 : 16) / NT;  // 16-B chunks per thread
    u32x4 x[n16];
};

template <int DT, int NT, int ROWS>
__device__ __forceinline__ void page_load(PageRegs<DT, NT, ROWS>& r, KvSrc page, int rs,
                                          int tid) {
    const rsrc_t rk = make_rsrc(page.p, page.records);
    constexpr int lanes_per_row = (DT == kFP8) ? 8 : 16;
    constexpr int rows_per_pass = NT / lanes_per_row;
    const int voff = (tid / lanes_per_row) * rs + (tid % lanes_per_row) * 16;
#pragma unroll
    for (int i = 0; i < PageRegs<DT, NT, ROWS>::n16; ++i)
        r.x[i] = buf_load16(rk, voff, i * rows_per_pass * rs);
}

// K rows into the K area of an LDS stage
template <int DT, int NT, int ROWS>
__device__ __forceinline__ void store_k(const PageRegs<DT, NT, ROWS>& r, unsigned char* stage,
                                        int tid) {
    constexpr int KP = KLds<DT>::pitch;
    constexpr int lanes_per_row = (DT == kFP8) ? 8 : 16;
    constexpr int rows_per_pass = NT / lanes_per_row;
    const int row0 = tid / lanes_per_row, col = tid % lanes_per_row;
#pragma unroll
    for (int i = 0; i < PageRegs<DT, NT, ROWS>::n16; ++i)
        *(u32x4*)(stage + (row0 + i * rows_per_pass) * KP + col * 16) = r.x[i];
}

// V rows (fp8 widened to bf16) into the V area `vs` of an LDS stage
template <int DT, int NT, int ROWS>
__device__ __forceinline__ void store_v(const PageRegs<DT, NT, ROWS>& r, unsigned char* vs,
                                        int tid) {
    constexpr int lanes_per_row = (DT == kFP8) ? 8 : 16;
    constexpr int rows_per_pass = NT / lanes_per_row;
    const int row0 = tid / lanes_per_row, col = tid % lanes_per_row;
#pragma unroll
    for (int i = 0; i < PageRegs<DT, NT, ROWS>::n16; ++i) {
        const int row = row0 + i * rows_per_pass;
        if constexpr (DT == kFP8) {
            const u32x4 vx = r.x[i];
            const u32x2 c0 = fp8x4_to_bf16x4(vx[0]), c1 = fp8x4_to_bf16x4(vx[1]);
            const u32x2 c2 = fp8x4_to_bf16x4(vx[2]), c3 = fp8x4_to_bf16x4(vx[3]);
            u32x4* vd = (u32x4*)(vs + row * kVPitch + col * 32);
            vd[0] = (u32x4){c0[0], c0[1], c1[0], c1[1]};
            vd[1] = (u32x4){c2[0], c2[1], c3[0], c3[1]};
        } else {
            *(u32x4*)(vs + row * kVPitch + col * 16) = r.x[i];
        }
    }
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// e4m3 x e4m3 with K = 128 per instruction (a 16-token tile against the whole head dim).
// A and B are loaded with the same head-dim assignment, so the product is the full dot
// product whatever order the instruction uses internally.
__device__ __forceinline__ f32x4 mfma_16x16x128_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1,
                                                    f32x4 c) {
    const i32x8 a = (i32x8){(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                            (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8 b = (i32x8){(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                            (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int NQ>
struct QTile {
    // 16-bit: [tile][head-dim chunk kk]: lane holds d = kk*32 + (lane/16)*8 .. +8
    // fp8:    [tile][0..1]: lane holds d = (lane/16)*32 .. +32
    u32x4 q[NQ][4];
};

// QK^T for one 16-token tile of a half page: sacc[nq] += K_tile Q^T.
template <int DT, int NQ>
__device__ __forceinline__ void qk_tile(const unsigned char* ks, const QTile<NQ>& qt, int row,
                                        int lgrp, f32x4 (&sacc)[NQ]) {
    constexpr int KP = KLds<DT>::pitch;
    const unsigned char* kr = ks + row * KP;
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) sacc[nq] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == kFP8) {
        const u32x4 a0 = *(const u32x4*)(kr + lgrp * 32);
        const u32x4 a1 = *(const u32x4*)(kr + lgrp * 32 + 16);
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq)
            sacc[nq] = mfma_16x16x128_fp8(a0, a1, qt.q[nq][0], qt.q[nq][1], sacc[nq]);
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const u32x4 ka = *(const u32x4*)(kr + (kk * 32 + lgrp * 8) * 2);
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq) sacc[nq] = mfma_16x16x32<DT>(ka, qt.q[nq][kk], sacc[nq]);
        }
    }
}

// Mask (when needed) and the running-max update of TT 16-token tiles starting at token tok0 of
// the page; returns the max to use.
template <int NQ, bool UM, int TT = 4>
__device__ __forceinline__ void half_max(const FwdArgs& a, f32x4 (&s)[TT][NQ], int tok0, int cls,
                                         const int (&vlo)[NQ], const int (&vhi)[NQ], int64_t p0,
                                         const UMaskRow (&um)[NQ], const float (&colscale)[NQ],
                                         int lgrp, float (&mrun)[NQ], float (&muse)[NQ],
                                         float (&alpha)[NQ]) {
    if (cls == 2) {
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rel = tok0 + tt * 16 + lgrp * 4 + i;
                    if (rel < vlo[nq] || rel > vhi[nq]) s[tt][nq][i] = kNegInf;
                }
    }
    if constexpr (UM) {  // the user mask applies to every visible block
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const uint32_t w = umask_word(a, um[nq], p0 + tok0 + tt * 16 + lgrp * 4);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if ((w >> (8 * i)) & 0xffu) s[tt][nq][i] = kNegInf;
            }
    }
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
        float mx = kNegInf;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tt][nq][i]);
        mx = wave_max_cols(mx);
        const float mnew = lazy_max(mrun[nq], mx == kNegInf ? kNegInf : mx * colscale[nq]);
        muse[nq] = (mnew == kNegInf) ? 0.f : mnew;
        alpha[nq] = fast_exp2(mrun[nq] - muse[nq]);
        mrun[nq] = mnew;
    }
}

// exp2 of one 16-token tile of S^T (all NQ columns) into packed 16-bit P^T, with row sums.
template <int PT, int NQ>
__device__ __forceinline__ void exp_tile(const f32x4 (&s)[NQ], const float (&colscale)[NQ],
                                         const float (&muse)[NQ], uint32_t (&pk)[NQ][2],
                                         float (&ls)[NQ]) {
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = fast_exp2(__builtin_fmaf(s[nq][i], colscale[nq], -muse[nq]));
            ls[nq] += pv[i];
        }
        pk[nq][0] = pack2<PT>(pv[0], pv[1]);
        pk[nq][1] = pack2<PT>(pv[2], pv[3]);
    }
}

// O^T += V^T P^T for one 32-token chunk kc of the staged V rows; pb[nq] is the B operand
// (P^T of token tiles 2kc, 2kc + 1 for query tile nq).
template <int PT, int NQ>
__device__ __forceinline__ void pv_chunk4(const unsigned char* vs, int kc, const u32x4 (&pb)[NQ],
                                          int lane, f32x4 (&o)[8][NQ]) {
    const int lrow = lane & 15, lgrp = lane >> 4;
    const unsigned char* vrow = vs + (kc * 32 + lgrp * 4 + (lrow >> 2)) * kVPitch + (lane & 3) * 8;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const u32x2 v0 = lds_read_tr16(vrow + dt * 32);
        const u32x2 v1 = lds_read_tr16(vrow + 16 * kVPitch + dt * 32);
        const u32x4 va = (u32x4){v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) o[dt][nq] = mfma_16x16x32<PT>(va, pb[nq], o[dt][nq]);
    }
}

template <int PT, int NQ>
__device__ __forceinline__ void pv_chunk(const unsigned char* vs, int kc, const uint32_t (&pa)[NQ][2],
                                         const uint32_t (&pb2)[NQ][2], int lane, f32x4 (&o)[8][NQ]) {
    u32x4 pb[NQ];
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) pb[nq] = (u32x4){pa[nq][0], pa[nq][1], pb2[nq][0], pb2[nq][1]};
    pv_chunk4<PT, NQ>(vs, kc, pb, lane, o);
}

template <int NQ>
__device__ __forceinline__ void rescale(float (&alpha)[NQ], f32x4 (&o)[8][NQ]) {
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
        if (__ballot(alpha[nq] != 1.f)) {  // skipped unless some running max moved
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) o[dt][nq] *= alpha[nq];
        }
    }
}

// State carried from the first to the second part of a key slice.
template <int NQ, int TT>
struct SliceMid {
    uint32_t p[TT][NQ][2];
};

// The wave's key slice of a page when the workgroup splits the keys: the TT 16-token tiles
// from token tok0 (a multiple of 32). Part A: QK^T, mask, running max, rescale, exp2 and row
// sums; part B: PV.
template <int DT, int NQ, bool UM, int TT>
__device__ __forceinline__ void slice_part_a(const FwdArgs& a, const unsigned char* stage,
                                             const QTile<NQ>& qt, const float (&colscale)[NQ],
                                             const int (&trow)[NQ], const UMaskRow (&um)[NQ],
                                             int j, int cls, int skv, int off, int lane, int tok0,
                                             float (&mrun)[NQ], float (&lrun)[NQ],
                                             f32x4 (&o)[8][NQ], SliceMid<NQ, TT>& mid) {
    constexpr int PT = (DT == kF16) ? kF16 : kBF16;
    const int lrow = lane & 15, lgrp = lane >> 4;
    int vlo[NQ], vhi[NQ];
    if (cls == 2) {
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq)
            key_range(a, (int64_t)j * 128, skv, (int64_t)trow[nq] + off, &vlo[nq], &vhi[nq]);
    }
    f32x4 s[TT][NQ];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) qk_tile<DT, NQ>(stage, qt, tok0 + tt * 16 + lrow, lgrp, s[tt]);
    float muse[NQ], alpha[NQ], ls[NQ];
    half_max<NQ, UM, TT>(a, s, tok0, cls, vlo, vhi, (int64_t)j * 128, um, colscale, lgrp, mrun,
                         muse, alpha);
    rescale<NQ>(alpha, o);
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) ls[nq] = 0.f;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) exp_tile<PT, NQ>(s[tt], colscale, muse, mid.p[tt], ls);
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) lrun[nq] = lrun[nq] * alpha[nq] + ls[nq];
}

template <int DT, int NQ, int TT>
__device__ __forceinline__ void slice_part_b(const unsigned char* stage, int lane, int tok0,
                                             f32x4 (&o)[8][NQ], const SliceMid<NQ, TT>& mid) {
    constexpr int PT = (DT == kF16) ? kF16 : kBF16;
    const unsigned char* vs = stage + PageStage<DT>::k_bytes;
#pragma unroll
    for (int c = 0; c < TT / 2; ++c)
        pv_chunk<PT, NQ>(vs, tok0 / 32 + c, mid.p[2 * c], mid.p[2 * c + 1], lane, o);
}

// Query tiles of this wave (B operand of S^T = K Q^T) and the per-column state.
template <int DT, int NQ>
__device__ __forceinline__ void load_q(const FwdArgs& a, const UnitIter& it, int t0, int rows_exist,
                                       int row0, int lane, QTile<NQ>& qt, float (&colscale)[NQ],
                                       int (&trow)[NQ], bool (&rvalid)[NQ]) {
    const int lrow = lane & 15, lgrp = lane >> 4;
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
        const int r = row0 + nq * 16 + lrow;
        const bool exists = r < rows_exist;
        const int t = t0 + (exists ? r / a.G : 0);
        const int h = it.n2 * a.G + (exists ? r % a.G : 0);
        trow[nq] = t;
        rvalid[nq] = exists && t < it.sq;
        float cs = a.scale_log2;
        if constexpr (DT == kFP8) cs *= a.qs[h] * a.ks[it.n2];
        colscale[nq] = cs;
        const int64_t qoff = ((it.row0 + t) * a.N1 + h) * 128;
        if constexpr (DT == kFP8) {
            const u32x4* qp = (const u32x4*)((const uint8_t*)a.q + qoff + lgrp * 32);
            qt.q[nq][0] = exists ? qp[0] : (u32x4){0, 0, 0, 0};
            qt.q[nq][1] = exists ? qp[1] : (u32x4){0, 0, 0, 0};
            qt.q[nq][2] = qt.q[nq][3] = (u32x4){0, 0, 0, 0};
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint16_t* qp = (const uint16_t*)a.q + qoff + kk * 32 + lgrp * 8;
                qt.q[nq][kk] = exists ? *(const u32x4*)qp : (u32x4){0, 0, 0, 0};
            }
        }
    }
}

// Normalised O and LSE of this wave's rows (whole selection), or the unnormalised partial
// (O, running max, row sum) of a split unit into workspace slot `slot`.
template <int DT, int OUT, int NQ>
__device__ __forceinline__ void write_rows(const FwdArgs& a, const UnitIter& it, bool complete,
                                           int slot, int row0, int lane, const int (&trow)[NQ],
                                           const bool (&rvalid)[NQ], const float (&mrun)[NQ],
                                           const float (&lrun)[NQ], const f32x4 (&o)[8][NQ]) {
    const int lrow = lane & 15, lgrp = lane >> 4;
    const float vscale = (DT == kFP8) ? a.vs[it.n2] : 1.f;
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
        const float ltot = wave_sum_cols(lrun[nq]);
        const int r = row0 + nq * 16 + lrow;
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
                const u32x2 v2 = (u32x2){pack2<OUT>(o[dt][nq][0] * inv, o[dt][nq][1] * inv),
                                         pack2<OUT>(o[dt][nq][2] * inv, o[dt][nq][3] * inv)};
                *(u32x2*)(op + d) = v2;
            }
            if (a.return_lse && lgrp == 0)
                a.lse[orow] = ltot > 0.f ? (mrun[nq] + __log2f(ltot)) * kLn2 : kNegInf;
        } else {
            const rsrc_t ro = ws_o_rsrc(a, slot);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const int d = dt * 16 + lgrp * 4;
                ws_put4(ro, (r * 128 + d) * 4, o[dt][nq] * vscale);
            }
            if (lgrp == 0) {
                ws_put1(a.ws_m + (int64_t)slot * a.M + r, mrun[nq]);
                ws_put1(a.ws_l + (int64_t)slot * a.M + r, ltot);
            }
        }
    }
}

// Every page's keys are split KS ways: waves rw, rw + RW, ... (RW = NW / KS) hold the same
// NQ*16 rows and take token slices 0, 128/KS, ... of each page, so each staged page is read
// from LDS KS times rather than once per wave; the slices' softmax states are combined through
// LDS at the end of the task (FA article, "three steps").
template <int DT, int OUT, int NW, int NQ, int KS, int LAYOUT, bool UM>
__global__ __launch_bounds__(NW * 64, 1) void fwd_prefill_kernel(FwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int RW = NW / KS;  // waves per key slice
    constexpr int R = RW * NQ * 16;
    constexpr int TT = 128 / KS / 16;  // 16-token tiles per key slice
    constexpr int esz = (DT == kFP8) ? 1 : 2;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * PageStage<DT>::bytes];
    static_assert(sizeof(smem) >= kPieceListBytes, "the split merge borrows the stages");
    static_assert(KS > 1 && NQ == 1 && NW % KS == 0 && TT % 2 == 0, "key split shape");
    static_assert((KS - 1) * RW * (8 * 64 * 16 + 2 * 64 * 4) <= (int)sizeof(smem),
                  "the key-slice merge fits in the stages");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform for the compiler
    const int rw = wave % RW, kp = wave / RW;  // row wave and key slice
    const int lrow = lane & 15, lgrp = lane >> 4;
    if (!header_ok(a)) {
        refuse(a);
        return;
    }
    const int U = a.meta[3];
    __shared__ int task_word[2];
    run_tasks<!UM>(a, U, task_word, [&](const FwdArgs& a, const Task& tk) {
        const int w = tk.w, st = tk.st;
        const Bound b0 = tk.b0, b1 = tk.b1;
        if (!bound_less(b0, b1) || b0.u >= U) return;
        UnitIter it = locate_unit(a, b0.u);
        if (it.b < 0) return;

        const int rs = a.N2 * 128 * esz;  // bytes between tokens of a page

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
                const KvSeq kv = kv_seq<LAYOUT>(a, it.b);
                const int skv = kv.len;
                const int off = diag_off(a, skv, it.sq);
                QTile<NQ> qt;
                float colscale[NQ];
                int trow[NQ];
                bool rvalid[NQ];
                load_q<DT, NQ>(a, it, t0, rows_exist, row_base + rw * NQ * 16, lane, qt, colscale,
                               trow, rvalid);
                UMaskRow um[NQ];
#pragma unroll
                for (int nq = 0; nq < NQ; ++nq)
                    um[nq] = UM ? umask_row(a, it.b, trow[nq], rvalid[nq])
                                : UMaskRow{make_rsrc(nullptr, 0), -1};
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
                const int64_t head_off = (int64_t)it.n2 * 128 * esz;

                // ---- stream the task's visible pages through the double-buffered stage ------
                // lane l of every wave holds slot c0 + l of the current 64-slot chunk
                PageRegs<DT, NT, 128> pr;
                SliceMid<NQ, TT> smid;
                const int tok0 = kp * (128 / KS);
                int buf = 0;
                bool have_prev = false;  // a page is waiting in stage[buf]
                int prev_j = 0, prev_cls = 0;
                for (int c0 = sa; c0 < se; c0 += 64) {
                    const int n = min(64, se - c0);
                    int jl = -1, pl = 0, cl = 0;
                    if (lane < n) {
                        jl = sel[c0 + lane];
                        if (jl >= 0) {
                            cl = block_class(a, (int64_t)jl * 128, skv, off, t_lo, t_hi);
                            if (cl != 0) pl = kv.unit<LAYOUT>(jl);
                        }
                    }
                    uint64_t todo = __ballot(cl != 0);
                    while (todo) {
                        const int i = __builtin_ctzll(todo);
                        todo &= todo - 1;
                        const int unit = __builtin_amdgcn_readlane(pl, i);
                        const int64_t pb = (int64_t)unit * a.kv_stride * esz + head_off;
                        const int nv = skv - 128 * __builtin_amdgcn_readlane(jl, i);
                        // the first page goes straight into stage[buf]; later ones into the
                        // other buffer while stage[buf] is consumed
                        unsigned char* cur = smem + buf * PageStage<DT>::bytes;
                        unsigned char* dst = have_prev ? smem + (buf ^ 1) * PageStage<DT>::bytes : cur;
                        page_load<DT, NT>(pr, kv_src(a.k, pb, rs, nv), rs, tid);
                        if (have_prev)
                            slice_part_a<DT, NQ, UM, TT>(a, cur, qt, colscale, trow, um, prev_j,
                                                         prev_cls, skv, off, lane, tok0, mrun, lrun,
                                                         o, smid);
                        store_k<DT, NT>(pr, dst, tid);
                        page_load<DT, NT>(pr, kv_src(a.v, pb, rs, nv), rs, tid);
                        if (have_prev) slice_part_b<DT, NQ, TT>(cur, lane, tok0, o, smid);
                        store_v<DT, NT>(pr, dst + PageStage<DT>::k_bytes, tid);
                        if (have_prev) buf ^= 1;
                        __syncthreads();
                        have_prev = true;
                        prev_j = __builtin_amdgcn_readlane(jl, i);
                        prev_cls = __builtin_amdgcn_readlane(cl, i);
                    }
                }
                if (have_prev) {
                    unsigned char* cur = smem + buf * PageStage<DT>::bytes;
                    slice_part_a<DT, NQ, UM, TT>(a, cur, qt, colscale, trow, um, prev_j, prev_cls,
                                                 skv, off, lane, tok0, mrun, lrun, o, smid);
                    slice_part_b<DT, NQ, TT>(cur, lane, tok0, o, smid);
                }
                __syncthreads();  // the stage is reused by the next task

                {
                    // key slices 1..KS-1 hand (O, running max, row sums) to slice 0 through the
                    // free stage memory; the lane layout is the same in every slice
                    f32x4* so = (f32x4*)smem;
                    float* sml = (float*)(smem + (KS - 1) * RW * 8 * 64 * 16);
                    if (kp > 0) {
                        const int slot = (kp - 1) * RW + rw;
#pragma unroll
                        for (int dt = 0; dt < 8; ++dt) so[(slot * 8 + dt) * 64 + lane] = o[dt][0];
                        sml[slot * 128 + lane] = mrun[0];
                        sml[slot * 128 + 64 + lane] = lrun[0];
                    }
                    __syncthreads();
                    if (kp == 0) {
#pragma unroll
                        for (int k = 1; k < KS; ++k) {
                            const int slot = (k - 1) * RW + rw;
                            const float m1 = sml[slot * 128 + lane], l1 = sml[slot * 128 + 64 + lane];
                            const float m = fmaxf(mrun[0], m1);
                            const float f0 = (m == kNegInf) ? 0.f : fast_exp2(mrun[0] - m);
                            const float f1 = (m == kNegInf) ? 0.f : fast_exp2(m1 - m);
                            mrun[0] = m;
                            lrun[0] = lrun[0] * f0 + l1 * f1;
#pragma unroll
                            for (int dt = 0; dt < 8; ++dt)
                                o[dt][0] = o[dt][0] * f0 + so[(slot * 8 + dt) * 64 + lane] * f1;
                        }
                    }
                    __syncthreads();  // the stage is reused by the next task
                }

                // ---- epilogue: normalised output + LSE, or a split-KV partial --------------
                if (kp == 0)
                    write_rows<DT, OUT, NQ>(a, it, complete, 2 * w + (sa > 0 ? 0 : 1),
                                            row_base + rw * NQ * 16, lane, trow, rvalid, mrun, lrun,
                                            o);
                if (!complete) {
                    int* list = (int*)smem;  // the stages are free until the next task
                    const int np = piece_arrive(a, w, u, st, a.nst, list);
                    if (np > 0)
                        merge_rows<OUT>(a, list, np, row_base, min(row_base + R, rows_exist), it.n2,
                                        t0, it.row0, it.sq);
                    __syncthreads();
                }
            }
            advance_unit(a, it);
        }
    });
}


// ---------------------------------------------------------------------------------------------
// 256-row units: two-group ping-pong over half pages.
//
// Waves w and w + 4 of a workgroup share a SIMD. Waves 0-3 (group 0) and 4-7 (group 1) each
// hold 32 query rows per wave and run the same sequence of items over the task's 2n visible
// half pages (64 tokens each), group 1 one barrier slot behind group 0:
//   MFMA item k (k = 0..2n):      S_k = K_k Q^T (k < 2n)  and  O += V_{k-1}^T P_{k-1}^T (k > 0)
//   softmax item k (k < 2n):      mask, running max, rescale of O, P_k = exp2(.), row sums
// so in every slot one wave of each SIMD issues MFMAs while its partner does the softmax and
// moves its group's share of the KV stream into LDS (group 0: V_k, group 1: K_{k+2}). K_k and
// V_k live in LDS buffer k % 2; each is written one slot after the last read of the half page
// that used the buffer before it, which the slot order guarantees.
// ---------------------------------------------------------------------------------------------

// 16-bit K and V rows with one LDS pitch can share one store routine
constexpr bool kSharedPitch = KLds<kBF16>::pitch == kVPitch;

// Bytes per fp8 V row in LDS when P·V runs on fp8 MFMA (V kept as e4m3): 160 = 128 + 32 puts the
// eight rows of each half-wave of an 8-bit transposing read (32 bytes per row) on distinct
// 8-bank groups (row r at bank 40 r mod 64).
constexpr int kV8Pitch = 160;

template <int DT, bool P8 = false>
struct HalfStage {
    static constexpr int k_bytes = 64 * KLds<DT>::pitch;
    static constexpr int v_bytes = 64 * (P8 ? kV8Pitch : kVPitch);
};

// fp8 V rows as they are (P·V on fp8 MFMA) into the V area `vs` of a stage, pitch kV8Pitch
template <int NT, int ROWS>
__device__ __forceinline__ void store_v8(const PageRegs<kFP8, NT, ROWS>& r, unsigned char* vs,
                                         int tid) {
    constexpr int lanes_per_row = 8;
    constexpr int rows_per_pass = NT / lanes_per_row;
    const int row0 = tid / lanes_per_row, col = tid % lanes_per_row;
#pragma unroll
    for (int i = 0; i < PageRegs<kFP8, NT, ROWS>::n16; ++i)
        *(u32x4*)(vs + (row0 + i * rows_per_pass) * kV8Pitch + col * 16) = r.x[i];
}

// 8-bit transpose read from LDS (ds_read_b64_tr_b8). Within each group of 16 lanes, lanes 2r and
// 2r + 1 supply the two 8-byte halves of row r of an 8 x 16-byte block; lane i receives column
// i, i.e. the bytes block[0..7][i].
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                         (GBSA_LDS i32x2*)(p)));
}

// LDS fragments in flight in the MFMA item
constexpr int kPipeDepth = 4;

// One LDS operand fragment of the MFMA item (b is used by the fp8 QK step only).
struct Frag {
    u32x4 a, b;
};

// ---------------------------------------------------------------------------------------------
// 32x32 MFMA tiles (v_mfma_f32_32x32x16_{bf16,f16}; fp8 QK^T: v_mfma_scale_f32_32x32x64_f8f6f4).
// Half the instructions of the 16x16 forms for the same work, which leaves the partner wave of
// a SIMD more VALU issue. Lane layouts (checked on the hardware): A (32 x K): lane l holds row
// l % 32 and k slots (h = l / 32, j); B (K x 32): lane l holds column l % 32 and the same k
// slots; C (32 x 32): lane l holds column l % 32, element i at row 8 (i / 4) + 4 h + i % 4.
// With S^T = K Q^T a lane therefore holds, for its query row, keys 8 (i / 4) + 4 h + i % 4 of
// each 32-key tile. PV contracts over keys in whatever order the lane's P values come: k slot
// (h, j) of chunk c = 2 t + a is key 32 t + 16 a + 8 (j / 4) + 4 h + j % 4, and the V^T operand
// is read with the transpose read in that same order.
// ---------------------------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int DT>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == kF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// e4m3 x e4m3, K = 64 per instruction: lane holds 32 consecutive head dims (h = l / 32).
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1,
                                                    f32x16 c) {
    const i32x8 a = (i32x8){(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                            (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8 b = (i32x8){(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                            (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Query column of a wave (32 rows, one per lane pair l, l + 32) as B operands of S^T = K Q^T.
//  16-bit: q[kk] holds head dims 16 kk + 8 h .. + 8.   fp8: q[2 ks + e] holds 64 ks + 32 h + 16 e .. + 16.
struct QCol32 {
    u32x4 q[8];
};

template <int DT>
__device__ __forceinline__ void load_q32(const FwdArgs& a, const UnitIter& it, int t0,
                                         int rows_exist, int row0, int lane, QCol32& qc,
                                         float& colscale, int& trow, bool& rvalid) {
    const int h2 = lane >> 5;
    const int r = row0 + (lane & 31);
    const bool exists = r < rows_exist;
    const int t = t0 + (exists ? r / a.G : 0);
    const int h = it.n2 * a.G + (exists ? r % a.G : 0);
    trow = t;
    rvalid = exists && t < it.sq;
    float cs = a.scale_log2;
    if constexpr (DT == kFP8) cs *= a.qs[h] * a.ks[it.n2];
    colscale = cs;
    const int64_t qoff = ((it.row0 + t) * a.N1 + h) * 128;
    const u32x4 z = (u32x4){0, 0, 0, 0};
    if constexpr (DT == kFP8) {
        const uint8_t* qp = (const uint8_t*)a.q + qoff;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                qc.q[2 * ks + e] = exists ? *(const u32x4*)(qp + 64 * ks + 32 * h2 + 16 * e) : z;
#pragma unroll
        for (int kk = 4; kk < 8; ++kk) qc.q[kk] = z;
    } else {
        const uint16_t* qp = (const uint16_t*)a.q + qoff;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qc.q[kk] = exists ? *(const u32x4*)(qp + 16 * kk + 8 * h2) : z;
    }
}

// MFMA item on 32x32 tiles: QK^T of a half page (two 32-key tiles) and PV of the previous one,
// as a software-pipelined sequence of steps (one LDS fragment and the MFMA that uses it).
// P8 (fp8 with a P quantisation scale): PV on v_mfma_scale_f32_32x32x64_f8f6f4, one instruction
// per 32 head dims for the whole half page, V^T read from the fp8 rows with the 8-bit transpose
// read (four reads give a lane its 32 keys in order) and P as fp8 in the same key order (p[0],
// p[1], from the softmax item).
template <int DT, bool qk, bool pv, bool P8 = false>
__device__ __forceinline__ void mfma_item32(const unsigned char* ks, const unsigned char* vs,
                                            const QCol32& qc, f32x16 (&s)[2],
                                            const u32x4 (&p)[4], f32x16 (&o)[4], int lane) {
    static_assert(!P8 || DT == kFP8, "fp8 P is the fp8 path");
    constexpr int PT = (DT == kF16) ? kF16 : kBF16;
    constexpr int KP = KLds<DT>::pitch;
    constexpr int QS = qk ? ((DT == kFP8) ? 2 : 8) : 0;  // QK steps per 32-key tile
    // PV steps per 32-key tile: 2 chunks x 4 d tiles, or with fp8 P two d tiles of 64 keys
    constexpr int VS = pv ? (P8 ? 2 : 8) : 0;
    constexpr int PC = QS + VS, NS = 2 * PC, D = kPipeDepth;
    const int h2 = lane >> 5;
    const unsigned char* krow = ks + (lane & 31) * KP;
    // transpose-read address of this lane (row offset within a 4-row group, column block)
    const unsigned char* vbase = vs + (4 * h2 + ((lane & 15) >> 2)) * kVPitch +
                                 (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    // fp8 V^T: this lane's row within the 8-row block of read m (keys 32 h + 8 m ..) and byte
    // column (head dims 16 (lane / 16 % 2) + 8 (lane % 2) of the d tile)
    const unsigned char* v8base = vs + (32 * h2 + ((lane & 15) >> 1)) * kV8Pitch +
                                  16 * ((lane >> 4) & 1) + 8 * (lane & 1);
    const f32x16 zero = {};

    auto load = [&](int st) {
        Frag f;
        const int t = st / PC, j = st % PC;
        if (j < QS) {
            if constexpr (DT == kFP8) {
                const unsigned char* kr = krow + t * 32 * KP + 64 * j + 32 * h2;
                f.a = *(const u32x4*)kr;
                f.b = *(const u32x4*)(kr + 16);
            } else {
                f.a = *(const u32x4*)(krow + t * 32 * KP + (16 * j + 8 * h2) * 2);
            }
        } else if constexpr (P8) {
            const int dt = 2 * t + (j - QS);  // d tile: head dims 32 dt .. 32 dt + 31
            const unsigned char* vr = v8base + 32 * dt;
            const u32x2 r0 = lds_read_tr8(vr), r1 = lds_read_tr8(vr + 8 * kV8Pitch);
            const u32x2 r2 = lds_read_tr8(vr + 16 * kV8Pitch), r3 = lds_read_tr8(vr + 24 * kV8Pitch);
            f.a = (u32x4){r0[0], r0[1], r1[0], r1[1]};
            f.b = (u32x4){r2[0], r2[1], r3[0], r3[1]};
        } else {
            const int v = j - QS, a2 = v >> 2, dt = v & 3;  // chunk 2t + a2, d tile dt
            const unsigned char* vr = vbase + (32 * t + 16 * a2) * kVPitch + dt * 64;
            const u32x2 v0 = lds_read_tr16(vr);
            const u32x2 v1 = lds_read_tr16(vr + 8 * kVPitch);
            f.a = (u32x4){v0[0], v0[1], v1[0], v1[1]};
        }
        return f;
    };
    auto compute = [&](int st, const Frag& f) {
        const int t = st / PC, j = st % PC;
        if (j < QS) {
            if constexpr (DT == kFP8)
                s[t] = mfma_32x32x64_fp8(f.a, f.b, qc.q[2 * j], qc.q[2 * j + 1], j == 0 ? zero : s[t]);
            else
                s[t] = mfma_32x32x16<DT>(f.a, qc.q[j], j == 0 ? zero : s[t]);
        } else if constexpr (P8) {
            const int dt = 2 * t + (j - QS);
            o[dt] = mfma_32x32x64_fp8(f.a, f.b, p[0], p[1], o[dt]);
        } else {
            const int v = j - QS, a2 = v >> 2, dt = v & 3;
            o[dt] = mfma_32x32x16<PT>(f.a, p[2 * t + a2], o[dt]);
        }
    };
    Frag fr[D];
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (i < NS) fr[i] = load(i);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const Frag f = fr[st % D];
        if (st + D < NS) fr[st % D] = load(st + D);
        compute(st, f);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// User-mask words of one softmax item (keys half * 64 .. + 63 of block j) for this lane's
// row, in element order: word 4 t + q holds keys 32 t + 8 q + 4 h .. + 3 of the half page.
// Loaded one MFMA item ahead of their use, so the latency hides behind it.
__device__ __forceinline__ void umask_words32(const FwdArgs& a, const UMaskRow& um, int j,
                                              int half, int lane, uint32_t (&w)[8]) {
    const int h2 = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[4 * t + q] = umask_word(a, um, (int64_t)j * 128 + half * 64 + 32 * t + 8 * q + 4 * h2);
}

// The lazy bound of the running max (device_common.hpp) on probabilities: 2^kLazyMax. The 32-row
// softmax items test it on the lane's sum of probabilities, which bounds each of them.
constexpr float kLazyBound = 256.f;

// Softmax item on 32x32 tiles for half page `half` of block j (class cls): mask, then P^T as
// the PV B operands and the row sums against the running max. The block max (in-lane max over
// 32 keys, then the lane pair l, l ^ 32) is taken on every item by the fp8-P and HS forms, which
// move the running max where the block max exceeds it (fp8 P) or exceeds it by more than the
// lazy bound (HS); the 16-bit-P form takes it only where the item leaves the lazy bound or a row
// has seen no key yet. O is rescaled only where the running max moves.
// HS (f16 only): softmax precision 1 of the GBSA article's "softmax precision" section. The
// online-softmax stage runs in the output's 16-bit type: the logits are rounded to f16, and the
// scaling and max subtraction (packed f16 FMA) and the exponentials are f16; the block max is
// taken on the fp32 logits and the running max kept at an f16 value, and the rescale of O and
// the row sums stay fp32 (the sums accumulate the f16 exponentials with v_dot2_f32_f16, so they
// add exactly the P that the PV product uses).
// P8 (quant mode 5 with a P quantisation scale, GBSA article "quantisation": FP8_E4M3_STATIC_CAST_P):
// P is cast to e4m3 after scaling by pq (the row's p_quant_scale, at most the destination
// type's max) and handed to the fp8 P·V product in its B-operand order: lane l needs the 32 keys
// 32 h .. 32 h + 31 (h = l / 32) in order and holds, per 32-key tile, the 16 keys 8 u + 4 h + r;
// one v_permlane32_swap per dword u trades the other lane half's share (tile 0 to the low half,
// tile 1 to the high half). The running max is exact (no lazy threshold), so P <= 1 and
// P * pq stays within the type. The row sums add the unquantised P in fp32.
template <int DT, bool UM, bool HS = false, bool P8 = false>
__device__ __forceinline__ void softmax_item32(const FwdArgs& a, f32x16 (&s)[2], u32x4 (&p)[4],
                                               float colscale, int trow, const uint32_t (&umw)[8],
                                               int j, int half, int cls, int skv, int off,
                                               int lane, float& mrun, float& lrun,
                                               f32x16 (&o)[4], float pq = 1.f) {
    constexpr int PT = (DT == kF16) ? kF16 : kBF16;
    const int h2 = lane >> 5;
    if (cls == 2) {
        int vlo, vhi;
        key_range(a, (int64_t)j * 128, skv, (int64_t)trow + off, &vlo, &vhi);
        // element (t, i) of this lane is key half * 64 + 32 t + 8 (i / 4) + 4 h + i % 4 of the page
        const int lo = vlo - half * 64 - 4 * h2, hi = vhi - half * 64 - 4 * h2;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c = 32 * t + 8 * (i / 4) + (i % 4);
                const uint32_t out = (uint32_t)(((c - lo) | (hi - c)) >> 31);  // ~0 outside
                // (bit_cast of a vector element reads element 0: go through a scalar copy)
                const float x = s[t][i];
                s[t][i] = __uint_as_float((__float_as_uint(x) & ~out) | (0xff800000u & out));
            }
    }
    if constexpr (UM) {  // the user mask applies to every visible block
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if ((umw[4 * t + q] >> (8 * r)) & 0xffu) s[t][4 * q + r] = kNegInf;
    }
    if constexpr (HS) {
        static_assert(DT == kF16, "the 16-bit softmax is the f16 path");
        // pair q = 4 c + e holds elements 8 (c & 1) + 2 e and + 1 of tile c >> 1: the order of P
        f16x2 h[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int t = q >> 3, i = 8 * ((q >> 2) & 1) + 2 * (q & 3);
            const float x0 = s[t][i], x1 = s[t][i + 1];
            h[q] = __builtin_convertvector((f32x2){x0, x1}, f16x2);
        }
        // the block max from the fp32 logits, and a running max that f16 represents exactly:
        // the f16 subtraction then removes exactly the max the LSE is built on
        float mx = kNegInf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
        mx = pair_max(mx, true);
        float mnew = lazy_max(mrun, mx == kNegInf ? kNegInf : mx * colscale);
        if (mnew != mrun && mnew != kNegInf) mnew = (float)(_Float16)mnew;
        const float muse = (mnew == kNegInf) ? 0.f : mnew;
        const float alpha = fast_exp2(mrun - muse);
        mrun = mnew;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
        }
        const _Float16 c16 = (_Float16)colscale, m16 = (_Float16)(-muse);
        const f16x2 cc = {c16, c16}, mm = {m16, m16}, one = {(_Float16)1.f, (_Float16)1.f};
        float ls = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f16x2 x = __builtin_elementwise_fma(h[4 * c + e], cc, mm);
                const f16x2 e2 = __builtin_elementwise_exp2(x);
                ls = __builtin_amdgcn_fdot2(e2, one, ls, false);
                w[e] = __builtin_bit_cast(uint32_t, e2);
            }
            p[c] = (u32x4){w[0], w[1], w[2], w[3]};
        }
        lrun = lrun * alpha + ls;
        return;
    }
    // exponentials of the item against the shift mu, packed as the PV B operands; returns the
    // lane's sum of the fp32 values. Chunk c = 2 t + a: elements 8 a .. 8 a + 7 of tile t.
    auto exp_pack = [&](float mu) {
        float ls = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = fast_exp2(__builtin_fmaf(s[c >> 1][8 * (c & 1) + e], colscale, -mu));
                ls += pv[e];
            }
            p[c] = (u32x4){pack2<PT>(pv[0], pv[1]), pack2<PT>(pv[2], pv[3]),
                           pack2<PT>(pv[4], pv[5]), pack2<PT>(pv[6], pv[7])};
        }
        return ls;
    };
    if constexpr (!P8) {
        // Against the running max as it stands, without the block max: every probability is at
        // most the lane's sum, so a sum within 2^kLazyMax keeps the lazy bound. Only where some
        // lane's sum leaves it (or is not a number), or a row has seen no key yet, is the block
        // max taken and the item recomputed with the running max moved to it (exact, as the
        // FA article's online softmax); there O is rescaled. The max is the one the exponentials
        // use, so the result does not depend on when it moves.
        float ls = exp_pack((mrun == kNegInf) ? 0.f : mrun);
        float alpha = 1.f;
        if (__builtin_amdgcn_ballot_w64(mrun == kNegInf || !(ls <= kLazyBound))) {
            float mx = kNegInf;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
            mx = pair_max(mx, true);
            const float mnew = fmaxf(mrun, mx == kNegInf ? kNegInf : mx * colscale);
            const float muse = (mnew == kNegInf) ? 0.f : mnew;
            alpha = fast_exp2(mrun - muse);
            mrun = mnew;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
            ls = exp_pack(muse);
        }
        lrun = lrun * alpha + ls;
    } else {
        // fp8 P: the exact running max, moved (with its exp2 and the O rescale) only where some
        // row's block max exceeds it; elsewhere alpha is 1
        float mx = kNegInf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
        mx = pair_max(mx, true);
        const float bmax = mx == kNegInf ? kNegInf : mx * colscale;
        float alpha = 1.f;
        if (__builtin_amdgcn_ballot_w64(bmax > mrun)) {
            const float mnew = fmaxf(mrun, bmax);
            alpha = fast_exp2(mrun - ((mnew == kNegInf) ? 0.f : mnew));
            mrun = mnew;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
        }
        const float muse = (mrun == kNegInf) ? 0.f : mrun;
        float ls = 0.f;
        uint32_t q8[2][4];  // [tile][u]: keys 8 u + 4 h .. + 3, e4m3, scaled by pq
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float pv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pv[r] = fast_exp2(__builtin_fmaf(s[t][4 * u + r], colscale, -muse));
                    ls += pv[r];
                }
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0] * pq, pv[1] * pq, 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2] * pq, pv[3] * pq, w, true);
                q8[t][u] = (uint32_t)w;
            }
        uint32_t b[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const auto r = __builtin_amdgcn_permlane32_swap(q8[0][u], q8[1][u], false, false);
            b[2 * u] = (uint32_t)r[0];
            b[2 * u + 1] = (uint32_t)r[1];
        }
        p[0] = (u32x4){b[0], b[1], b[2], b[3]};
        p[1] = (u32x4){b[4], b[5], b[6], b[7]};
        lrun = lrun * alpha + ls;
    }
}

// Fixes the softmax item's results where they are computed. The exponentials and conversions
// are plain arithmetic, which the compiler may sink past the barrier that follows into the next
// slot; there they would run one after the other with the wave's own MFMA item instead of beside
// the partner wave's. The empty statement claims to read and rewrite them, so nothing that
// produces them can move below it.
__device__ __forceinline__ void pin_softmax(u32x4 (&p)[4], float& lrun) {
    asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(lrun));
}

// The P quantisation scale of this lane's query row (quant mode 5 with p_quant_scale): the
// row's head's scale, at most the destination type's max (P <= 1, so P * scale stays in range).
__device__ __forceinline__ float p_quant(const FwdArgs& a, const UnitIter& it, int row0,
                                         int rows_exist, int lane) {
    const int r = row0 + (lane & 31);
    const int h = it.n2 * a.G + (r < rows_exist ? r % a.G : 0);
    return fminf(a.ps[h], a.ps_max);
}

// Normalised O and LSE of a wave's 32 rows (lane pair l, l + 32 per row), or the split partial.
template <int DT, int OUT>
__device__ __forceinline__ void write_rows32(const FwdArgs& a, const UnitIter& it, bool complete,
                                             int slot, int row0, int lane, int trow, bool rvalid,
                                             float mrun, float lrun, const f32x16 (&o)[4],
                                             float pdeq = 1.f) {
    const int h2 = lane >> 5;
    const float ltot = pair_sum(lrun, true);
    const int r = row0 + (lane & 31);
    if (!rvalid) return;
    // (pdeq: 1 / the P quantisation scale when P·V ran on fp8)
    const float vscale = ((DT == kFP8) ? a.vs[it.n2] : 1.f) * pdeq;
    if (complete) {
        const float inv = ltot > 0.f ? vscale / ltot : 0.f;
        const int h = it.n2 * a.G + r % a.G;
        const int64_t orow = ((it.row0 + trow) * a.N1 + h);
        uint16_t* op = (uint16_t*)a.out + orow * 128;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {  // elements 4 g .. 4 g + 3: head dims dt*32 + 8 g + 4 h ..
                const int d = dt * 32 + 8 * g + 4 * h2;
                *(u32x2*)(op + d) = (u32x2){pack2<OUT>(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                                            pack2<OUT>(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
            }
        if (a.return_lse && h2 == 0)
            a.lse[orow] = ltot > 0.f ? (mrun + __log2f(ltot)) * kLn2 : kNegInf;
    } else {
        const rsrc_t ro = ws_o_rsrc(a, slot);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = dt * 32 + 8 * g + 4 * h2;
                ws_put4(ro, (r * 128 + d) * 4,
                        (f32x4){o[dt][4 * g], o[dt][4 * g + 1], o[dt][4 * g + 2],
                                o[dt][4 * g + 3]} * vscale);
            }
        if (h2 == 0) {
            ws_put1(a.ws_m + (int64_t)slot * a.M + r, mrun);
            ws_put1(a.ws_l + (int64_t)slot * a.M + r, ltot);
        }
    }
}


// The 256-row kernel (schedule above) on 32x32 tiles: each wave's 32 query rows are one
// 32-column tile.
template <int DT, int OUT, int LAYOUT, bool UM, bool P8 = false>
__global__ __launch_bounds__(512, 1) void fwd_prefill_pp32_kernel(FwdArgs a) {
    constexpr int R = 256;
    constexpr int esz = (DT == kFP8) ? 1 : 2;
    constexpr int KB = HalfStage<DT, P8>::k_bytes, VB = HalfStage<DT, P8>::v_bytes;
    // [K buffer 0][K buffer 1][V buffer 0][V buffer 1]
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * KB + 2 * VB];
    // the task's visible blocks in order: (unit, j * 4 + class, records of half 0, of half 1)
    __shared__ int4 plist[256];
    __shared__ int flag[1];
    static_assert(sizeof(smem) >= kPieceListBytes, "the split merge borrows the stages");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;  // waves w and w + 4 share a SIMD
    const int tg = tid & 255;   // thread index within the group
    if (!header_ok(a)) {
        refuse(a);
        return;
    }
    const int U = a.meta[3];
    __shared__ int task_word[2];
    run_tasks<!UM>(a, U, task_word, [&](const FwdArgs& a, const Task& tk) {
        const int w = tk.w, st = tk.st;
        const Bound b0 = tk.b0, b1 = tk.b1;
        if (!bound_less(b0, b1) || b0.u >= U) return;
        UnitIter it = locate_unit(a, b0.u);
        if (it.b < 0) return;

        const int rs = a.N2 * 128 * esz;  // bytes between tokens of a page
        const unsigned char* kbase = (const unsigned char*)a.k;
        const unsigned char* vbase = (const unsigned char*)a.v;
        unsigned char* const kst = smem;
        unsigned char* const vst = smem + 2 * KB;

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
            const int row_base = st * R;
            if (row_base < rows_exist) {
                const KvSeq kv = kv_seq<LAYOUT>(a, it.b);
                const int skv = kv.len;
                const int off = diag_off(a, skv, it.sq);
                const int row0 = row_base + wave * 32;
                QCol32 qc;
                float colscale, mrun = kNegInf, lrun = 0.f;
                int trow;
                bool rvalid;
                load_q32<DT>(a, it, t0, rows_exist, row0, lane, qc, colscale, trow, rvalid);
                const float pq = P8 ? p_quant(a, it, row0, rows_exist, lane) : 1.f;
                const UMaskRow um =
                    UM ? umask_row(a, it.b, trow, rvalid) : UMaskRow{make_rsrc(nullptr, 0), -1};
                f32x16 o[4];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] = (f32x16){};
                const int t_lo = t0 + row_base / a.G;
                const int t_hi = t0 + (min(row_base + R, rows_exist) - 1) / a.G;
                const int32_t* sel = a.idx + ((int64_t)it.n2 * a.tqb + g) * a.topK;
                const int64_t head_off = (int64_t)it.n2 * 128 * esz;

                // ---- visible pages of this task's selection range, compacted in order ---------
                if (wave == 0) {
                    int n = 0;
                    for (int c0 = sa; c0 < se; c0 += 64) {
                        int jl = -1, pl = 0, cl = 0;
                        if (c0 + lane < se) {
                            jl = sel[c0 + lane];
                            if (jl >= 0) {
                                cl = block_class(a, (int64_t)jl * 128, skv, off, t_lo, t_hi);
                                if (cl != 0) pl = kv.unit<LAYOUT>(jl);
                            }
                        }
                        const uint64_t m = __ballot(cl != 0);
                        if (cl != 0) {
                            const int pos = n + __builtin_amdgcn_mbcnt_hi(
                                                    (uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                            plist[pos] = make_int4(pl, jl * 4 + cl,
                                                   kv_records(rs, skv - 128 * jl),
                                                   kv_records(rs, skv - 128 * jl - 64));
                        }
                        n += __builtin_popcountll(m);
                    }
                    if (lane == 0) flag[0] = n;
                }
                __syncthreads();
                const int nh = 2 * __builtin_amdgcn_readfirstlane(flag[0]);  // half pages

                // address of half page q (K or V) of this head in HBM
                auto half_src = [&](const unsigned char* base, int q) {
                    const int4 e = plist[q >> 1];
                    const int unit = __builtin_amdgcn_readfirstlane(e.x);
                    const int rec = __builtin_amdgcn_readfirstlane((q & 1) ? e.w : e.z);
                    return KvSrc{base + (int64_t)unit * a.kv_stride * esz + head_off +
                                     (q & 1) * 64 * rs,
                                 rec};
                };
                if (nh > 0) {
                    f32x16 s[2];
                    u32x4 p[4];  // P^T of the last softmax item, as PV B operands
                    {  // K_0 by the whole workgroup before the first slot
                        PageRegs<DT, 512, 64> pr0;
                        page_load<DT, 512, 64>(pr0, half_src(kbase, 0), rs, tid);
                        store_k<DT, 512, 64>(pr0, kst, tid);
                    }
                    __syncthreads();
                    // Each group's share of the KV stream is loaded one softmax item ahead of its
                    // store, so the load latency spans an MFMA and a softmax item. Softmax item k
                    // stores V_k (group 0) or K_{k+2} (group 1) into buffer k % 2. Past the end of
                    // the stream the index is clamped: group 1 then rewrites a K half that nobody
                    // reads again, and the last load is simply not stored.
                    auto move_half = [&](int k) { return min(grp == 0 ? k : k + 2, nh - 1); };
                    PageRegs<DT, 256, 64> pr;  // the group's next move, in flight
                    if (grp == 1) {            // group 1 starts one slot late: K_1 moves meanwhile
                        PageRegs<DT, 256, 64> pr1;
                        page_load<DT, 256, 64>(pr1, half_src(kbase, 1), rs, tg);
                        page_load<DT, 256, 64>(pr, half_src(kbase, move_half(0)), rs, tg);
                        store_k<DT, 256, 64>(pr1, kst + KB, tg);
                        __syncthreads();
                    } else {
                        page_load<DT, 256, 64>(pr, half_src(vbase, move_half(0)), rs, tg);
                    }
                    // page-list entries for the next softmax item, read before its LDS stores are
                    // queued (a wait on the list read would otherwise also wait for the stores)
                    int jc_next = __builtin_amdgcn_readfirstlane(plist[0].y);
                    uint32_t umw[8];  // user-mask words of the next softmax item
                    const int4 m1 = plist[move_half(1) >> 1];
                    int mv_page = __builtin_amdgcn_readfirstlane(m1.x);
                    int mv_rec = __builtin_amdgcn_readfirstlane((move_half(1) & 1) ? m1.w : m1.z);
                    auto softmax_and_move = [&](int k) {
                        const int jc = jc_next;
                        if constexpr (P8) {  // fp8 V as it is (P·V on fp8 MFMA)
                            if (grp == 0)
                                store_v8<256, 64>(pr, vst + (k & 1) * VB, tg);
                            else
                                store_k<DT, 256, 64>(pr, kst + (k & 1) * KB, tg);
                        } else if constexpr (DT == kFP8) {  // V is widened to bf16 into LDS
                            if (grp == 0)
                                store_v<DT, 256, 64>(pr, vst + (k & 1) * VB, tg);
                            else
                                store_k<DT, 256, 64>(pr, kst + (k & 1) * KB, tg);
                        } else if constexpr (kSharedPitch) {  // one store for both groups
                            store_k<DT, 256, 64>(pr, grp == 0 ? vst + (k & 1) * VB : kst + (k & 1) * KB, tg);
                        } else {
                            if (grp == 0)
                                store_v<DT, 256, 64>(pr, vst + (k & 1) * VB, tg);
                            else
                                store_k<DT, 256, 64>(pr, kst + (k & 1) * KB, tg);
                        }
                        {
                            const int q = move_half(k + 1);
                            const KvSrc src{(grp == 0 ? vbase : kbase) +
                                                (int64_t)mv_page * a.kv_stride * esz + head_off +
                                                (q & 1) * 64 * rs,
                                            mv_rec};
                            page_load<DT, 256, 64>(pr, src, rs, tg);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        softmax_item32<DT, UM, false, P8>(a, s, p, colscale, trow, umw, jc >> 2,
                                                          k & 1, jc & 3, skv, off, lane, mrun,
                                                          lrun, o, pq);
                        pin_softmax(p, lrun);
                        __builtin_amdgcn_sched_barrier(0);
                        const int jn = plist[min(k + 1, nh - 1) >> 1].y;
                        const int qn = move_half(k + 2);
                        const int4 mn = plist[qn >> 1];
                        __syncthreads();
                        jc_next = __builtin_amdgcn_readfirstlane(jn);
                        mv_page = __builtin_amdgcn_readfirstlane(mn.x);
                        mv_rec = __builtin_amdgcn_readfirstlane((qn & 1) ? mn.w : mn.z);
                    };
                    if constexpr (UM) umask_words32(a, um, jc_next >> 2, 0, lane, umw);
                    mfma_item32<DT, true, false, P8>(kst, vst, qc, s, p, o, lane);
                    __syncthreads();
                    softmax_and_move(0);
                    for (int k = 1; k < nh; ++k) {
                        if constexpr (UM) umask_words32(a, um, jc_next >> 2, k & 1, lane, umw);
                        mfma_item32<DT, true, true, P8>(kst + (k & 1) * KB, vst + ((k - 1) & 1) * VB,
                                                        qc, s, p, o, lane);
                        __syncthreads();
                        softmax_and_move(k);
                    }
                    mfma_item32<DT, false, true, P8>(kst, vst + ((nh - 1) & 1) * VB, qc, s, p, o,
                                                     lane);
                    if (grp == 0) __syncthreads();
                }
                __syncthreads();  // LDS (stages, page list) is reused by the next task

                write_rows32<DT, OUT>(a, it, complete, 2 * w + (sa > 0 ? 0 : 1), row0, lane, trow, rvalid,
                                      mrun, lrun, o, 1.f / pq);
                if (!complete) {
                    int* list = (int*)smem;  // the stages are free until the next task
                    const int np = piece_arrive(a, w, u, st, a.nst, list);
                    if (np > 0)
                        merge_rows<OUT>(a, list, np, row_base, min(row_base + R, rows_exist), it.n2,
                                        t0, it.row0, it.sq);
                    __syncthreads();
                }
            }
            advance_unit(a, it);
        }
    });
}


// ---------------------------------------------------------------------------------------------
// The 256-row ping-pong kernel with K/V moved by LDS DMA (16-bit key/value): the moved half
// pages go from memory straight into LDS (buffer loads with the LDS destination), so the
// softmax wave neither stages them in registers nor spends its item storing them.
//
// LDS layout of a half page (64 rows of 256 B) written by 16 DMA instructions of 1 KB: DMA
// instruction i (0..15) holds logical rows i, i + 16, i + 32, i + 48 in four 256-byte slots at
// byte i * 1088 + 256 * (row / 16), and inside a slot physical 16-byte chunk p holds logical
// chunk p ^ (i >> 2). Rows four apart sit 64 bytes apart in bank position (the eight rows of a
// transposing V read cover every bank), and sixteen consecutive rows map one logical chunk to
// sixteen distinct bank groups (the K fragment reads); both read patterns are conflict-free.
// Four buffers per operand (power-of-two indexing keeps the fragment addresses cheap): the DMA
// of a half page is issued at least two slots before its first reader, into a buffer whose last
// reader finished two slots earlier, and every wave lets only its newest DMA batch stay in
// flight across a barrier.
// ---------------------------------------------------------------------------------------------
// Slot trace (diagnostic build, -DGBSA_SLOT_TRACE, libgbsa_slot_trace.so). The first unit of
// at least 12 pages that a workgroup of one of the ping-pong kernels (the two DMA kernels, the
// register-staged key-split kernel) meets (one per launch, claimed with an atomic) records, per
// wave, an s_memtime stamp (shader clock) at every item boundary of its loop: event codes 1
// softmax item start, 2 softmax item end, 3 before its barrier, 4 after it, 5 MFMA item start,
// 6 MFMA item end (loads waited for), 7 after its barrier; the register-staged key-split kernel
// adds 8 K stored (its load waited for) and 9 MFMA instructions issued (before the V store). In
// the normal build the marks compile to nothing.
constexpr int kTraceEvents = 1024;  // per wave
#ifdef GBSA_SLOT_TRACE
__device__ unsigned long long g_slot_trace[8 * kTraceEvents];
__device__ int g_slot_trace_claim;
struct SlotTrace {
    unsigned long long* p = nullptr;
    int ev = 0;
    __device__ void begin(bool on, int wave) {
        p = on ? g_slot_trace + wave * kTraceEvents : nullptr;
        ev = 0;
    }
    __device__ void mark(int code, int lane) {
        __builtin_amdgcn_sched_barrier(0);
        const unsigned long long t = __builtin_amdgcn_s_memtime();
        if (p != nullptr && lane == 0 && ev < kTraceEvents)
            p[ev] = ((unsigned long long)code << 56) | (t & ((1ull << 56) - 1));
        ev += p != nullptr ? 1 : 0;
        __builtin_amdgcn_sched_barrier(0);
    }
};
// one wave's lane 0, with the unit's visible page count: whether this unit is the traced one
__device__ __forceinline__ int slot_trace_claim(int pages) {
    return pages >= 12 && atomicCAS(&g_slot_trace_claim, 0, 1) == 0;
}
#else
struct SlotTrace {
    __device__ void begin(bool, int) {}
    __device__ void mark(int, int) {}
};
__device__ __forceinline__ int slot_trace_claim(int) { return 0; }
#endif

constexpr int kDmaStride = 1088;             // bytes between the DMA instructions of a half page
constexpr int kDmaHalf = 16 * kDmaStride;    // one half page

// DMA instruction i (0..15) of the half page behind buffer resource r into the half-page buffer
// dst. No destination register: the data goes to LDS; completion is awaited with vmcnt. An
// instruction that reads M0 for an LDS DMA needs one wait state after the M0 write (the
// compiler keeps that distance for its own buffer-to-LDS loads), hence the nop.
__device__ __forceinline__ void dma_one(rsrc_t r, int rs, unsigned char* dst, int i, int lane) {
    const int row = i + 16 * (lane >> 4);
    const int voff = row * rs + 16 * ((lane & 15) ^ (i >> 2));
    const uint32_t m0 = (uint32_t)(uintptr_t)(GBSA_LDS unsigned char*)(dst + i * kDmaStride);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "memory", "m0");
}
// DMA instructions [i0, i0 + n) of half page `src` into the half-page buffer `dst`.
__device__ __forceinline__ void dma_half16(const KvSrc& src, int rs, unsigned char* dst, int i0,
                                           int n, int lane) {
    const rsrc_t r = make_rsrc(src.p, src.records);
#pragma unroll
    for (int x = 0; x < n; ++x) dma_one(r, rs, dst, i0 + x, lane);
}

// Page-list entry of the DMA kernel: byte offset of the page's head slice from the K (or V)
// base, and the readable bytes of its two half pages (0 past the visible keys).
__device__ __forceinline__ KvSrc page_half(const unsigned char* base, u32x4 e, int half, int rs) {
    const uint64_t off = (uint64_t)__builtin_amdgcn_readfirstlane(e[0]) |
                         ((uint64_t)__builtin_amdgcn_readfirstlane(e[1]) << 32);
    const int rec = (int)__builtin_amdgcn_readfirstlane(half ? e[3] : e[2]);
    return KvSrc{base + off + half * 64 * rs, rec};
}

// One wave's share (four DMA instructions) of moving a half page, issued from inside an MFMA
// item: the page-list entry is read at step 0 and the instructions go out at steps 3, 5, 7, 9,
// where the wave waits for the matrix pipe anyway.
struct ItemMove {
    const u32x4* entry;  // LDS page-list entry of the half page
    int half;           // which half of the page
    const unsigned char* base;
    unsigned char* dst;  // half-page buffer
    int i0;              // first of the wave's four DMA instructions
};

// Waits until at most n of this wave's vector-memory loads are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// MFMA item of the 256-row kernel on the DMA layout (as mfma_item32, 16-bit types), optionally
// issuing one half-page move (MOVE) between its MFMAs.
template <int DT, bool qk, bool pv, bool MOVE = false>
__device__ __forceinline__ void mfma_item32d(const unsigned char* ks, const unsigned char* vs,
                                             const QCol32& qc, f32x16 (&s)[2],
                                             const u32x4 (&p)[4], f32x16 (&o)[4], int lane,
                                             const ItemMove& mv = ItemMove{}, int rs = 0) {
    constexpr int QS = qk ? 8 : 0;
    constexpr int VS = pv ? 8 : 0;
    constexpr int PC = QS + VS, NS = 2 * PC, D = kPipeDepth;
    const int h2 = lane >> 5, m = (lane & 15) >> 2, g = (lane >> 4) & 1, cc = lane & 3;
    // K: row t * 32 + (lane & 31) -> instruction lane & 15, slot 2 t + g; chunk 2 j + h2
    const unsigned char* kl = ks + (lane & 15) * kDmaStride + g * 256;
    const unsigned char* ka0 = kl + 16 * (h2 ^ m);        // even j
    const unsigned char* ka1 = kl + 16 * ((2 + h2) ^ m);  // odd j
    // V^T: rows 4 h + (lane & 15) / 4 (+ 8), chunk 2 g + cc / 2, 8-byte half cc & 1
    const int i0 = 4 * h2 + m;
    const unsigned char* vb0 = vs + i0 * kDmaStride + 16 * ((2 * g + (cc >> 1)) ^ h2) + 8 * (cc & 1);
    const unsigned char* vb1 =
        vs + (i0 + 8) * kDmaStride + 16 * ((2 * g + (cc >> 1)) ^ (h2 + 2)) + 8 * (cc & 1);
    const f32x16 zero = {};
    auto load = [&](int st) {
        Frag f;
        const int t = st / PC, j = st % PC;
        if (j < QS) {
            f.a = *(const u32x4*)(((j & 1) ? ka1 : ka0) + t * 512 + 64 * (j >> 1));
        } else {
            const int v = j - QS, a2 = v >> 2, dt = v & 3;
            const int o2 = (2 * t + a2) * 256 + dt * 64;
            const u32x2 v0 = lds_read_tr16(vb0 + o2);
            const u32x2 v1 = lds_read_tr16(vb1 + o2);
            f.a = (u32x4){v0[0], v0[1], v1[0], v1[1]};
        }
        return f;
    };
    auto compute = [&](int st, const Frag& f) {
        const int t = st / PC, j = st % PC;
        if (j < QS) {
            s[t] = mfma_32x32x16<DT>(f.a, qc.q[j], j == 0 ? zero : s[t]);
        } else {
            const int v = j - QS, a2 = v >> 2, dt = v & 3;
            o[dt] = mfma_32x32x16<DT>(f.a, p[2 * t + a2], o[dt]);
        }
    };
    static_assert(!MOVE || NS >= 10, "the move needs ten steps");
    u32x4 ent;
    rsrc_t mr;
    Frag fr[D];
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (i < NS) fr[i] = load(i);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const Frag f = fr[st % D];
        if (st + D < NS) fr[st % D] = load(st + D);
        if constexpr (MOVE) {
            if (st == 0) ent = *(const GBSA_LDS u32x4*)mv.entry;
            if (st == 2) {
                const KvSrc src = page_half(mv.base, ent, mv.half, rs);
                mr = make_rsrc(src.p, src.records);
            }
            if (st >= 3 && st <= 9 && (st & 1)) dma_one(mr, rs, mv.dst, mv.i0 + (st - 3) / 2, lane);
        }
        compute(st, f);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int DT, int OUT, int LAYOUT, bool UM, bool HS = false>
__global__ __launch_bounds__(512, 1) void fwd_prefill_pp32d_kernel(FwdArgs a) {
    static_assert(DT != kFP8, "the DMA layout holds 16-bit rows");
    constexpr int R = 256;
    constexpr int esz = 2;
    // [K buffers 0..3][V buffers 0..3], one half page each
    __shared__ __attribute__((aligned(16))) unsigned char smem[8 * kDmaHalf];
    // per visible page: byte offset of this head's slice, readable bytes of its two halves
    __shared__ u32x4 plist[256];
    __shared__ int jlist[256];  // per visible page: block index * 4 + mask class
    __shared__ int flag[2];  // visible pages of the unit; slot trace on
    static_assert(sizeof(smem) >= kPieceListBytes, "the split merge borrows the stages");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int gw = wave & 3;  // wave within its group
    if (!header_ok(a)) {
        refuse(a);
        return;
    }
    const int U = a.meta[3];
    __shared__ int task_word[2];
    run_tasks<!UM>(a, U, task_word, [&](const FwdArgs& a, const Task& tk) {
        const int w = tk.w, st = tk.st;
        const Bound b0 = tk.b0, b1 = tk.b1;
        if (!bound_less(b0, b1) || b0.u >= U) return;
        UnitIter it = locate_unit(a, b0.u);
        if (it.b < 0) return;

        const int rs = a.N2 * 128 * esz;
        const unsigned char* kbase = (const unsigned char*)a.k;
        const unsigned char* vbase = (const unsigned char*)a.v;
        unsigned char* const kst = smem;
        unsigned char* const vst = smem + 4 * kDmaHalf;

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
            const int row_base = st * R;
            if (row_base < rows_exist) {
                const KvSeq kv = kv_seq<LAYOUT>(a, it.b);
                const int skv = kv.len;
                const int off = diag_off(a, skv, it.sq);
                const int row0 = row_base + wave * 32;
                QCol32 qc;
                float colscale, mrun = kNegInf, lrun = 0.f;
                int trow;
                bool rvalid;
                load_q32<DT>(a, it, t0, rows_exist, row0, lane, qc, colscale, trow, rvalid);
                const UMaskRow um =
                    UM ? umask_row(a, it.b, trow, rvalid) : UMaskRow{make_rsrc(nullptr, 0), -1};
                f32x16 o[4];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] = (f32x16){};
                const int t_lo = t0 + row_base / a.G;
                const int t_hi = t0 + (min(row_base + R, rows_exist) - 1) / a.G;
                const int32_t* sel = a.idx + ((int64_t)it.n2 * a.tqb + g) * a.topK;
                const int64_t head_off = (int64_t)it.n2 * 128 * esz;

                if (wave == 0) {
                    int n = 0;
                    for (int c0 = sa; c0 < se; c0 += 64) {
                        int jl = -1, pl = 0, cl = 0;
                        if (c0 + lane < se) {
                            jl = sel[c0 + lane];
                            if (jl >= 0) {
                                cl = block_class(a, (int64_t)jl * 128, skv, off, t_lo, t_hi);
                                if (cl != 0) pl = kv.unit<LAYOUT>(jl);
                            }
                        }
                        const uint64_t mm = __ballot(cl != 0);
                        if (cl != 0) {
                            const int pos = n + __builtin_amdgcn_mbcnt_hi(
                                                    (uint32_t)(mm >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0));
                            const uint64_t po = (uint64_t)((int64_t)pl * a.kv_stride * esz + head_off);
                            plist[pos] = (u32x4){(uint32_t)po, (uint32_t)(po >> 32),
                                                 (uint32_t)kv_records(rs, skv - 128 * jl),
                                                 (uint32_t)kv_records(rs, skv - 128 * jl - 64)};
                            jlist[pos] = jl * 4 + cl;
                        }
                        n += __builtin_popcountll(mm);
                    }
                    if (lane == 0) {
                        flag[0] = n;
                        flag[1] = slot_trace_claim(n);
                    }
                }
                __syncthreads();
                const int nh = 2 * __builtin_amdgcn_readfirstlane(flag[0]);  // half pages
                SlotTrace tr;
                tr.begin(__builtin_amdgcn_readfirstlane(flag[1]) != 0, wave);

                // half page q (clamped into the stream) of K or V of this head
                auto half_src = [&](const unsigned char* base, int q) {
                    q = min(q, nh - 1);
                    return page_half(base, plist[q >> 1], q & 1, rs);
                };
                if (nh > 0) {
                    f32x16 s[2];
                    u32x4 p[4];
                    if constexpr (!UM) {
                        // Intervals, one barrier per item pair. In interval i both groups run
                        // MFMA item i (QK^T of K_i, PV of V_{i-1}): group 0 before its softmax
                        // item i, group 1 after its softmax item i - 1, so that on each SIMD one
                        // wave issues MFMAs while its partner exponentiates, twice per interval,
                        // and neither waits at a barrier between the two. Moves of interval i,
                        // from inside the MFMA item: group 0 V_{i+1}, group 1 K_{i+2} (clamped
                        // into the stream, so every MFMA item with QK^T issues four DMA
                        // instructions per wave). Before the barrier that ends an interval a
                        // wave waits for all but its newest batch: a move of interval i is in
                        // LDS from interval i + 2, its first reader, and replaces a half page
                        // whose last reader ran in interval i - 2. Before the first interval:
                        // K_0, K_1 and V_0 by all eight waves.
                        dma_half16(half_src(kbase, 0), rs, kst, 2 * wave, 2, lane);
                        dma_half16(half_src(kbase, 1), rs, kst + kDmaHalf, 2 * wave, 2, lane);
                        dma_half16(half_src(vbase, 0), rs, vst, 2 * wave, 2, lane);
                        wait_vm<0>();
                        __syncthreads();
                        auto imove = [&](int i) {
                            const int q = min(grp == 0 ? i + 1 : i + 2, nh - 1);
                            return ItemMove{plist + (q >> 1), q & 1, grp == 0 ? vbase : kbase,
                                            grp == 0 ? vst + ((i + 1) & 3) * kDmaHalf
                                                     : kst + ((i + 2) & 3) * kDmaHalf,
                                            4 * gw};
                        };
                        const uint32_t umw0[8] = {};  // (no user mask)
                        int jc_next = __builtin_amdgcn_readfirstlane(jlist[0]);
                        auto softmax = [&](int k) {
                            const int jc = jc_next;
                            __builtin_amdgcn_sched_barrier(0);
                            tr.mark(1, lane);
                            softmax_item32<DT, false, HS>(a, s, p, colscale, trow, umw0, jc >> 2,
                                                          k & 1, jc & 3, skv, off, lane, mrun, lrun,
                                                          o);
                            pin_softmax(p, lrun);
                            __builtin_amdgcn_sched_barrier(0);
                            tr.mark(2, lane);
                        };
                        // knext: the half page of this wave's next softmax item
                        auto end_interval = [&](int knext) {
                            const int jn = jlist[min(knext, nh - 1) >> 1];
                            wait_vm<4>();  // all but this interval's batch are in LDS
                            tr.mark(3, lane);
                            __syncthreads();
                            tr.mark(4, lane);
                            jc_next = __builtin_amdgcn_readfirstlane(jn);
                        };
                        tr.mark(5, lane);
                        __builtin_amdgcn_s_setprio(3);
                        mfma_item32d<DT, true, false, true>(kst, vst, qc, s, p, o, lane, imove(0), rs);
                        __builtin_amdgcn_s_setprio(0);
                        tr.mark(6, lane);
                        if (grp == 0) softmax(0);
                        end_interval(grp == 0 ? 1 : 0);
                        for (int i = 1; i < nh; ++i) {
                            if (grp == 1) softmax(i - 1);
                            tr.mark(5, lane);
                            __builtin_amdgcn_s_setprio(3);
                            mfma_item32d<DT, true, true, true>(kst + (i & 3) * kDmaHalf,
                                                               vst + ((i - 1) & 3) * kDmaHalf, qc, s,
                                                               p, o, lane, imove(i), rs);
                            __builtin_amdgcn_s_setprio(0);
                            tr.mark(6, lane);
                            if (grp == 0) softmax(i);
                            end_interval(grp == 0 ? i + 1 : i);
                        }
                        if (grp == 1) softmax(nh - 1);
                        __builtin_amdgcn_s_setprio(3);
                        mfma_item32d<DT, false, true>(kst, vst + ((nh - 1) & 3) * kDmaHalf, qc, s, p,
                                                      o, lane);
                        __builtin_amdgcn_s_setprio(0);
                        wait_vm<0>();  // nothing may land in LDS after the task
                    } else {
                    // Readers: MFMA item k reads K_k (K buffer k % 4) and V_{k-1} (V buffer
                    // (k - 1) % 4); group 0 runs it in slot 2 k, group 1 in slot 2 k + 1.
                    // Writers (each group's four waves issue four DMA instructions each): group 0
                    // moves V_{k+1}, group 1 K_{k+3}, during their MFMA item k (without a user
                    // mask: the wave has issue slots to spare between its MFMAs) or else at the
                    // end of their softmax item k, a slot later. Either way a move lands in a
                    // buffer whose last reader is past a barrier, and a wave lets only its newest
                    // batch stay in flight across a barrier, so every batch has two slots to land
                    // before its first reader. (With a user mask, the compiler's own vmcnt waits
                    // for the mask words would also wait for DMA issued after them.)
                    // Before the first slot: K_0 by all eight waves, K_1 and V_0 by group 1
                    // and 0, and K_2 by group 1 in its first slot.
                    // Issue priority: the two waves on a SIMD compete for instruction issue, and
                    // the older one wins ties. Unless its MFMAs go out as soon as the matrix pipe
                    // frees, the pipe idles while the softmax wave issues; so the MFMA item runs
                    // at raised priority and the softmax item takes the remaining issue cycles
                    // (without the raise, the slots where the younger group does its MFMA item
                    // ran about 40 % longer).
                    dma_half16(half_src(kbase, 0), rs, kst, 2 * wave, 2, lane);
                    if (grp == 1)
                        dma_half16(half_src(kbase, 1), rs, kst + kDmaHalf, 4 * gw, 4, lane);
                    else
                        dma_half16(half_src(vbase, 0), rs, vst, 4 * gw, 4, lane);
                    wait_vm<0>();
                    __syncthreads();
                    if (grp == 1) {  // group 1 starts one slot late; its K_2 move goes out now
                        dma_half16(half_src(kbase, 2), rs, kst + 2 * kDmaHalf, 4 * gw, 4, lane);
                        __syncthreads();
                    }
                    int jc_next = __builtin_amdgcn_readfirstlane(jlist[0]);
                    constexpr bool kItemMove = !UM;
                    auto raise = [] { if constexpr (kItemMove) __builtin_amdgcn_s_setprio(3); };
                    auto lower = [] { if constexpr (kItemMove) __builtin_amdgcn_s_setprio(0); };
                    auto move_of = [&](int k) {
                        const int q = min(grp == 0 ? k + 1 : k + 3, nh - 1);
                        return ItemMove{plist + (q >> 1), q & 1, grp == 0 ? vbase : kbase,
                                        grp == 0 ? vst + ((k + 1) & 3) * kDmaHalf
                                                 : kst + ((k + 3) & 3) * kDmaHalf,
                                        4 * gw};
                    };
                    uint32_t umw[8];  // user-mask words of the next softmax item
                    auto softmax_and_move = [&](int k) {
                        const int jc = jc_next;
                        __builtin_amdgcn_sched_barrier(0);
                        tr.mark(1, lane);
                        softmax_item32<DT, UM, HS>(a, s, p, colscale, trow, umw, jc >> 2, k & 1, jc & 3,
                                               skv, off, lane, mrun, lrun, o);
                        pin_softmax(p, lrun);
                        __builtin_amdgcn_sched_barrier(0);
                        tr.mark(2, lane);
                        if constexpr (!kItemMove) {  // group 0 V_{k+1}, group 1 K_{k+3}
                            if (grp == 0)
                                dma_half16(half_src(vbase, k + 1), rs,
                                           vst + ((k + 1) & 3) * kDmaHalf, 4 * gw, 4, lane);
                            else
                                dma_half16(half_src(kbase, k + 3), rs,
                                           kst + ((k + 3) & 3) * kDmaHalf, 4 * gw, 4, lane);
                        }
                        const int jn = jlist[min(k + 1, nh - 1) >> 1];
                        wait_vm<4>();  // all but this item's batch are in LDS
                        tr.mark(3, lane);
                        __syncthreads();
                        tr.mark(4, lane);
                        jc_next = __builtin_amdgcn_readfirstlane(jn);
                    };
                    if constexpr (UM) umask_words32(a, um, jc_next >> 2, 0, lane, umw);
                    raise();
                    mfma_item32d<DT, true, false, kItemMove>(kst, vst, qc, s, p, o, lane, move_of(0),
                                                             rs);
                    lower();
                    wait_vm<UM ? 12 : 4>();
                    __syncthreads();
                    softmax_and_move(0);
                    for (int k = 1; k < nh; ++k) {
                        if constexpr (UM) umask_words32(a, um, jc_next >> 2, k & 1, lane, umw);
                        tr.mark(5, lane);
                        raise();
                        mfma_item32d<DT, true, true, kItemMove>(kst + (k & 3) * kDmaHalf,
                                                                vst + ((k - 1) & 3) * kDmaHalf, qc, s,
                                                                p, o, lane, move_of(k), rs);
                        lower();
                        wait_vm<UM ? 12 : 4>();
                        tr.mark(6, lane);
                        __syncthreads();
                        tr.mark(7, lane);
                        softmax_and_move(k);
                    }
                    raise();
                    mfma_item32d<DT, false, true>(kst, vst + ((nh - 1) & 3) * kDmaHalf, qc, s, p, o,
                                                  lane);
                    lower();
                    wait_vm<0>();  // nothing may land in LDS after the task
                    if (grp == 0) __syncthreads();
                    }
                }
                __syncthreads();

                write_rows32<DT, OUT>(a, it, complete, 2 * w + (sa > 0 ? 0 : 1), row0, lane, trow,
                                      rvalid, mrun, lrun, o);
                if (!complete) {
                    int* list = (int*)smem;
                    const int np = piece_arrive(a, w, u, st, a.nst, list);
                    if (np > 0)
                        merge_rows<OUT>(a, list, np, row_base, min(row_base + R, rows_exist), it.n2,
                                        t0, it.row0, it.sq);
                    __syncthreads();
                }
            }
            advance_unit(a, it);
        }
    });
}


// ---------------------------------------------------------------------------------------------
// Units of 65-256 rows: 128-row subtiles, two-group ping-pong with the keys split.
//
// Both groups hold the same 128 query rows (4 waves x 32 rows). Group 0 takes the first half
// (64 tokens) of every visible page, group 1 the second half, one barrier slot behind, with the
// same MFMA / softmax item sequence as above. Global half page q = 2k + g is group g's item k;
// in slot s the MFMA item reads K_s and V_{s-2}, which always sit in the LDS buffers of the
// group that owns them (K and V buffer g for group g). Moves: group g's softmax item k brings
// K of its next half page (2k + 2 + g) into its own K buffer; its MFMA item k brings V of the
// half page the partner has just exponentiated (2k + g - 1) into the partner's V buffer. Each
// buffer is rewritten one slot after its last reader. At the end the two groups' online-softmax
// states of each row are merged through LDS (FA article, "three steps": partial results over
// disjoint key sets combine exactly after rescaling to the common max).
// ---------------------------------------------------------------------------------------------
// The 128-row kernel (schedule above) on 32x32 tiles: each wave's 32 query rows are one
// 32-column tile.
template <int DT, int OUT, int LAYOUT, bool UM, bool HS = false, bool P8 = false>
__global__ __launch_bounds__(512, 1) void fwd_prefill_ks32_kernel(FwdArgs a) {
    constexpr int R = 128;
    constexpr int esz = (DT == kFP8) ? 1 : 2;
    constexpr int KB = HalfStage<DT, P8>::k_bytes, VB = HalfStage<DT, P8>::v_bytes;
    constexpr int kStateBytes = 4 * (64 * 64 * 4 + 64 * 16);  // group 1's O, m, l for the merge
    constexpr int kLds = (2 * KB + 2 * VB > kStateBytes) ? 2 * KB + 2 * VB : kStateBytes;
    // [K buffer 0][K buffer 1][V buffer 0][V buffer 1]; reused for the final merge
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
    __shared__ int4 plist[256];  // as in the row-split kernel
    __shared__ int flag[2];
    static_assert(sizeof(smem) >= kPieceListBytes, "the split merge borrows the stages");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;  // waves w and w + 4 share a SIMD and the same query rows
    const int tg = tid & 255;
    if (!header_ok(a)) {
        refuse(a);
        return;
    }
    const int U = a.meta[3];
    __shared__ int task_word[2];
    run_tasks<!UM>(a, U, task_word, [&](const FwdArgs& a, const Task& tk) {
        const int w = tk.w, st = tk.st;
        const Bound b0 = tk.b0, b1 = tk.b1;
        if (!bound_less(b0, b1) || b0.u >= U) return;
        UnitIter it = locate_unit(a, b0.u);
        if (it.b < 0) return;

        const int rs = a.N2 * 128 * esz;
        const unsigned char* kbase = (const unsigned char*)a.k;
        const unsigned char* vbase = (const unsigned char*)a.v;
        unsigned char* const kst = smem;
        unsigned char* const vst = smem + 2 * KB;

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
            const int row_base = st * R;
            if (row_base < rows_exist) {
                const KvSeq kv = kv_seq<LAYOUT>(a, it.b);
                const int skv = kv.len;
                const int off = diag_off(a, skv, it.sq);
                const int row0 = row_base + (wave & 3) * 32;
                QCol32 qc;
                float colscale, mrun = kNegInf, lrun = 0.f;
                int trow;
                bool rvalid;
                load_q32<DT>(a, it, t0, rows_exist, row0, lane, qc, colscale, trow, rvalid);
                const float pq = P8 ? p_quant(a, it, row0, rows_exist, lane) : 1.f;
                const UMaskRow um =
                    UM ? umask_row(a, it.b, trow, rvalid) : UMaskRow{make_rsrc(nullptr, 0), -1};
                f32x16 o[4];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] = (f32x16){};
                const int t_lo = t0 + row_base / a.G;
                const int t_hi = t0 + (min(row_base + R, rows_exist) - 1) / a.G;
                const int32_t* sel = a.idx + ((int64_t)it.n2 * a.tqb + g) * a.topK;
                const int64_t head_off = (int64_t)it.n2 * 128 * esz;

                if (wave == 0) {
                    int n = 0;
                    for (int c0 = sa; c0 < se; c0 += 64) {
                        int jl = -1, pl = 0, cl = 0;
                        if (c0 + lane < se) {
                            jl = sel[c0 + lane];
                            if (jl >= 0) {
                                cl = block_class(a, (int64_t)jl * 128, skv, off, t_lo, t_hi);
                                if (cl != 0) pl = kv.unit<LAYOUT>(jl);
                            }
                        }
                        const uint64_t m = __ballot(cl != 0);
                        if (cl != 0) {
                            const int pos = n + __builtin_amdgcn_mbcnt_hi(
                                                    (uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                            plist[pos] = make_int4(pl, jl * 4 + cl,
                                                   kv_records(rs, skv - 128 * jl),
                                                   kv_records(rs, skv - 128 * jl - 64));
                        }
                        n += __builtin_popcountll(m);
                    }
                    if (lane == 0) {
                        flag[0] = n;
                        flag[1] = slot_trace_claim(n);
                    }
                }
                __syncthreads();
                const int n = __builtin_amdgcn_readfirstlane(flag[0]);  // items per group
                SlotTrace tr;
                tr.begin(__builtin_amdgcn_readfirstlane(flag[1]) != 0, wave);
                const int nh = 2 * n;                                   // half pages

                // address of half page q (K or V) of this head in HBM; q is clamped into the stream
                auto half_src = [&](const unsigned char* base, int q) {
                    q = min(max(q, 0), nh - 1);
                    const int4 e = plist[q >> 1];
                    const int unit = __builtin_amdgcn_readfirstlane(e.x);
                    const int rec = __builtin_amdgcn_readfirstlane((q & 1) ? e.w : e.z);
                    return KvSrc{base + (int64_t)unit * a.kv_stride * esz + head_off +
                                     (q & 1) * 64 * rs,
                                 rec};
                };
                if (n > 0) {
                    f32x16 s[2];
                    u32x4 p[4];
                    {  // K_0 by the whole workgroup before the first slot
                        PageRegs<DT, 512, 64> pr0;
                        page_load<DT, 512, 64>(pr0, half_src(kbase, 0), rs, tid);
                        store_k<DT, 512, 64>(pr0, kst, tid);
                    }
                    __syncthreads();
                    if (grp == 1) {  // group 1 starts one slot late: K_1 moves meanwhile
                        PageRegs<DT, 256, 64> pr1;
                        page_load<DT, 256, 64>(pr1, half_src(kbase, 1), rs, tg);
                        store_k<DT, 256, 64>(pr1, kst + KB, tg);
                        __syncthreads();
                    }
                    unsigned char* const my_k = kst + grp * KB;
                    unsigned char* const my_v = vst + grp * VB;
                    unsigned char* const other_v = vst + (grp ^ 1) * VB;
                    // V of the half page the partner has just exponentiated, into its V buffer
                    auto v_move_store = [&](const PageRegs<DT, 256, 64>& pr) {
                        if constexpr (P8)
                            store_v8<256, 64>(pr, other_v, tg);  // fp8 V as it is
                        else if constexpr (DT == kFP8 || !kSharedPitch)
                            store_v<DT, 256, 64>(pr, other_v, tg);
                        else
                            store_k<DT, 256, 64>(pr, other_v, tg);  // same row pitch as K
                    };
                    uint32_t umw[8];  // user-mask words of the next softmax item
                    auto mask_words = [&](int k) {
                        if constexpr (UM)
                            umask_words32(a, um, __builtin_amdgcn_readfirstlane(plist[k].y) >> 2, grp,
                                          lane, umw);
                    };
                    auto softmax_and_move = [&](int k) {
                        const int jc = __builtin_amdgcn_readfirstlane(plist[k].y);
                        tr.mark(1, lane);
                        PageRegs<DT, 256, 64> pr;
                        page_load<DT, 256, 64>(pr, half_src(kbase, 2 * k + 2 + grp), rs, tg);
                        __builtin_amdgcn_sched_barrier(0);
                        softmax_item32<DT, UM, HS, P8>(a, s, p, colscale, trow, umw, jc >> 2, grp,
                                                       jc & 3, skv, off, lane, mrun, lrun, o, pq);
                        pin_softmax(p, lrun);
                        __builtin_amdgcn_sched_barrier(0);
                        tr.mark(2, lane);
                        store_k<DT, 256, 64>(pr, my_k, tg);
                        tr.mark(8, lane);
                        __syncthreads();
                        tr.mark(4, lane);
                    };
                    {
                        PageRegs<DT, 256, 64> pr;
                        page_load<DT, 256, 64>(pr, half_src(vbase, grp - 1), rs, tg);
                        mask_words(0);
                        __builtin_amdgcn_sched_barrier(0);
                        mfma_item32<DT, true, false, P8>(my_k, my_v, qc, s, p, o, lane);
                        __builtin_amdgcn_sched_barrier(0);
                        v_move_store(pr);
                    }
                    __syncthreads();
                    softmax_and_move(0);
                    for (int k = 1; k < n; ++k) {
                        tr.mark(5, lane);
                        PageRegs<DT, 256, 64> pr;
                        page_load<DT, 256, 64>(pr, half_src(vbase, 2 * k + grp - 1), rs, tg);
                        mask_words(k);
                        __builtin_amdgcn_sched_barrier(0);
                        mfma_item32<DT, true, true, P8>(my_k, my_v, qc, s, p, o, lane);
                        __builtin_amdgcn_sched_barrier(0);
                        tr.mark(9, lane);
                        v_move_store(pr);
                        tr.mark(6, lane);
                        __syncthreads();
                        tr.mark(7, lane);
                        softmax_and_move(k);
                    }
                    {
                        PageRegs<DT, 256, 64> pr;
                        page_load<DT, 256, 64>(pr, half_src(vbase, 2 * n + grp - 1), rs, tg);
                        __builtin_amdgcn_sched_barrier(0);
                        mfma_item32<DT, false, true, P8>(my_k, my_v, qc, s, p, o, lane);
                        __builtin_amdgcn_sched_barrier(0);
                        v_move_store(pr);
                    }
                    if (grp == 0) __syncthreads();
                }
                __syncthreads();  // stages are free: group 1 hands its row states to group 0

                if (grp == 1) {
                    f32x4* so = (f32x4*)(smem + (wave - 4) * (64 * 64 * 4 + 64 * 16));
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4)
                            so[(dt * 4 + g4) * 64 + lane] = (f32x4){o[dt][4 * g4], o[dt][4 * g4 + 1],
                                                                   o[dt][4 * g4 + 2], o[dt][4 * g4 + 3]};
                    so[16 * 64 + lane] = (f32x4){mrun, lrun, 0.f, 0.f};
                }
                __syncthreads();
                if (grp == 0) {
                    const f32x4* so = (const f32x4*)(smem + wave * (64 * 64 * 4 + 64 * 16));
                    const f32x4 ml = so[16 * 64 + lane];
                    const float m = fmaxf(mrun, ml[0]);
                    const float a0 = (m == kNegInf) ? 0.f : fast_exp2(mrun - m);
                    const float a1 = (m == kNegInf) ? 0.f : fast_exp2(ml[0] - m);
                    mrun = m;
                    lrun = lrun * a0 + ml[1] * a1;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const f32x4 x = so[(dt * 4 + g4) * 64 + lane];
#pragma unroll
                            for (int e = 0; e < 4; ++e) o[dt][4 * g4 + e] = o[dt][4 * g4 + e] * a0 + x[e] * a1;
                        }
                    write_rows32<DT, OUT>(a, it, complete, 2 * w + (sa > 0 ? 0 : 1), row0, lane, trow,
                                          rvalid, mrun, lrun, o, 1.f / pq);
                }
                __syncthreads();  // LDS is reused by the next task
                if (!complete) {
                    int* list = (int*)smem;  // the stages are free until the next task
                    const int np = piece_arrive(a, w, u, st, a.nst, list);
                    if (np > 0)
                        merge_rows<OUT>(a, list, np, row_base, min(row_base + R, rows_exist), it.n2,
                                        t0, it.row0, it.sq);
                    __syncthreads();
                }
            }
            advance_unit(a, it);
        }
    });
}

// ---------------------------------------------------------------------------------------------
// The 128-row key-split kernel with K and V moved by LDS DMA (fp8 key/value, no user mask). The
// items of fwd_prefill_ks32_kernel (group g takes half page g of every page: half page q is
// group q % 2's item q / 2), with the half pages reaching LDS as e4m3 rows by `buffer_load ...
// lds` issued from inside the MFMA items, so no load has to land within the item that issues it,
// and one barrier per item pair (the schedule is with the kernel). MFMA item k of group g reads
// K_q and V_{q-2} (q = 2 k + g) and moves K_{q+4} and V_{q+2} (clamped into the stream, so every
// item issues the same four instructions per wave), each wave two DMA instructions of each; both
// rings hold eight half pages (indexed q % 8). V^T comes from the e4m3 rows with the 8-bit
// transposing read and is widened exactly to bf16 in registers right before its MFMA; with a P
// quantisation scale (P8) P·V runs on fp8 MFMA straight from the e4m3 rows.
//
// LDS layout of an fp8 half page (64 rows of 128 B): DMA instruction i (0..7) writes rows
// 8 i .. 8 i + 7 as 1 KB at byte 1024 i; 16-byte chunk c of row r (head dims 16 c ..) sits at
// position c ^ sw8(r) of the row, sw8(r) = f((r / 2) % 8) with f(x) = 4 (x1 ^ x2) + 2 x0 + x2
// (x2 x1 x0 the bits of x): a permutation of 0..7 whose two high bits differ across x = 0..3,
// 4..7, {0, 1, 4, 5} and {2, 3, 6, 7}. All three read patterns are then free of bank conflicts
// (checked for every row and chunk): the K fragment reads (16 consecutive rows, one chunk) cover
// the 16 bank groups of 256 B once, and so do the 8-bit transposing V reads of a half wave,
// rows b .. b + 3 and b + 8 .. b + 11 (b a multiple of 4; bf16 P) or rows 8 m .. 8 m + 7 (fp8
// P), two adjacent chunks each.
// ---------------------------------------------------------------------------------------------
constexpr int kHalf8 = 64 * 128;  // one fp8 half page

__device__ __forceinline__ int sw8(int r) {
    const int x = (r >> 1) & 7, x0 = x & 1, x1 = (x >> 1) & 1, x2 = x >> 2;
    return ((x1 ^ x2) << 2) | (x0 << 1) | x2;
}

// DMA instruction i (0..7) of the fp8 half page behind buffer resource r into buffer dst.
__device__ __forceinline__ void dma8_one(rsrc_t r, int rs, unsigned char* dst, int i, int lane) {
    const int row = 8 * i + (lane >> 3);
    const int voff = row * rs + 16 * ((lane & 7) ^ sw8(row));
    const uint32_t m0 = (uint32_t)(uintptr_t)(GBSA_LDS unsigned char*)(dst + i * 1024);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "memory", "m0");
}

// The two half-page moves of one MFMA item (K_{s+4} and V_{s+2}), two DMA instructions each per
// wave.
struct ItemMove8 {
    const u32x4* kent;  // LDS page-list entries of the two half pages
    const u32x4* vent;
    unsigned char* kdst;  // their buffers
    unsigned char* vdst;
    int khalf, vhalf;  // which half of each page
    int i0;            // first of the wave's two DMA instructions of each move
};

// Both moves of an item at once (the first item, which has too few steps to spread them).
__device__ __forceinline__ void moves8_now(const ItemMove8& mv, const unsigned char* kbase,
                                           const unsigned char* vbase, int rs, int lane) {
    const KvSrc ks = page_half(kbase, *(const GBSA_LDS u32x4*)mv.kent, mv.khalf, rs);
    const rsrc_t rk = make_rsrc(ks.p, ks.records);
    dma8_one(rk, rs, mv.kdst, mv.i0, lane);
    dma8_one(rk, rs, mv.kdst, mv.i0 + 1, lane);
    const KvSrc vsrc = page_half(vbase, *(const GBSA_LDS u32x4*)mv.vent, mv.vhalf, rs);
    const rsrc_t rv = make_rsrc(vsrc.p, vsrc.records);
    dma8_one(rv, rs, mv.vdst, mv.i0, lane);
    dma8_one(rv, rs, mv.vdst, mv.i0 + 1, lane);
}

// MFMA item of the fp8 DMA kernel: QK^T of a half page on v_mfma_scale_f32_32x32x64_f8f6f4 (two
// steps per 32-key tile) and PV of the previous one on bf16 MFMA (eight steps per tile, V^T
// widened from e4m3 in registers), optionally issuing the item's two moves between its MFMAs
// (entries read at steps 0 and 1, DMA at steps 4, 6, 8, 10).
template <bool qk, bool pv, bool MOVE = false, bool P8 = false>
__device__ __forceinline__ void mfma_item32d8(const unsigned char* ks, const unsigned char* vs,
                                              const QCol32& qc, f32x16 (&s)[2],
                                              const u32x4 (&p)[4], f32x16 (&o)[4], int lane,
                                              const ItemMove8& mv = ItemMove8{},
                                              const unsigned char* kbase = nullptr,
                                              const unsigned char* vbase = nullptr, int rs = 0) {
    constexpr int QS = qk ? 2 : 0;
    // PV steps per 32-key tile: 2 chunks x 4 d tiles, or with fp8 P two d tiles of the whole
    // half page (64 keys) each
    constexpr int VS = pv ? (P8 ? 2 : 8) : 0;
    constexpr int PC = QS + VS, NS = 2 * PC, D = kPipeDepth;
    const int h2 = lane >> 5;
    // K: row 32 t + lane % 32, chunks 4 e + 2 h and + 1 (head dims 64 e + 32 h ..)
    const int kr = lane & 31, ksw = sw8(kr);
    const unsigned char* krow = ks + kr * 128;
    // V^T: block row (lane % 16) / 2 is key 4 h + m % 4 + 8 (m / 4) of each 16-key chunk, byte
    // half lane % 2 of chunk 2 dt + (lane / 16) % 2
    const int m = (lane & 15) >> 1, kv = 4 * h2 + (m & 3) + 8 * (m >> 2);
    const int vseg = (lane >> 4) & 1, vsw = sw8(kv);
    const unsigned char* vrow = vs + kv * 128 + 8 * (lane & 1);
    // fp8 P: read r (0..3) of d tile dt gives a lane keys 32 h + 8 r .. + 7 (block row
    // (lane % 16) / 2), byte half lane % 2 of chunk 2 dt + (lane / 16) % 2. The row's swizzle
    // sw8(32 h + 8 r + m) depends on r only through r % 2: 4 ((m / 4) % 2) + 2 ((m / 2) % 2) for
    // even r, that ^ 5 for odd r.
    const unsigned char* v8row = vs + (32 * h2 + m) * 128 + 8 * (lane & 1);
    const int v8x = vseg ^ (4 * ((m >> 2) & 1) + 2 * ((m >> 1) & 1));
    const f32x16 zero = {};
    auto load = [&](int st) {
        Frag f;
        const int t = st / PC, j = st % PC;
        if (j < QS) {
            const unsigned char* kp = krow + t * 4096;
            f.a = *(const u32x4*)(kp + 16 * ((4 * j + 2 * h2) ^ ksw));
            f.b = *(const u32x4*)(kp + 16 * ((4 * j + 2 * h2 + 1) ^ ksw));
        } else if constexpr (P8) {
            const int dt = 2 * t + (j - QS);  // d tile: head dims 32 dt .. 32 dt + 31
            u32x2 r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                r[q] = lds_read_tr8(v8row + 8 * q * 128 + 16 * ((2 * dt) ^ v8x ^ (q & 1 ? 5 : 0)));
            f.a = (u32x4){r[0][0], r[0][1], r[1][0], r[1][1]};
            f.b = (u32x4){r[2][0], r[2][1], r[3][0], r[3][1]};
        } else {
            const int v = j - QS, a2 = v >> 2, dt = v & 3;
            const u32x2 r = lds_read_tr8(vrow + (32 * t + 16 * a2) * 128 + 16 * ((2 * dt + vseg) ^ vsw));
            f.a = (u32x4){r[0], r[1], 0u, 0u};
        }
        return f;
    };
    auto compute = [&](int st, const Frag& f) {
        const int t = st / PC, j = st % PC;
        if (j < QS) {
            s[t] = mfma_32x32x64_fp8(f.a, f.b, qc.q[2 * j], qc.q[2 * j + 1], j == 0 ? zero : s[t]);
        } else if constexpr (P8) {
            const int dt = 2 * t + (j - QS);
            o[dt] = mfma_32x32x64_fp8(f.a, f.b, p[0], p[1], o[dt]);
        } else {
            const int v = j - QS, a2 = v >> 2, dt = v & 3;
            const u32x2 w0 = fp8x4_to_bf16x4(f.a[0]), w1 = fp8x4_to_bf16x4(f.a[1]);
            o[dt] = mfma_32x32x16<kBF16>((u32x4){w0[0], w0[1], w1[0], w1[1]}, p[2 * t + a2], o[dt]);
        }
    };
    // the moves' DMA instructions go out at steps 4, 6, 8, 10 (every other MFMA), or with fp8 P
    // (eight steps) at 4, 5, 6, 7
    constexpr int kDs = P8 ? 1 : 2;
    static_assert(!MOVE || NS > 4 + 3 * kDs, "the moves need their steps");
    u32x4 ek, ev;
    rsrc_t rk, rv;
    Frag fr[D];
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (i < NS) fr[i] = load(i);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const Frag f = fr[st % D];
        if (st + D < NS) fr[st % D] = load(st + D);
        if constexpr (MOVE) {
            if (st == 0) ek = *(const GBSA_LDS u32x4*)mv.kent;
            if (st == 1) ev = *(const GBSA_LDS u32x4*)mv.vent;
            if (st == 2) {
                const KvSrc src = page_half(kbase, ek, mv.khalf, rs);
                rk = make_rsrc(src.p, src.records);
            }
            if (st == 3) {
                const KvSrc src = page_half(vbase, ev, mv.vhalf, rs);
                rv = make_rsrc(src.p, src.records);
            }
            if (st == 4 || st == 4 + kDs) dma8_one(rk, rs, mv.kdst, mv.i0 + (st - 4) / kDs, lane);
            if (st == 4 + 2 * kDs || st == 4 + 3 * kDs)
                dma8_one(rv, rs, mv.vdst, mv.i0 + (st - 4 - 2 * kDs) / kDs, lane);
        }
        compute(st, f);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int OUT, int LAYOUT, bool P8 = false>
__global__ __launch_bounds__(512, 1) void fwd_prefill_ks32d_kernel(FwdArgs a) {
    constexpr int DT = kFP8;
    constexpr int R = 128;
    constexpr int esz = 1;
    constexpr int kStateBytes = 4 * (64 * 64 * 4 + 64 * 16);  // group 1's O, m, l for the merge
    constexpr int kLds = (16 * kHalf8 > kStateBytes) ? 16 * kHalf8 : kStateBytes;
    // [K buffers 0..7][V buffers 0..7], one fp8 half page each; reused for the final merge
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
    // per visible page: byte offset of this head's slice, readable bytes of its two halves
    __shared__ u32x4 plist[256];
    __shared__ int jlist[256];  // per visible page: block index * 4 + mask class
    __shared__ int flag[2];     // visible pages of the unit; slot trace on
    static_assert(sizeof(smem) >= kPieceListBytes, "the split merge borrows the stages");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;  // waves w and w + 4 share a SIMD and the same query rows
    const int gw = wave & 3;    // wave within its group
    if (!header_ok(a)) {
        refuse(a);
        return;
    }
    const int U = a.meta[3];
    __shared__ int task_word[2];
    run_tasks<true>(a, U, task_word, [&](const FwdArgs& a, const Task& tk) {
        const int w = tk.w, st = tk.st;
        const Bound b0 = tk.b0, b1 = tk.b1;
        if (!bound_less(b0, b1) || b0.u >= U) return;
        UnitIter it = locate_unit(a, b0.u);
        if (it.b < 0) return;

        const int rs = a.N2 * 128 * esz;
        const unsigned char* kbase = (const unsigned char*)a.k;
        const unsigned char* vbase = (const unsigned char*)a.v;
        unsigned char* const kst = smem;
        unsigned char* const vst = smem + 8 * kHalf8;

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
            const int row_base = st * R;
            if (row_base < rows_exist) {
                const KvSeq kv = kv_seq<LAYOUT>(a, it.b);
                const int skv = kv.len;
                const int off = diag_off(a, skv, it.sq);
                const int row0 = row_base + gw * 32;
                QCol32 qc;
                float colscale, mrun = kNegInf, lrun = 0.f;
                int trow;
                bool rvalid;
                load_q32<DT>(a, it, t0, rows_exist, row0, lane, qc, colscale, trow, rvalid);
                const float pq = P8 ? p_quant(a, it, row0, rows_exist, lane) : 1.f;
                f32x16 o[4];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] = (f32x16){};
                const int t_lo = t0 + row_base / a.G;
                const int t_hi = t0 + (min(row_base + R, rows_exist) - 1) / a.G;
                const int32_t* sel = a.idx + ((int64_t)it.n2 * a.tqb + g) * a.topK;
                const int64_t head_off = (int64_t)it.n2 * 128 * esz;

                if (wave == 0) {
                    int n = 0;
                    for (int c0 = sa; c0 < se; c0 += 64) {
                        int jl = -1, pl = 0, cl = 0;
                        if (c0 + lane < se) {
                            jl = sel[c0 + lane];
                            if (jl >= 0) {
                                cl = block_class(a, (int64_t)jl * 128, skv, off, t_lo, t_hi);
                                if (cl != 0) pl = kv.unit<LAYOUT>(jl);
                            }
                        }
                        const uint64_t mm = __ballot(cl != 0);
                        if (cl != 0) {
                            const int pos = n + __builtin_amdgcn_mbcnt_hi(
                                                    (uint32_t)(mm >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0));
                            const uint64_t po = (uint64_t)((int64_t)pl * a.kv_stride * esz + head_off);
                            plist[pos] = (u32x4){(uint32_t)po, (uint32_t)(po >> 32),
                                                 (uint32_t)kv_records(rs, skv - 128 * jl),
                                                 (uint32_t)kv_records(rs, skv - 128 * jl - 64)};
                            jlist[pos] = jl * 4 + cl;
                        }
                        n += __builtin_popcountll(mm);
                    }
                    if (lane == 0) {
                        flag[0] = n;
                        flag[1] = slot_trace_claim(n);
                    }
                }
                __syncthreads();
                const int n = __builtin_amdgcn_readfirstlane(flag[0]);  // items per group
                const int nh = 2 * n;                                   // half pages
                SlotTrace tr;
                tr.begin(__builtin_amdgcn_readfirstlane(flag[1]) != 0, wave);

                if (n > 0) {
                    f32x16 s[2];
                    u32x4 p[4];
                    const uint32_t umw[8] = {};  // (no user mask)
                    // Intervals, one barrier per item pair: in interval i group 0 runs its MFMA
                    // item i (half page 2 i) and then its softmax item i, group 1 its softmax
                    // item i - 1 and then its MFMA item i (half page 2 i + 1), so that on each
                    // SIMD one wave issues MFMAs while its partner exponentiates, twice per
                    // interval. The moves of MFMA item i of group g (K_{2i+4+g}, V_{2i+2+g}) are
                    // read in interval i + 2: before the barrier that ends an interval a wave
                    // waits for all but its newest batch. Each replaces a half page whose last
                    // reader ran in interval i - 2. Before the first interval: K_0 .. K_3, V_0
                    // and V_1 by all eight waves (instruction `wave` of each).
                    auto pre_move = [&](const unsigned char* base, int q, unsigned char* dst) {
                        q = min(q, nh - 1);
                        const KvSrc src = page_half(base, plist[q >> 1], q & 1, rs);
                        dma8_one(make_rsrc(src.p, src.records), rs, dst, wave, lane);
                    };
#pragma unroll
                    for (int q = 0; q < 4; ++q) pre_move(kbase, q, kst + q * kHalf8);
                    pre_move(vbase, 0, vst);
                    pre_move(vbase, 1, vst + kHalf8);
                    wait_vm<0>();
                    __syncthreads();
                    // the moves of this group's MFMA item k (half page q = 2 k + grp): K_{q+4}
                    // and V_{q+2}, sources clamped into the stream (a clamped move fills a buffer
                    // that is not read again)
                    auto move_of = [&](int k) {
                        const int q = 2 * k + grp;
                        const int kq = min(q + 4, nh - 1), vq = min(q + 2, nh - 1);
                        return ItemMove8{plist + (kq >> 1), plist + (vq >> 1),
                                         kst + ((q + 4) & 7) * kHalf8, vst + ((q + 2) & 7) * kHalf8,
                                         kq & 1, vq & 1, 2 * gw};
                    };
                    int jc_next = __builtin_amdgcn_readfirstlane(jlist[0]);
                    auto softmax_item = [&](int k) {
                        const int jc = jc_next;
                        __builtin_amdgcn_sched_barrier(0);
                        tr.mark(1, lane);
                        softmax_item32<DT, false, false, P8>(a, s, p, colscale, trow, umw, jc >> 2,
                                                             grp, jc & 3, skv, off, lane, mrun, lrun,
                                                             o, pq);
                        pin_softmax(p, lrun);
                        __builtin_amdgcn_sched_barrier(0);
                        tr.mark(2, lane);
                    };
                    // knext: the page of this wave's next softmax item
                    auto end_interval = [&](int knext) {
                        const int jn = jlist[min(knext, n - 1)];
                        wait_vm<4>();  // all but this interval's moves are in LDS
                        tr.mark(3, lane);
                        __syncthreads();
                        tr.mark(4, lane);
                        jc_next = __builtin_amdgcn_readfirstlane(jn);
                    };
                    // Issue priority as in the 256-row DMA kernel: the MFMA items run raised.
                    moves8_now(move_of(0), kbase, vbase, rs, lane);
                    tr.mark(5, lane);
                    __builtin_amdgcn_s_setprio(3);
                    mfma_item32d8<true, false, false, P8>(kst + grp * kHalf8, vst, qc, s, p, o, lane);
                    __builtin_amdgcn_s_setprio(0);
                    tr.mark(6, lane);
                    if (grp == 0) softmax_item(0);
                    end_interval(grp == 0 ? 1 : 0);
                    for (int k = 1; k < n; ++k) {
                        const int q = 2 * k + grp;
                        if (grp == 1) softmax_item(k - 1);
                        tr.mark(5, lane);
                        __builtin_amdgcn_s_setprio(3);
                        mfma_item32d8<true, true, true, P8>(kst + (q & 7) * kHalf8,
                                                            vst + ((q - 2) & 7) * kHalf8, qc, s, p, o,
                                                            lane, move_of(k), kbase, vbase, rs);
                        __builtin_amdgcn_s_setprio(0);
                        tr.mark(6, lane);
                        if (grp == 0) softmax_item(k);
                        end_interval(grp == 0 ? k + 1 : k);
                    }
                    if (grp == 1) softmax_item(n - 1);
                    __builtin_amdgcn_s_setprio(3);
                    mfma_item32d8<false, true, false, P8>(kst, vst + ((nh - 2 + grp) & 7) * kHalf8, qc,
                                                          s, p, o, lane);
                    __builtin_amdgcn_s_setprio(0);
                    wait_vm<0>();  // nothing may land in LDS after the task
                }
                __syncthreads();  // stages are free: group 1 hands its row states to group 0

                if (grp == 1) {
                    f32x4* so = (f32x4*)(smem + gw * (64 * 64 * 4 + 64 * 16));
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4)
                            so[(dt * 4 + g4) * 64 + lane] = (f32x4){o[dt][4 * g4], o[dt][4 * g4 + 1],
                                                                   o[dt][4 * g4 + 2], o[dt][4 * g4 + 3]};
                    so[16 * 64 + lane] = (f32x4){mrun, lrun, 0.f, 0.f};
                }
                __syncthreads();
                if (grp == 0) {
                    const f32x4* so = (const f32x4*)(smem + gw * (64 * 64 * 4 + 64 * 16));
                    const f32x4 ml = so[16 * 64 + lane];
                    const float m = fmaxf(mrun, ml[0]);
                    const float a0 = (m == kNegInf) ? 0.f : fast_exp2(mrun - m);
                    const float a1 = (m == kNegInf) ? 0.f : fast_exp2(ml[0] - m);
                    mrun = m;
                    lrun = lrun * a0 + ml[1] * a1;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const f32x4 x = so[(dt * 4 + g4) * 64 + lane];
#pragma unroll
                            for (int e = 0; e < 4; ++e) o[dt][4 * g4 + e] = o[dt][4 * g4 + e] * a0 + x[e] * a1;
                        }
                    write_rows32<DT, OUT>(a, it, complete, 2 * w + (sa > 0 ? 0 : 1), row0, lane, trow,
                                          rvalid, mrun, lrun, o, 1.f / pq);
                }
                __syncthreads();  // LDS is reused by the next task
                if (!complete) {
                    int* list = (int*)smem;  // the stages are free until the next task
                    const int np = piece_arrive(a, w, u, st, a.nst, list);
                    if (np > 0)
                        merge_rows<OUT>(a, list, np, row_base, min(row_base + R, rows_exist), it.n2,
                                        t0, it.row0, it.sq);
                    __syncthreads();
                }
            }
            advance_unit(a, it);
        }
    });
}

// Whole units per task pay off once the units outnumber the resident workgroups this many
// times over (the last tasks then are a small share of every workgroup's time).
constexpr int kUnitTaskFactor = 8;

// Launches KERN with its grid: one workgroup per worker and row subtile (the worker plan), or,
// with many units and a kernel built for them (DYN), as many workgroups as stay resident on
// the device, taking whole units.
template <auto KERN, bool DYN>
hipError_t launch_k(FwdArgs a, hipStream_t s) {
    static std::atomic<int> per_cu{0};  // resident workgroups per CU (0: not yet asked)
    int occ = per_cu.load(std::memory_order_relaxed);
    if (occ == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, KERN, 512, 0) != hipSuccess ||
            n < 1)
            n = 1;
        per_cu.store(n, std::memory_order_relaxed);
        occ = n;
    }
    const int64_t resident = (int64_t)a.cus * occ;
    int64_t grid = (int64_t)a.P * a.nst;
    a.unit_tasks = 0;
    if (DYN && (int64_t)a.N2 * a.tqb * a.nst >= kUnitTaskFactor * resident) {
        a.unit_tasks = 1;
        grid = resident >= kQueues ? resident / kQueues * kQueues : resident;
    }
    hipLaunchKernelGGL(KERN, dim3((unsigned)grid), dim3(512), 0, s, a);
    return hipGetLastError();
}

template <int DT, int OUT, int LAYOUT, bool UM>
hipError_t launch_l(const FwdArgs& a, int rows, hipStream_t s) {
    // 8 waves per workgroup either way: 32 rows per wave for large units, 16 below (more
    // workgroups, fewer registers)
    // softmax precision 1 with f16 runs the 16-bit softmax item in the two ping-pong kernels
    // (the other kernels and the user-mask variants compute it in fp32, which the mode allows)
    constexpr bool kHalf = DT == kF16 && !UM;
    if (rows == 256 && DT != kFP8) {
        if constexpr (kHalf)
            if (a.half_softmax)
                return launch_k<fwd_prefill_pp32d_kernel<kF16, OUT, LAYOUT, false, true>, true>(a, s);
        // (the dtype expression keeps the fp8 instantiation, which never runs, compilable)
        return launch_k<fwd_prefill_pp32d_kernel<(DT == kFP8 ? kBF16 : DT), OUT, LAYOUT, UM>, !UM>(a,
                                                                                             s);
    }
    // quant mode 5 with a P quantisation scale: P·V on fp8 MFMA in the two fp8 ping-pong
    // kernels (the user-mask variants, the decode and the 17-64-row kernels keep P in bf16)
    constexpr bool kP8 = DT == kFP8 && !UM;
    if (rows == 256) {
        if constexpr (kP8)
            if (a.ps != nullptr)
                return launch_k<fwd_prefill_pp32_kernel<kFP8, OUT, LAYOUT, false, true>, true>(a, s);
        return launch_k<fwd_prefill_pp32_kernel<DT, OUT, LAYOUT, UM>, !UM>(a, s);
    }
    if (a.M > 64) {
        if constexpr (kHalf)
            if (a.half_softmax)
                return launch_k<fwd_prefill_ks32_kernel<kF16, OUT, LAYOUT, false, true>, true>(a, s);
        if constexpr (kP8)
            if (a.ps != nullptr)
                return launch_k<fwd_prefill_ks32d_kernel<OUT, LAYOUT, true>, true>(a, s);
        // fp8 without a user mask: the DMA kernel
        if constexpr (DT == kFP8 && !UM)
            return launch_k<fwd_prefill_ks32d_kernel<OUT, LAYOUT>, true>(a, s);
        else
            return launch_k<fwd_prefill_ks32_kernel<DT, OUT, LAYOUT, UM>, !UM>(a, s);
    }
    // 17-64 rows: the keys of every page are split over 2 or 4 wave groups, so that no wave
    // computes on missing rows and each page goes through LDS 2 or 4 times, not 8
    if (a.M > 32) return launch_k<fwd_prefill_kernel<DT, OUT, 8, 1, 2, LAYOUT, UM>, !UM>(a, s);
    return launch_k<fwd_prefill_kernel<DT, OUT, 8, 1, 4, LAYOUT, UM>, !UM>(a, s);
}

// The KV layout and the user mask are template arguments, so that the plain paged kernels
// carry neither test.
template <int DT, int OUT>
hipError_t launch_t(const FwdArgs& a, int rows, hipStream_t s) {
    const bool tnd = a.cu_kv != nullptr;
    if (a.umask != nullptr)
        return tnd ? launch_l<DT, OUT, kTnd, true>(a, rows, s)
                   : launch_l<DT, OUT, kPaged, true>(a, rows, s);
    return tnd ? launch_l<DT, OUT, kTnd, false>(a, rows, s)
               : launch_l<DT, OUT, kPaged, false>(a, rows, s);
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, int dtype, int out_dtype, int rows, hipStream_t s) {
    if (dtype == kF16) return launch_t<kF16, kF16>(a, rows, s);
    if (dtype == kBF16) return launch_t<kBF16, kBF16>(a, rows, s);
    if (out_dtype == kF16) return launch_t<kFP8, kF16>(a, rows, s);
    return launch_t<kFP8, kBF16>(a, rows, s);
}

}  // namespace gbsa

#ifdef GBSA_SLOT_TRACE
// Readout of the diagnostic build (declared in gbsa_slot_trace.h).
extern "C" int gbsa_slot_trace_read(unsigned long long* host_dst) {
    return (int)hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(gbsa::g_slot_trace),
                                    sizeof(unsigned long long) * 8 * gbsa::kTraceEvents);
}
extern "C" int gbsa_slot_trace_reset(void) {
    static unsigned long long zeros[8 * gbsa::kTraceEvents];
    static const int zero = 0;
    hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(gbsa::g_slot_trace_claim), &zero, sizeof(int));
    if (e != hipSuccess) return (int)e;
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(gbsa::g_slot_trace), zeros, sizeof(zeros));
}
#endif
