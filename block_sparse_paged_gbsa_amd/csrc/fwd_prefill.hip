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
//  * fwd_prefill_pp32_kernel (more than 256 rows, 256-row subtiles) and
//    fwd_prefill_ks32_kernel (65-256 rows, 128-row subtiles): two wave groups alternate MFMA and
//    softmax items on the same SIMDs over half pages (schedules described with each), on 32x32
//    MFMA tiles;
//  * fwd_prefill_kernel (17-64 rows): all waves in phase, 16 rows each, whole pages through a
//    double-buffered LDS stage with one barrier per page, each page's keys split over 2
//    (33-64 rows) or 4 (17-32 rows) wave groups that hold the same rows, 16x16 MFMA tiles.
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

template <int DT>
struct HalfStage {
    static constexpr int k_bytes = 64 * KLds<DT>::pitch;
    static constexpr int v_bytes = 64 * kVPitch;
};

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
template <int DT, bool qk, bool pv>
__device__ __forceinline__ void mfma_item32(const unsigned char* ks, const unsigned char* vs,
                                            const QCol32& qc, f32x16 (&s)[2],
                                            const u32x4 (&p)[4], f32x16 (&o)[4], int lane) {
    constexpr int PT = (DT == kF16) ? kF16 : kBF16;
    constexpr int KP = KLds<DT>::pitch;
    constexpr int QS = qk ? ((DT == kFP8) ? 2 : 8) : 0;  // QK steps per 32-key tile
    constexpr int VS = pv ? 8 : 0;                       // PV steps per 32-key tile (2 chunks x 4 d)
    constexpr int PC = QS + VS, NS = 2 * PC, D = kPipeDepth;
    const int h2 = lane >> 5;
    const unsigned char* krow = ks + (lane & 31) * KP;
    // transpose-read address of this lane (row offset within a 4-row group, column block)
    const unsigned char* vbase = vs + (4 * h2 + ((lane & 15) >> 2)) * kVPitch +
                                 (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
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

// Softmax item on 32x32 tiles for half page `half` of block j (class cls): mask, lazy running
// max (in-lane max over 32 keys, then the lane pair l, l ^ 32), rescale, P^T as PV B operands.
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

template <int DT, bool UM>
__device__ __forceinline__ void softmax_item32(const FwdArgs& a, f32x16 (&s)[2], u32x4 (&p)[4],
                                               float colscale, int trow, const uint32_t (&umw)[8],
                                               int j, int half, int cls, int skv, int off,
                                               int lane, float& mrun, float& lrun,
                                               f32x16 (&o)[4]) {
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
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
    mx = pair_max(mx, true);
    const float mnew = lazy_max(mrun, mx == kNegInf ? kNegInf : mx * colscale);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(mrun - muse);
    mrun = mnew;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // skipped unless some running max moved
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    float ls = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // chunk c = 2 t + a: elements 8 a .. 8 a + 7 of tile t
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pv[e] = fast_exp2(__builtin_fmaf(s[c >> 1][8 * (c & 1) + e], colscale, -muse));
            ls += pv[e];
        }
        p[c] = (u32x4){pack2<PT>(pv[0], pv[1]), pack2<PT>(pv[2], pv[3]), pack2<PT>(pv[4], pv[5]),
                       pack2<PT>(pv[6], pv[7])};
    }
    lrun = lrun * alpha + ls;
}

// Normalised O and LSE of a wave's 32 rows (lane pair l, l + 32 per row), or the split partial.
template <int DT, int OUT>
__device__ __forceinline__ void write_rows32(const FwdArgs& a, const UnitIter& it, bool complete,
                                             int slot, int row0, int lane, int trow, bool rvalid,
                                             float mrun, float lrun, const f32x16 (&o)[4]) {
    const int h2 = lane >> 5;
    const float ltot = pair_sum(lrun, true);
    const int r = row0 + (lane & 31);
    if (!rvalid) return;
    const float vscale = (DT == kFP8) ? a.vs[it.n2] : 1.f;
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
template <int DT, int OUT, int LAYOUT, bool UM>
__global__ __launch_bounds__(512, 1) void fwd_prefill_pp32_kernel(FwdArgs a) {
    constexpr int R = 256;
    constexpr int esz = (DT == kFP8) ? 1 : 2;
    constexpr int KB = HalfStage<DT>::k_bytes, VB = HalfStage<DT>::v_bytes;
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
                    if constexpr (DT == kFP8) {  // V is widened to bf16 on its way into LDS
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
                    softmax_item32<DT, UM>(a, s, p, colscale, trow, umw, jc >> 2, k & 1, jc & 3,
                                           skv, off, lane, mrun, lrun, o);
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
                mfma_item32<DT, true, false>(kst, vst, qc, s, p, o, lane);
                __syncthreads();
                softmax_and_move(0);
                for (int k = 1; k < nh; ++k) {
                    if constexpr (UM) umask_words32(a, um, jc_next >> 2, k & 1, lane, umw);
                    mfma_item32<DT, true, true>(kst + (k & 1) * KB, vst + ((k - 1) & 1) * VB, qc, s,
                                                p, o, lane);
                    __syncthreads();
                    softmax_and_move(k);
                }
                mfma_item32<DT, false, true>(kst, vst + ((nh - 1) & 1) * VB, qc, s, p, o, lane);
                if (grp == 0) __syncthreads();
            }
            __syncthreads();  // LDS (stages, page list) is reused by the next task

            write_rows32<DT, OUT>(a, it, complete, 2 * w + (sa > 0 ? 0 : 1), row0, lane, trow, rvalid,
                                  mrun, lrun, o);
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
template <int DT, int OUT, int LAYOUT, bool UM>
__global__ __launch_bounds__(512, 1) void fwd_prefill_ks32_kernel(FwdArgs a) {
    constexpr int R = 128;
    constexpr int esz = (DT == kFP8) ? 1 : 2;
    constexpr int KB = HalfStage<DT>::k_bytes, VB = HalfStage<DT>::v_bytes;
    constexpr int kStateBytes = 4 * (64 * 64 * 4 + 64 * 16);  // group 1's O, m, l for the merge
    constexpr int kLds = (2 * KB + 2 * VB > kStateBytes) ? 2 * KB + 2 * VB : kStateBytes;
    // [K buffer 0][K buffer 1][V buffer 0][V buffer 1]; reused for the final merge
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
    __shared__ int4 plist[256];  // as in the row-split kernel
    __shared__ int flag[1];
    static_assert(sizeof(smem) >= kPieceListBytes, "the split merge borrows the stages");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;  // waves w and w + 4 share a SIMD and the same query rows
    const int tg = tid & 255;
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
                if (lane == 0) flag[0] = n;
            }
            __syncthreads();
            const int n = __builtin_amdgcn_readfirstlane(flag[0]);  // items per group
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
                    if constexpr (DT == kFP8 || !kSharedPitch)
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
                    PageRegs<DT, 256, 64> pr;
                    page_load<DT, 256, 64>(pr, half_src(kbase, 2 * k + 2 + grp), rs, tg);
                    __builtin_amdgcn_sched_barrier(0);
                    softmax_item32<DT, UM>(a, s, p, colscale, trow, umw, jc >> 2, grp, jc & 3,
                                           skv, off, lane, mrun, lrun, o);
                    __builtin_amdgcn_sched_barrier(0);
                    store_k<DT, 256, 64>(pr, my_k, tg);
                    __syncthreads();
                };
                {
                    PageRegs<DT, 256, 64> pr;
                    page_load<DT, 256, 64>(pr, half_src(vbase, grp - 1), rs, tg);
                    mask_words(0);
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_item32<DT, true, false>(my_k, my_v, qc, s, p, o, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    v_move_store(pr);
                }
                __syncthreads();
                softmax_and_move(0);
                for (int k = 1; k < n; ++k) {
                    PageRegs<DT, 256, 64> pr;
                    page_load<DT, 256, 64>(pr, half_src(vbase, 2 * k + grp - 1), rs, tg);
                    mask_words(k);
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_item32<DT, true, true>(my_k, my_v, qc, s, p, o, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    v_move_store(pr);
                    __syncthreads();
                    softmax_and_move(k);
                }
                {
                    PageRegs<DT, 256, 64> pr;
                    page_load<DT, 256, 64>(pr, half_src(vbase, 2 * n + grp - 1), rs, tg);
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_item32<DT, false, true>(my_k, my_v, qc, s, p, o, lane);
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
                                      rvalid, mrun, lrun, o);
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
}

template <int DT, int OUT, int LAYOUT, bool UM>
hipError_t launch_l(const FwdArgs& a, int rows, hipStream_t s) {
    const int grid = a.P * a.nst;
    // 8 waves per workgroup either way: 32 rows per wave for large units, 16 below (more
    // workgroups, fewer registers)
    if (rows == 256) {
        hipLaunchKernelGGL((fwd_prefill_pp32_kernel<DT, OUT, LAYOUT, UM>), dim3(grid), dim3(512),
                           0, s, a);
    } else if (a.M > 64) {
        hipLaunchKernelGGL((fwd_prefill_ks32_kernel<DT, OUT, LAYOUT, UM>), dim3(grid), dim3(512),
                           0, s, a);
    } else if (a.M > 32) {
        // 17-64 rows: the keys of every page are split over 2 or 4 wave groups, so that no
        // wave computes on missing rows and each page goes through LDS 2 or 4 times, not 8
        hipLaunchKernelGGL((fwd_prefill_kernel<DT, OUT, 8, 1, 2, LAYOUT, UM>), dim3(grid),
                           dim3(512), 0, s, a);
    } else {
        hipLaunchKernelGGL((fwd_prefill_kernel<DT, OUT, 8, 1, 4, LAYOUT, UM>), dim3(grid),
                           dim3(512), 0, s, a);
    }
    return hipGetLastError();
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
