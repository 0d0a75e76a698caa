// Main kernel for units with at most 16 query rows (packed-GQA tile M = blockShapeX * G <= 16),
// the decode shape. These units are bound by the bytes of the gathered KV pages, so the design
// keeps page loads in flight on every compute unit:
//  * a workgroup of 4 waves per worker; two fit on a CU (<= 256 VGPRs per lane), the default
//    worker count puts one on each;
//  * wave q owns token quarter q (32 tokens) of every selected page of the task and keeps its
//    own online-softmax state for the <= 16 query columns; the four states are merged through
//    LDS at the end of the task (fixed order);
//  * the next page's quarter is loaded into registers (full 256-byte rows, coalesced) while
//    the current one is computed;
//  * K and V of the quarter are staged in a wave-private LDS buffer: K is read back in MFMA
//    A-operand layout (S^T = K Q^T, 16x16x32), V with the gfx950 transpose read as the A
//    operand of O^T = V^T P^T;
//  * split units are merged in-kernel by the last arriving workgroup (split_merge.hpp).
// GenericBlockSparseAttention article (cf-1.com), "sparse attention mechanism" and
// "implementation architecture"; FlashAttention article (ai6s.net), "three steps".
#include "split_merge.hpp"

namespace gbsa {
namespace {

constexpr int kNW = 4;
constexpr int kVPitch = 288;                       // bytes per staged V row (16-bit)
template <int DT>
struct KPitch {
    static constexpr int value = (DT == kFP8) ? 136 : 272;  // bytes per staged K row
};
template <int DT>
struct Stage {
    static constexpr int k_bytes = 32 * KPitch<DT>::value;
    static constexpr int bytes = k_bytes + 32 * kVPitch;  // one quarter page per wave
};
constexpr int kMergeFloats = 16 * 128 + 32;        // per wave: O^T tile + m + l
template <int DT>
struct Lds {
    static constexpr int a = kNW * Stage<DT>::bytes, b = kNW * kMergeFloats * 4;
    static constexpr int bytes = a > b ? a : b;
};

// Registers of one quarter page (32 tokens), loaded with full-row coalescing:
// 16-bit rows are 256 B (16 lanes per row, 4 rows per load), fp8 rows 128 B (8 lanes, 8 rows).
struct Quarter {
    u32x4 k[8];
    u32x4 v[8];
};

__device__ __forceinline__ int row_off(int rs, int lane, int esz) {
    return esz == 2 ? (lane >> 4) * rs + (lane & 15) * 16 : (lane >> 3) * rs + (lane & 7) * 16;
}

// kq / vq: wave-uniform window of this wave's 32-token quarter of the K / V block slice.
template <int DT>
__device__ __forceinline__ void load_quarter(Quarter& qt, KvSrc kq, KvSrc vq, int rs, int loff) {
    const rsrc_t rk = make_rsrc(kq.p, kq.records), rv = make_rsrc(vq.p, vq.records);
    if constexpr (DT == kFP8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) qt.k[q] = buf_load16<kNT>(rk, loff, q * 8 * rs);
#pragma unroll
        for (int q = 0; q < 4; ++q) qt.v[q] = buf_load16<kNT>(rv, loff, q * 8 * rs);
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) qt.k[q] = buf_load16<kNT>(rk, loff, q * 4 * rs);
#pragma unroll
        for (int q = 0; q < 8; ++q) qt.v[q] = buf_load16<kNT>(rv, loff, q * 4 * rs);
    }
}

struct WaveState {
    float m, l;
    f32x4 o[8];
};

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int DT, bool UM>
__device__ __forceinline__ void compute_quarter(const FwdArgs& a, const Quarter& qt,
                                                const u32x4 (&qf)[4], const u32x2 (&q8)[4],
                                                float cs, int64_t p0, int cls, int skv, int64_t d,
                                                const UMaskRow& um, unsigned char* stage,
                                                int lane, WaveState& st) {
    constexpr int PT = (DT == kF16) ? kF16 : kBF16;
    constexpr int KP = KPitch<DT>::value;
    const int lrow = lane & 15, lgrp = lane >> 4;
    unsigned char* ks = stage;
    unsigned char* vs = stage + Stage<DT>::k_bytes;
    // stage K and V rows in LDS: K is re-read in MFMA A layout, V with the transpose read
    if constexpr (DT == kFP8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = q * 8 + (lane >> 3);
            u32x2* kd = (u32x2*)(ks + row * KP + (lane & 7) * 16);
            kd[0] = (u32x2){qt.k[q][0], qt.k[q][1]};
            kd[1] = (u32x2){qt.k[q][2], qt.k[q][3]};
            const u32x4 vx = qt.v[q];
            const u32x2 c0 = fp8x4_to_bf16x4(vx[0]), c1 = fp8x4_to_bf16x4(vx[1]);
            const u32x2 c2 = fp8x4_to_bf16x4(vx[2]), c3 = fp8x4_to_bf16x4(vx[3]);
            u32x4* vd = (u32x4*)(vs + row * kVPitch + (lane & 7) * 32);
            vd[0] = (u32x4){c0[0], c0[1], c1[0], c1[1]};
            vd[1] = (u32x4){c2[0], c2[1], c3[0], c3[1]};
        }
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            *(u32x4*)(ks + (q * 4 + lgrp) * KP + lrow * 16) = qt.k[q];
            *(u32x4*)(vs + (q * 4 + lgrp) * kVPitch + lrow * 16) = qt.v[q];
        }
    }
    wave_sync_lds();
    f32x4 sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
        const unsigned char* kr = ks + (tt * 16 + lrow) * KP;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if constexpr (DT == kFP8) {
                acc = mfma_16x16x32_fp8(*(const u32x2*)(kr + kk * 32 + lgrp * 8), q8[kk], acc);
            } else {
                acc = mfma_16x16x32<DT>(*(const u32x4*)(kr + (kk * 32 + lgrp * 8) * 2), qf[kk], acc);
            }
        }
        sacc[tt] = acc;
    }
    if (cls == 2) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!key_visible(a, p0 + tt * 16 + lgrp * 4 + i, skv, d)) sacc[tt][i] = kNegInf;
    }
    if constexpr (UM) {  // the user mask applies to every visible block
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const uint32_t w = umask_word(a, um, p0 + tt * 16 + lgrp * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if ((w >> (8 * i)) & 0xffu) sacc[tt][i] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[tt][i]);
    mx = wave_max_cols(mx);
    const float mnew = lazy_max(st.m, mx == kNegInf ? kNegInf : mx * cs);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(st.m - muse);
    st.m = mnew;
    uint32_t pk[2][2];
    float ls = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = fast_exp2(__builtin_fmaf(sacc[tt][i], cs, -muse));
            ls += pv[i];
        }
        pk[tt][0] = pack2<PT>(pv[0], pv[1]);
        pk[tt][1] = pack2<PT>(pv[2], pv[3]);
    }
    st.l = st.l * alpha + ls;
    if (__ballot(alpha != 1.f)) {  // skip the rescale when no running max moved
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;
    }

    const u32x4 pb = (u32x4){pk[0][0], pk[0][1], pk[1][0], pk[1][1]};
    const unsigned char* vrow = vs + (lgrp * 4 + (lrow >> 2)) * kVPitch + (lane & 3) * 8;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const u32x2 v0 = lds_read_tr16(vrow + dt * 32);
        const u32x2 v1 = lds_read_tr16(vrow + 16 * kVPitch + dt * 32);
        st.o[dt] = mfma_16x16x32<PT>((u32x4){v0[0], v0[1], v1[0], v1[1]}, pb, st.o[dt]);
    }
    wave_sync_lds();
}

template <int DT, int OUT, int LAYOUT, bool UM>
__global__ __launch_bounds__(256, 2) void fwd_decode_kernel(FwdArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[Lds<DT>::bytes];
    static_assert(sizeof(smem) >= kPieceListBytes, "the split merge borrows the stages");
    constexpr int esz = (DT == kFP8) ? 1 : 2;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform for the compiler
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int w = xcd_remap(blockIdx.x, gridDim.x);

    // one round trip for the header, this worker's bounds and the first 64 sequences' lengths
    // (the metadata buffer always holds kMetaWords words, so the bound reads stay inside it)
    const bool ok = header_ok(a);
    const Bound b0 = read_bound(a.meta, w), b1 = read_bound(a.meta, w + 1);
    const int U = a.meta[3];
    const SeqLens first = seq_lens(a, lane);
    if (!ok) {
        refuse(a);
        return;
    }
    if (!bound_less(b0, b1) || b0.u >= U) return;
    UnitIter it = locate_unit(a, b0.u, &first);
    if (it.b < 0) return;

    unsigned char* stage = smem + wave * Stage<DT>::bytes;
    const int rs = a.N2 * 128 * esz;  // bytes between tokens of a page
    const int loff = row_off(rs, lane, esz);

    for (int u = b0.u;; ++u) {
        const int sa = (u == b0.u) ? b0.s : 0;
        if (u >= U || u > b1.u || (u == b1.u && sa >= b1.s)) break;
        const int g = it.qbase + it.gl;
        const int32_t* sel = a.idx + ((int64_t)it.n2 * a.tqb + g) * a.topK;
        // the first 64 slots are read together with their count (in-row reads past the count
        // are ignored)
        int jfirst = -1;
        if (g < a.tqb && sa + lane < a.topK) jfirst = sel[sa + lane];
        int cnt = 0;
        if (g < a.tqb) cnt = min(max(a.cnt[(int64_t)it.n2 * a.tqb + g], 0), a.topK);
        const int se = (u == b1.u) ? b1.s : cnt;
        const bool complete = (sa == 0) && (se == cnt);
        const int t0 = it.gl * a.X;
        const int rows_exist = min(a.X, it.storage - t0) * a.G;
        const KvSeq kv = kv_seq<LAYOUT>(a, it.b);
        const int skv = kv.len;
        const int off = diag_off(a, skv, it.sq);

        // Q as the B operand: column = query row (lane & 15), k = head dim.
        const bool exists = lrow < rows_exist;
        const int t = t0 + (exists ? lrow / a.G : 0);
        const UMaskRow um =
            UM ? umask_row(a, it.b, t, exists) : UMaskRow{make_rsrc(nullptr, 0), -1};
        const int h = it.n2 * a.G + (exists ? lrow % a.G : 0);
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
                qf[kk] = (u32x4){0, 0, 0, 0};
            } else {
                qf[kk] = exists ? *(const u32x4*)((const uint16_t*)a.q + qoff + d)
                                : (u32x4){0, 0, 0, 0};
                q8[kk] = (u32x2){0, 0};
            }
        }
        const int t_lo = t0, t_hi = t0 + (rows_exist - 1) / a.G;
        const int64_t dpos = (int64_t)t + off;

        WaveState st;
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.o[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};

        const int64_t qbyte = (int64_t)wave * 32 * rs;  // this wave's token quarter
        for (int c0 = sa; c0 < se; c0 += 64) {
            // slots c0 .. c0+63: lane l holds slot c0 + l
            const int n = min(64, se - c0);
            // per slot: block index and class packed as j * 4 + class, its storage unit and
            // the records of this wave's quarter window
            int jcl = 0, pl = 0, rl = 0;
            if (lane < n) {
                const int jl = (c0 == sa) ? jfirst : sel[c0 + lane];
                if (jl >= 0) {
                    const int cl = block_class(a, (int64_t)jl * 128, skv, off, t_lo, t_hi);
                    if (cl != 0) {
                        jcl = jl * 4 + cl;
                        if constexpr (LAYOUT == kPaged) pl = kv.unit<LAYOUT>(jl);
                        rl = kv_records(rs, skv - 128 * jl - 32 * wave);
                    }
                }
            }
            uint64_t todo = __ballot(jcl != 0);
            if (todo == 0) continue;
            auto base_of = [&](int i, const void* p) {
                // token-major: the unit follows from the block index packed in jcl
                const int unit = (LAYOUT == kPaged)
                                     ? __builtin_amdgcn_readlane(pl, i)
                                     : kv.unit<LAYOUT>(__builtin_amdgcn_readlane(jcl, i) >> 2);
                return KvSrc{(const unsigned char*)p +
                                 ((int64_t)unit * a.kv_stride + (int64_t)it.n2 * 128) * esz +
                                 qbyte,
                             __builtin_amdgcn_readlane(rl, i)};
            };
            Quarter qa, qb;
            int ia = __builtin_ctzll(todo);
            todo &= todo - 1;
            load_quarter<DT>(qa, base_of(ia, a.k), base_of(ia, a.v), rs, loff);
            while (true) {
                int ib = -1;
                if (todo) {
                    ib = __builtin_ctzll(todo);
                    todo &= todo - 1;
                    load_quarter<DT>(qb, base_of(ib, a.k), base_of(ib, a.v), rs, loff);
                }
                {
                    const int jc = __builtin_amdgcn_readlane(jcl, ia);
                    const int j = jc >> 2, cls = jc & 3;
                    compute_quarter<DT, UM>(a, qa, qf, q8, cs, (int64_t)j * 128 + wave * 32, cls,
                                            skv, dpos, um, stage, lane, st);
                }
                if (ib < 0) break;
                ia = -1;
                if (todo) {
                    ia = __builtin_ctzll(todo);
                    todo &= todo - 1;
                    load_quarter<DT>(qa, base_of(ia, a.k), base_of(ia, a.v), rs, loff);
                }
                {
                    const int jc = __builtin_amdgcn_readlane(jcl, ib);
                    const int j = jc >> 2, cls = jc & 3;
                    compute_quarter<DT, UM>(a, qb, qf, q8, cs, (int64_t)j * 128 + wave * 32, cls,
                                            skv, dpos, um, stage, lane, st);
                }
                if (ia < 0) break;
            }
        }

        // ---- merge the four wave states (fixed order) ----------------------------------
        st.l = wave_sum_cols(st.l);
        __syncthreads();  // staging buffers are reused for the merge
        float* mg = (float*)smem + wave * kMergeFloats;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *(f32x4*)(mg + lrow * 128 + dt * 16 + lgrp * 4) = st.o[dt];
        if (lgrp == 0) {
            mg[16 * 128 + lrow] = st.m;
            mg[16 * 128 + 16 + lrow] = st.l;
        }
        __syncthreads();
        const int slot = 2 * w + (sa > 0 ? 0 : 1);
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
                    // 32-bit unsigned indices (2P x 16 rows fit): the compiler cannot split
                    // them into a per-lane 64-bit part and keep it live across the unit loop
                    const uint32_t mi = (uint32_t)slot * (uint32_t)a.M + (uint32_t)c;
                    const rsrc_t ro = ws_o_rsrc(a, slot);
                    ws_put4(ro, (c * 128 + d0) * 4,
                            (f32x4){acc[0], acc[1], acc[2], acc[3]} * vscale);
                    ws_put4(ro, (c * 128 + d0 + 4) * 4,
                            (f32x4){acc[4], acc[5], acc[6], acc[7]} * vscale);
                    if (d0 == 0) {
                        ws_put1(a.ws_m + mi, mstar);
                        ws_put1(a.ws_l + mi, lsum);
                    }
                }
            }
        }
        if (!complete) {
            int* list = (int*)smem;  // the stages are free until the next unit
            const int np = piece_arrive(a, w, u, 0, 1, list);
            if (np > 0) merge_rows<OUT>(a, list, np, 0, rows_exist, it.n2, t0, it.row0, it.sq);
        }
        __syncthreads();
        advance_unit(a, it);
    }
}

template <int DT, int OUT>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    // the layout and the user mask are template arguments: run-time ones cost the plain paged
    // path registers
    const dim3 g(a.P), b(256);
    const bool tnd = a.cu_kv != nullptr;
    if (a.umask != nullptr) {
        if (tnd)
            hipLaunchKernelGGL((fwd_decode_kernel<DT, OUT, kTnd, true>), g, b, 0, s, a);
        else
            hipLaunchKernelGGL((fwd_decode_kernel<DT, OUT, kPaged, true>), g, b, 0, s, a);
    } else if (tnd) {
        hipLaunchKernelGGL((fwd_decode_kernel<DT, OUT, kTnd, false>), g, b, 0, s, a);
    } else {
        hipLaunchKernelGGL((fwd_decode_kernel<DT, OUT, kPaged, false>), g, b, 0, s, a);
    }
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
