// Scheduler kernel: writes the load-balanced task split into the 1024-int32 metadata buffer.
//
// GenericBlockSparseAttention article (cf-1.com), "two-stage call": the metadata operator
// computes the AICore task split (load balancing) ahead of the main operator and stores it
// in a fixed (1024,) int32 tensor. The contents are this library's own format (described in
// gbsa_internal.hpp): work units (b, kv head, active q-block) cost count + 1 each and their
// kv slots are cut into P contiguous segments of equal cost. Everything is integer
// arithmetic, so the result is bit-exact and deterministic ("general constraints":
// deterministic by default).
#include "device_common.hpp"
#include "launch_lds.hpp"

namespace gbsa {
namespace {

template <typename T>
__device__ T block_exclusive_scan(T x, T* total, T* sh) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    T inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        T y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) sh[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        T v = lane < nw ? sh[lane] : T(0);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            T y = __shfl_up(v, o);
            if (lane >= o) v += y;
        }
        if (lane < nw) sh[lane] = v;
    }
    __syncthreads();
    const T prefix = wid > 0 ? sh[wid - 1] : T(0);
    *total = sh[nw - 1];
    __syncthreads();
    return prefix + inc - x;
}


// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by 1, 2, 4, 8
// within each row of 16 lanes, then lane 15 of each row into the next row and lane 31 into
// the upper half (lanes whose source is outside the row receive 0).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
    return x;
}

// Exclusive prefix sum over a 1024-thread workgroup (16 waves); sh holds 16 ints and must not
// be reused by the caller before the next barrier. One barrier.
__device__ __forceinline__ int block_exclusive_scan32(int x, int* total, int* sh) {
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int inc = wave_inclusive_scan(x);
    if (lane == 63) sh[wid] = inc;
    __syncthreads();
    const int winc = wave_inclusive_scan(lane < 16 ? sh[lane] : 0);  // every wave, redundantly
    const int before = wid > 0 ? __builtin_amdgcn_readlane(winc, wid - 1) : 0;
    *total = __builtin_amdgcn_readlane(winc, 15);
    return before + inc - x;
}

__device__ __forceinline__ int upper_bound_batch(const int* ubase, int B, int u) {
    // largest b with ubase[b] <= u (ubase is non-decreasing, ubase[0] = 0)
    int lo = 0, hi = B;  // invariant: ubase[lo] <= u, answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ubase[mid] <= u) lo = mid;
        else hi = mid;
    }
    return lo;
}

// A unit's place in (sequence, KV head, q-block) order, found once and then advanced one unit
// at a time without divisions (the chunked path's cost is per-unit integer work).
struct UnitPos {
    int b, n2, gl, nact;
};
__device__ __forceinline__ UnitPos unit_pos(const MetaArgs& a, const int* ubase, int u) {
    const int b = upper_bound_batch(ubase, a.B, u);
    const int nact = (ubase[b + 1] - ubase[b]) / a.N2;
    const int local = u - ubase[b];
    return UnitPos{b, local / nact, local % nact, nact};
}
__device__ __forceinline__ void unit_next(const MetaArgs& a, const int* ubase, UnitPos& p) {
    if (++p.gl < p.nact) return;
    p.gl = 0;
    if (++p.n2 < a.N2) return;
    p.n2 = 0;
    do {
        if (++p.b >= a.B) return;
        p.nact = (ubase[p.b + 1] - ubase[p.b]) / a.N2;
    } while (p.nact == 0);
}
__device__ __forceinline__ int pos_count(const MetaArgs& a, const int* qbase, const UnitPos& p) {
    const int g = qbase[p.b] + p.gl;
    int c = 0;
    if (p.b < a.B && g < a.tqb) c = a.count[(int64_t)p.n2 * a.tqb + g];
    return min(max(c, 0), a.topK);
}

__global__ __launch_bounds__(1024) void metadata_kernel(MetaArgs a) {
    extern __shared__ int tabs[];  // qbase[B+1], ubase[B+1], counts of the first ucap units
    __shared__ long long sh64[16];
    __shared__ int sh_split;
    static_assert(sizeof(sh64) + sizeof(sh_split) <= kMetaStaticLds, "static LDS budget");
    const int tid = threadIdx.x, nt = blockDim.x;
    int* qbase = tabs;
    int* ubase = tabs + a.B + 1;
    int* ucount = tabs + 2 * (a.B + 1);

    // Per-sequence q-block and unit offsets.
    long long cq = 0, cu = 0;
    for (int base = 0; base < a.B; base += nt) {
        const int b = base + tid;
        long long nq = 0, nu = 0;
        if (b < a.B) {
            const int64_t st = a.cu[b + 1] - a.cu[b];
            int64_t sq = st;
            if (a.squ != nullptr) sq = min((int64_t)max(a.squ[b], 0), st);
            nq = (st + a.X - 1) / a.X;
            nu = (long long)a.N2 * ((sq + a.X - 1) / a.X);
        }
        long long tq, tu;
        const long long eq = block_exclusive_scan<long long>(nq, &tq, sh64);
        const long long eu = block_exclusive_scan<long long>(nu, &tu, sh64);
        if (b < a.B) {
            qbase[b] = (int)(cq + eq);
            ubase[b] = (int)(cu + eu);
        }
        cq += tq;
        cu += tu;
    }
    if (tid == 0) {
        qbase[a.B] = (int)cq;
        ubase[a.B] = (int)cu;
        sh_split = 0;
    }
    __syncthreads();
    const int U = (int)cu;
    const int P = a.P;

    // Total cost (counts kept in LDS for the boundary pass). Each thread walks a contiguous
    // run of units, issuing eight independent count loads at a time.
    constexpr int kLoadBatch = 8;
    long long part = 0;
    {
        const int R = (U + nt - 1) / nt;
        const int ua = min(tid * R, U), ub = min(ua + R, U);
        UnitPos pos = ua < ub ? unit_pos(a, ubase, ua) : UnitPos{0, 0, 0, 1};
        for (int u0 = ua; u0 < ub; u0 += kLoadBatch) {
            int c[kLoadBatch];
#pragma unroll
            for (int k = 0; k < kLoadBatch; ++k) {
                c[k] = (u0 + k < ub) ? pos_count(a, qbase, pos) : 0;
                if (u0 + k < ub) unit_next(a, ubase, pos);
            }
#pragma unroll
            for (int k = 0; k < kLoadBatch; ++k) {
                const int u = u0 + k;
                if (u < ub) {
                    if (u < a.ucap) ucount[u] = c[k];
                    part += c[k] + 1;
                }
            }
        }
    }
    long long W;
    (void)block_exclusive_scan<long long>(part, &W, sh64);  // ends with a barrier

    // Boundaries: unit u owns the targets floor(w*W/P) that fall in [C_u, C_u + cost_u).
    // Each thread takes kRun consecutive units of a chunk: a local prefix over its run, one
    // block scan of the run totals per chunk; the first target at or after the run's start is
    // found with one division, and the targets are then walked (one division per boundary).
    constexpr int kRun = 4;
    long long carry = 0;
    for (int base = 0; base < U; base += kRun * nt) {
        const int u0 = base + tid * kRun;
        int c[kRun];
        if (u0 < U) {
            // counts past the LDS cache are read from memory, walking from the first such unit
            const int uw = max(u0, a.ucap);
            UnitPos pos = uw < min(u0 + kRun, U) ? unit_pos(a, ubase, uw) : UnitPos{0, 0, 0, 1};
#pragma unroll
            for (int k = 0; k < kRun; ++k) {
                const int u = u0 + k;
                c[k] = (u >= U) ? -1 : (u < a.ucap ? ucount[u] : pos_count(a, qbase, pos));
                if (u >= a.ucap && u < U) unit_next(a, ubase, pos);
            }
        } else {
#pragma unroll
            for (int k = 0; k < kRun; ++k) c[k] = -1;
        }
        long long run = 0;
#pragma unroll
        for (int k = 0; k < kRun; ++k) run += (c[k] >= 0) ? c[k] + 1 : 0;
        long long tot;
        long long Cu = carry + block_exclusive_scan<long long>(run, &tot, sh64);
        if (run > 0) {
            long long w = (Cu * P + W - 1) / W;  // first worker whose target is >= Cu
            long long t = w < P ? (w * W) / P : 0;
#pragma unroll
            for (int k = 0; k < kRun; ++k) {
                if (c[k] < 0) break;
                const int u = u0 + k;
                const long long cost = c[k] + 1;
                const int nslots = max(c[k], 1);
                bool split = false;  // a boundary strictly inside unit u
                while (w < P && t < Cu + cost) {
                    const int s = (int)(t - Cu);
                    uint32_t word;
                    if (s < nslots) {
                        word = ((uint32_t)u << kSlotBits) | (uint32_t)s;
                        split = split || (s > 0);
                    } else {
                        word = (uint32_t)(u + 1) << kSlotBits;
                    }
                    a.meta[kHeaderWords + w] = (int32_t)word;
                    ++w;
                    t = w < P ? (w * W) / P : 0;
                }
                if (split) atomicAdd(&sh_split, 1);
                Cu += cost;
            }
        }
        carry += tot;
    }
    if (U == 0) {
        for (int w = tid; w < P; w += nt) a.meta[kHeaderWords + w] = 0;
    }
    for (int i = kHeaderWords + P + 1 + tid; i < kMetaWords; i += nt) a.meta[i] = 0;
    __syncthreads();
    if (tid == 0) {
        a.meta[kHeaderWords + P] = (int32_t)((uint32_t)U << kSlotBits);
        a.meta[0] = (int32_t)kMagic;
        a.meta[1] = kVersion;
        a.meta[2] = P;
        a.meta[3] = U;
        a.meta[4] = (int32_t)(uint32_t)(W & 0xffffffffll);
        a.meta[5] = (int32_t)(uint32_t)(W >> 32);
        a.meta[6] = sh_split;
        for (int i = kCheckFirst; i <= kCheckLast; ++i) a.meta[i] = a.header[i];
        for (int i = kCheckLast + 1; i < kHeaderWords; ++i) a.meta[i] = 0;
    }
}


// Same task split for problems whose tables fit in LDS (at most kFastMaxB sequences and
// N2 * totalQBlocks clamped counts): every input is loaded at once, the unit costs are scanned
// once (each thread owns a contiguous run of units), and each worker's boundary is found by a
// binary search of its cost target in the unit prefix. Boundary w is the first cut position
// whose consumed cost reaches floor(w * W / P), exactly as above.
__global__ __launch_bounds__(1024) void metadata_fast_kernel(MetaArgs a) {
    extern __shared__ int tabs[];  // qbase[B+1], ubase[B+1], counts[N2*tqb], pre[N2*tqb+1], sp[1024]
    __shared__ int sh_a[16], sh_b[16], sh_c[16];
    __shared__ int sh_split;
    static_assert(sizeof(sh_a) * 3 + sizeof(sh_split) <= kMetaStaticLds, "static LDS budget");
    const int tid = threadIdx.x, nt = blockDim.x;
    const int NC = a.N2 * a.tqb;
    int* qbase = tabs;
    int* ubase = tabs + a.B + 1;
    int* counts = tabs + 2 * (a.B + 1);
    int* pre = counts + NC;
    int* sp = pre + NC + 1;

    // all global reads are issued up front
    // (all values below fit in 32 bits: at most N2 * tqb units, each costing at most topK + 1)
    int nq = 0, nu = 0;
    if (tid < a.B) {
        const int64_t st = a.cu[tid + 1] - a.cu[tid];
        int64_t sq = st;
        if (a.squ != nullptr) sq = min((int64_t)max(a.squ[tid], 0), st);
        nq = (int)((st + a.X - 1) / a.X);
        nu = a.N2 * (int)((sq + a.X - 1) / a.X);
    }
    for (int i = tid; i < NC; i += nt) counts[i] = min(max(a.count[i], 0), a.topK);
    if (tid == 0) sh_split = 0;
    int tq, tu;
    const int eq = block_exclusive_scan32(nq, &tq, sh_a);
    const int eu = block_exclusive_scan32(nu, &tu, sh_b);
    if (tid < a.B) {
        qbase[tid] = eq;
        ubase[tid] = eu;
    }
    if (tid == 0) {
        qbase[a.B] = tq;
        ubase[a.B] = tu;
    }
    __syncthreads();
    const int U = tu;
    const int P = a.P;

    // unit costs (count + 1) and their exclusive prefix
    const int R = (U + nt - 1) / nt;
    const int u0 = min(tid * R, U), u1 = min(u0 + R, U);
    int run = 0;
    for (int u = u0; u < u1; ++u) {
        const int b = upper_bound_batch(ubase, a.B, u);
        const int nact = (ubase[b + 1] - ubase[b]) / a.N2;
        const int local = u - ubase[b];
        const int n2 = local / nact, g = qbase[b] + local % nact;
        const int c = (g < a.tqb) ? counts[n2 * a.tqb + g] : 0;
        pre[u] = c + 1;  // cost, replaced by the prefix below
        run += c + 1;
    }
    int W;
    int acc = block_exclusive_scan32(run, &W, sh_c);
    for (int u = u0; u < u1; ++u) {
        const int cost = pre[u];
        pre[u] = acc;
        acc += cost;
    }
    if (tid == 0) pre[U] = W;
    __syncthreads();

    // boundary of worker w: the unit whose cost range holds the target t = floor(w W / P)
    if (tid < P) {
        const int w = tid;
        uint32_t word = 0;
        int spu = -1;
        if (U > 0) {
            const int t = (int)(((long long)w * W) / P);
            int lo = 0, hi = U;  // largest u with pre[u] <= t (pre[0] = 0 <= t < pre[U] = W)
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (pre[mid] <= t) lo = mid;
                else hi = mid;
            }
            const int u = lo;
            const int s = (int)(t - pre[u]);
            const int nslots = max(pre[u + 1] - pre[u] - 1, 1);
            if (s < nslots) {
                word = ((uint32_t)u << kSlotBits) | (uint32_t)s;
                if (s > 0) spu = u;
            } else {
                word = (uint32_t)(u + 1) << kSlotBits;
            }
        }
        a.meta[kHeaderWords + w] = (int32_t)word;
        sp[w] = spu;
    }
    for (int i = kHeaderWords + P + 1 + tid; i < kMetaWords; i += nt) a.meta[i] = 0;
    __syncthreads();
    // split units: distinct units holding a boundary strictly inside (consecutive in w)
    if (tid < P && sp[tid] >= 0 && (tid == 0 || sp[tid - 1] != sp[tid])) atomicAdd(&sh_split, 1);
    __syncthreads();
    if (tid == 0) {
        a.meta[kHeaderWords + P] = (int32_t)((uint32_t)U << kSlotBits);
        a.meta[0] = (int32_t)kMagic;
        a.meta[1] = kVersion;
        a.meta[2] = P;
        a.meta[3] = U;
        a.meta[4] = W;  // the total fits in 32 bits here
        a.meta[5] = 0;
        a.meta[6] = sh_split;
        for (int i = kCheckFirst; i <= kCheckLast; ++i) a.meta[i] = a.header[i];
        for (int i = kCheckLast + 1; i < kHeaderWords; ++i) a.meta[i] = 0;
    }
}

}  // namespace

hipError_t launch_metadata(const MetaArgs& a, hipStream_t s) {
    const size_t lds_max = 160 * 1024;
    // fast path: every table in LDS (the unit count is at most N2 * tqb)
    const size_t nc = (size_t)a.N2 * (size_t)a.tqb;
    const size_t fast_bytes = sizeof(int) * (2 * ((size_t)a.B + 1) + 2 * nc + 1 + 1024);
    if (a.B <= 1024 && a.P <= 1024 && fast_bytes + kMetaStaticLds <= lds_max) {
        static std::atomic<int> granted[kMaxDevices];
        const hipError_t e =
            ensure_dynamic_lds((const void*)metadata_fast_kernel, granted, fast_bytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(metadata_fast_kernel, dim3(1), dim3(1024), fast_bytes, s, a);
        return hipGetLastError();
    }
    // per-sequence tables plus the cached counts (the unit count is at most N2 * tqb),
    // within 160 KiB of LDS
    const size_t tab_bytes = sizeof(int) * 2 * (size_t)(a.B + 1);
    const size_t lds = tab_bytes + sizeof(int) * (size_t)a.ucap;
    static std::atomic<int> granted[kMaxDevices];
    const hipError_t e = ensure_dynamic_lds((const void*)metadata_kernel, granted, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(1024), lds, s, a);
    return hipGetLastError();
}

}  // namespace gbsa
