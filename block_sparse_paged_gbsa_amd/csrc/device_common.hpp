// Device helpers for gfx950: MFMA wrappers, LDS transpose reads, packing, task iteration.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gbsa_internal.hpp"

namespace gbsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define GBSA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescaling: the running max of a column only moves when a new block exceeds it by more
// than kLazyMax (log2 units). Probabilities are then bounded by 2^kLazyMax = 256, which fp32
// sums and 16-bit P represent without loss of relative precision, and the O rescale is skipped
// for most blocks. The result is unchanged: numerator and denominator use the same max.
constexpr float kLazyMax = 8.f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// MFMA: 16x16x32 with fp32 accumulation. Operand lane layout (wave64):
//   A (16 x 32): lane l holds row l%16, k = (l/16)*8 .. +8
//   B (32 x 16): lane l holds col l%16, k = (l/16)*8 .. +8
//   C (16 x 16): lane l holds col l%16, rows (l/16)*4 .. +4
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<kBF16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<kF16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// e4m3 x e4m3 (8 values per lane, same lane layout).
__device__ __forceinline__ f32x4 mfma_16x16x32_fp8(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a),
                                                      __builtin_bit_cast(long, b), c, 0, 0, 0);
}

// Two fp32 -> packed 16-bit (round to nearest even) of the PV operand type.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x, float y);
template <>
__device__ __forceinline__ uint32_t pack2<kBF16>(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
}
template <>
__device__ __forceinline__ uint32_t pack2<kF16>(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
}

// 16-bit transpose read from LDS (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane 4r+c supplies the address of elements [4c, 4c+4) of row r of a 4x16 block; lane i
// receives column i, i.e. the four elements block[0..3][i].
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
    bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GBSA_LDS bf16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four OCP e4m3 values (one dword) -> four bf16 (two dwords), exactly: every e4m3 value is
// representable in bf16. Uses gfx950's direct conversion with a unit scale. (Reassembling the
// two fp32 results of v_cvt_pk_f32_fp8 with shifts or v_perm was miscompiled by this
// toolchain: element 1 was folded onto element 0.)
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t x) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, 1.0f, true);
    return (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Reductions across the four 16-lane groups that share an MFMA column (lanes l, l^16, l^32,
// l^48), with the gfx950 lane-swap VALU ops. With both operands equal, permlane16_swap returns
// the pair {x[l], x[l^16]} (in a fixed order) in both lanes of the pair, permlane32_swap the
// pair {x[l], x[l^32]}; the results are therefore bit-identical across the four lanes.
__device__ __forceinline__ float pair_max(float x, bool wide) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = wide ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                  : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x, bool wide) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = wide ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                  : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float wave_max_cols(float x) { return pair_max(pair_max(x, false), true); }
__device__ __forceinline__ float wave_sum_cols(float x) { return pair_sum(pair_sum(x, false), true); }

// Workgroups are handed to the 8 XCDs round-robin; give each XCD a contiguous range of
// logical indices so that neighbouring work (same sequence and KV head) shares an L2.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
    constexpr int kXcd = 8;
    if (grid % kXcd != 0) return bid;
    const int per = grid / kXcd;
    return (bid % kXcd) * per + bid / kXcd;
}

// Buffer resource over a wave-uniform base: one VGPR offset per lane, per-instruction
// constants in the scalar offset. `records` bytes from the base are readable (at most
// 2^31-1); a dword at or beyond it reads as zero without a memory access. The range check
// counts the scalar offset too (checked on gfx950 hardware).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int records = 0x7fffffff) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, records,
                                             0x00020000);
}
// kNT: non-temporal streaming hint (data read once).
constexpr int kCached = 0, kNT = 2;
template <int POLICY = kCached>
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY));
}

// ---------------------------------------------------------------------------
// KV side of a sequence. Paged key/value (PA_BBND) locate logical block j through the
// block table; token-major key/value (TND) hold block j at rows cu_kv[b] + 128 j onwards
// (GenericBlockSparseAttention article, "general constraints": layoutKv TND takes
// cu_seqlens_kv, with seqused_kv as the optional visible length). Both give a storage unit
// whose byte address is unit * kv_stride * element size.
// ---------------------------------------------------------------------------
// The layout is fixed at compile time (kPaged, kTnd) or read from the arguments (kAnyLayout).
enum KvLayout : int { kAnyLayout = 0, kPaged = 1, kTnd = 2 };
template <int L>
__device__ __forceinline__ bool is_tnd(const FwdArgs& a) {
    return L == kAnyLayout ? a.cu_kv != nullptr : L == kTnd;
}
struct KvSeq {
    const int32_t* table;  // block-table row of the sequence, or null (token-major)
    int row0;              // token-major: first row of the sequence
    int len;               // visible keys
    template <int L = kAnyLayout>
    __device__ __forceinline__ int unit(int j) const {
        if constexpr (L == kPaged) return table[j];
        if constexpr (L == kTnd) return row0 + 128 * j;
        return table ? table[j] : row0 + 128 * j;
    }
};
// (b is clamped into [0, B): after the last unit advance_unit leaves b == B, and a load for
// that state must not reach past seqused_kv or the block table.)
template <int L = kAnyLayout>
__device__ __forceinline__ KvSeq kv_seq(const FwdArgs& a, int b) {
    b = min(max(b, 0), a.B - 1);
    KvSeq s;
    if (!is_tnd<L>(a)) {
        s.table = a.table + (int64_t)b * a.maxb;
        s.row0 = 0;
        s.len = a.skv[b];
    } else {
        // the sequence's rows, kept inside the tensor whatever cu_kv holds
        const int64_t c0 = min(max(a.cu_kv[b], (int64_t)0), a.kv_rows);
        const int64_t c1 = min(max(a.cu_kv[b + 1], c0), a.kv_rows);
        const int st = (int)(c1 - c0);
        s.table = nullptr;
        s.row0 = (int)c0;
        s.len = a.skv != nullptr ? min(a.skv[b], st) : st;
    }
    return s;
}
// A load window `off` bytes into key or value whose first `nv` rows are visible keys (rows
// are `rs` bytes apart). Its records end after those rows, so the rows past the visible
// length read as zeros without a memory access: whatever they hold (stale or unset cache
// memory, another sequence's keys) cannot reach the output through a zero softmax weight,
// and a token-major block that runs past the tensor's last row never reads beyond it (the
// visible length ends inside the tensor).
__device__ __forceinline__ int kv_records(int rs, int nv) {
    return (int)min((int64_t)max(nv, 0) * rs, (int64_t)0x7fffffff);
}
struct KvSrc {
    const unsigned char* p;
    int records;
};
__device__ __forceinline__ KvSrc kv_src(const void* base, int64_t off, int rs, int nv) {
    return KvSrc{(const unsigned char*)base + off, kv_records(rs, nv)};
}

// ---------------------------------------------------------------------------
// Metadata access shared by the main and combine kernels.
// ---------------------------------------------------------------------------
// Every word is compared (no short circuit), so the loads issue together: one round trip.
__device__ __forceinline__ bool header_ok(const FwdArgs& a) {
    const int32_t* m = a.meta;
    uint32_t diff = (uint32_t)(m[0] ^ a.expect[0]) | (uint32_t)(m[1] ^ a.expect[1]) |
                    (uint32_t)(m[2] ^ a.expect[2]);
#pragma unroll
    for (int i = kCheckFirst; i <= kCheckLast; ++i) diff |= (uint32_t)(m[i] ^ a.expect[i]);
    return diff == 0;
}

// A call whose metadata does not match its parameters computes nothing. Every workgroup of
// the grid fills its share of attention_out and softmax_lse with NaN, so that a caller who
// does not read the status word cannot take stale memory for a result, and the first one
// sets the status word.
__device__ __forceinline__ void refuse(const FwdArgs& a) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.ws_status, 1);
    const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n16 = a.T * a.N1 * 128 * 2 / 16;  // 16-bit outputs, 16 bytes per store
    const u32x4 nan8 = (u32x4){a.out_nan2, a.out_nan2, a.out_nan2, a.out_nan2};
    for (int64_t i = first; i < n16; i += nthr) ((u32x4*)a.out)[i] = nan8;
    if (a.lse != nullptr)
        for (int64_t i = first; i < a.T * a.N1; i += nthr) a.lse[i] = __builtin_nanf("");
}

struct Bound {
    int u, s;
};
__device__ __forceinline__ Bound read_bound(const int32_t* meta, int w) {
    uint32_t x = (uint32_t)meta[kHeaderWords + w];
    return Bound{(int)(x >> kSlotBits), (int)(x & kSlotMask)};
}
__device__ __forceinline__ bool bound_less(Bound a, Bound b) {
    return a.u < b.u || (a.u == b.u && a.s < b.s);
}

__device__ __forceinline__ int ceil_div_i(int64_t a, int b) { return (int)((a + b - 1) / b); }

// ---------------------------------------------------------------------------
// Task assignment of the prefill kernels.
//
// A task is one row subtile of a range of units. With the worker plan (small problems), task
// w * nst + st is worker w's range of unit slots (split units merged by the last piece) and
// every workgroup of the grid runs one task. With unit tasks (unit_tasks != 0; the host picks
// this when there are many more units than resident workgroups), task u * nst + st is all of
// unit u, and a grid of resident workgroups takes tasks until none are left: the XCDs of one
// device do not run at one clock under load, and a fixed share per XCD waits for the slowest.
// Each XCD has a queue over a contiguous eighth of the tasks (neighbouring units share key
// pages in that XCD's L2); a workgroup drains its own XCD's queue, then the others in turn.
// ---------------------------------------------------------------------------
struct Task {
    int w, st;      // worker (-1 for a unit task) and row subtile
    Bound b0, b1;   // unit slots [b0, b1)
};

constexpr int kQueues = 8;         // one per XCD
constexpr int kQueueStride = 4;    // words between queue counters
constexpr int kQueueDone = kQueues * kQueueStride;  // word of the finished-workgroup counter

// Thread 0: next task of the queues, starting at this workgroup's own (home) and moving on
// when one is empty; -1 when all are. `probe` (thread 0's) counts the queues found empty. A
// queue hands out its tasks in list order, or from its end (desc): with a causal or windowed
// selection, later q-blocks of a head select more blocks, so from the end the largest units go
// first and the smallest make up the tail.
__device__ __forceinline__ int task_grab(int32_t* q, int ntask, int home, int& probe, bool desc) {
    while (probe < kQueues) {
        const int x = (home + probe) & (kQueues - 1);
        const int lo = (int)((int64_t)ntask * x / kQueues);
        const int hi = (int)((int64_t)ntask * (x + 1) / kQueues);
        if (hi > lo) {
            const int t = __hip_atomic_fetch_add(q + x * kQueueStride, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            if (t < hi - lo) return desc ? hi - 1 - t : lo + t;
        }
        ++probe;
    }
    return -1;
}

// Whether the queues go from their ends: when the units' mean cost (selected blocks + 1) is
// under 3/4 of the most a unit can cost, so that unit sizes vary widely (dense causal
// selections: 1 .. topK blocks). With nearly equal units the list order measured faster.
__device__ __forceinline__ bool tasks_descending(const FwdArgs& a, int U) {
    const uint64_t W = (uint64_t)(uint32_t)a.meta[4] | ((uint64_t)(uint32_t)a.meta[5] << 32);
    return 4 * W < 3 * (uint64_t)U * (uint64_t)(a.topK + 1);
}

// Thread 0, once per workgroup after its last (failed) grab: the last workgroup of the grid
// to get here sets the counters back to zero for the next call. Every grab of every
// workgroup has returned before that workgroup counts itself here (the grabs return values
// it waits for), so no grab can land after the reset.
__device__ __forceinline__ void task_finish(int32_t* q) {
    const int done = __hip_atomic_fetch_add(q + kQueueDone, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - 1) {
        for (int x = 0; x < kQueues; ++x)
            __hip_atomic_store(q + x * kQueueStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + kQueueDone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The kernel's FwdArgs, read through a pointer the compiler cannot follow: the body then loads
// each argument where it uses it, instead of the compiler hoisting the loads to the top (out of
// the task loop) and keeping the values live, in spilled scalar registers, through every item
// of every task. The kernels take FwdArgs as their only argument, at the start of the kernel
// argument segment (taking the address of the parameter itself would copy it to private
// memory).
__device__ __forceinline__ const FwdArgs& opaque_args() {
    using KernArgs = const __attribute__((address_space(4))) FwdArgs;
    KernArgs* kp = (KernArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(kp));
    return *(const FwdArgs*)kp;
}

// Runs body(args, Task) for this workgroup's tasks. Whole workgroup; `word` points to two LDS ints
// (the next task, and thread 0's count of queues found empty), so that no loop state stays in
// registers across the body. The body may use barriers and LDS freely: the next task starts
// after a barrier. (One call site, so that the body is inlined once.) Kernels built without
// DYN run the worker plan only, with no loop around the body (their launcher never asks for
// unit tasks): the variants at the register limit keep their allocation.
template <bool DYN, class F>
__device__ __forceinline__ void run_tasks(const FwdArgs& a, int U, int* word, F&& body) {
    if constexpr (!DYN) {
        const int lin = xcd_remap(blockIdx.x, gridDim.x);
        const int w = lin / a.nst;
        body(opaque_args(), Task{w, lin - w * a.nst, read_bound(a.meta, w), read_bound(a.meta, w + 1)});
        return;
    }
    // word[1]: the count of queues found empty (low byte) and the queue order (bit 8)
    if (threadIdx.x == 0) word[1] = (a.unit_tasks && tasks_descending(a, U)) ? 256 : 0;
    for (;;) {
        if (threadIdx.x == 0) {
            int lin = -1;
            if (a.unit_tasks) {
                int probe = word[1] & 255;
                const bool desc = (word[1] >> 8) != 0;
                lin = task_grab(a.ws_queue, U * a.nst, blockIdx.x & (kQueues - 1), probe, desc);
                word[1] = (word[1] & ~255) | probe;
            } else if (word[1] == 0) {
                lin = xcd_remap(blockIdx.x, gridDim.x);  // the workgroup's one worker task
                word[1] = 1;
            }
            word[0] = lin;
        }
        __syncthreads();
        const int lin = __builtin_amdgcn_readfirstlane(word[0]);
        if (lin < 0) break;
        const int q = lin / a.nst;  // unit or worker
        Task tk{-1, lin - q * a.nst, Bound{q, 0}, Bound{q + 1, 0}};
        if (!a.unit_tasks) {
            tk.w = q;
            tk.b0 = read_bound(a.meta, q);
            tk.b1 = read_bound(a.meta, q + 1);
        }
        body(opaque_args(), tk);
        __syncthreads();
    }
    if (a.unit_tasks && threadIdx.x == 0) task_finish(a.ws_queue);
}

// Position in the ordered unit list (b, n2, active q-block gl).
struct UnitIter {
    int b, n2, gl;
    int nact;     // active q-blocks of batch b
    int qbase;    // global index of batch b's first q-block
    int64_t row0; // cu_seqlens_q[b]
    int storage;  // storage length of batch b
    int sq;       // active length of batch b
};

__device__ __forceinline__ void batch_lengths(const FwdArgs& a, int b, int64_t* row0, int* storage,
                                              int* sq) {
    const int64_t c0 = a.cu[b], c1 = a.cu[b + 1];
    const int st = (int)(c1 - c0);
    int s = st;
    if (a.squ != nullptr) s = min(max(a.squ[b], 0), st);
    *row0 = c0;
    *storage = st;
    *sq = s;
}

// Lengths of sequence b (zeros past the last one), one sequence per lane.
struct SeqLens {
    int64_t r0;  // cu_seqlens_q[b]
    int st, sq;  // storage and active length
};
__device__ __forceinline__ SeqLens seq_lens(const FwdArgs& a, int b) {
    SeqLens l{0, 0, 0};
    if (b < a.B) {
        // all three loads issue together: without seqused_q the third one rereads cu_seqlens_q
        const int32_t* su = a.squ != nullptr ? a.squ + b : (const int32_t*)(a.cu + b);
        const int64_t c0 = a.cu[b], c1 = a.cu[b + 1];
        const int sv = *su;
        l.r0 = c0;
        l.st = (int)(c1 - c0);
        l.sq = a.squ != nullptr ? min(max(sv, 0), l.st) : l.st;
    }
    return l;
}

// Find the batch holding unit u0. Every wave scans the batches on its own (64 per step, wave
// prefix sums, no LDS and no barrier), so all lanes of the block end with the same answer.
// `first` may carry the lengths of sequences 0..63 (lane = sequence), loaded early by the
// caller so that their latency overlaps its own first loads. Returns it.b = -1 when u0 lies
// beyond the last unit.
__device__ inline UnitIter locate_unit(const FwdArgs& a, int u0, const SeqLens* first = nullptr) {
    const int lane = threadIdx.x & 63;
    int ucarry = 0, qcarry = 0, found_b = -1, found_u = 0, found_q = 0;
    UnitIter it;
    for (int base = 0; base < a.B && found_b < 0; base += 64) {
        const int b = base + lane;
        const SeqLens l = (base == 0 && first != nullptr) ? *first : seq_lens(a, b);
        int nu = 0, nq = 0;
        if (b < a.B) {
            nq = ceil_div_i(l.st, a.X);
            nu = a.N2 * ceil_div_i(l.sq, a.X);
        }
        int iu = nu, iq = nq;  // inclusive wave scans
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int xu = __shfl_up(iu, o), xq = __shfl_up(iq, o);
            if (lane >= o) {
                iu += xu;
                iq += xq;
            }
        }
        const int uex = ucarry + iu - nu, qex = qcarry + iq - nq;
        const uint64_t hit = __ballot(b < a.B && nu > 0 && u0 >= uex && u0 < uex + nu);
        // values read across lanes are uniform: tell the compiler (scalar registers)
        if (hit) {
            const int h = __builtin_ctzll(hit);
            found_b = base + h;
            found_u = __builtin_amdgcn_readlane(uex, h);
            found_q = __builtin_amdgcn_readlane(qex, h);
            const uint64_t r0 = (uint64_t)l.r0;
            it.row0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(r0 >> 32), h)
                                 << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)r0, h));
            it.storage = __builtin_amdgcn_readlane(l.st, h);
            it.sq = __builtin_amdgcn_readlane(l.sq, h);
        }
        ucarry += __builtin_amdgcn_readlane(iu, 63);
        qcarry += __builtin_amdgcn_readlane(iq, 63);
    }
    it.b = found_b;
    if (found_b < 0) return it;
    const int local = u0 - found_u;
    it.nact = ceil_div_i(it.sq, a.X);
    it.n2 = local / it.nact;
    it.gl = local % it.nact;
    it.qbase = found_q;
    return it;
}

// Next unit in (b, n2, gl) order. After the last unit of the grid it leaves it.b == B, it.gl
// == it.n2 == 0 and qbase + gl == totalQBlocks, with the other fields those of the last
// sequence: no unit. Callers test the unit bound before loading anything for the new state;
// code that loads ahead for the next unit must not treat that state as a unit (its count and
// selection row are another KV head's or past the arrays, and its batch is one past
// seqused_kv and the block table).
__device__ __forceinline__ void advance_unit(const FwdArgs& a, UnitIter& it) {
    if (++it.gl < it.nact) return;
    it.gl = 0;
    if (++it.n2 < a.N2) return;
    it.n2 = 0;
    do {
        it.qbase += ceil_div_i(it.storage, a.X);
        ++it.b;
        if (it.b >= a.B) return;
        batch_lengths(a, it.b, &it.row0, &it.storage, &it.sq);
        it.nact = ceil_div_i(it.sq, a.X);
    } while (it.nact == 0);
}

// Key-block visibility classes for one query-row range [t_lo, t_hi] of batch b.
// Returns 0: nothing visible (skip), 1: everything visible (no mask), 2: mask per element.
__device__ __forceinline__ int block_class(const FwdArgs& a, int64_t p0, int skv, int off, int t_lo,
                                           int t_hi) {
    const int64_t p1 = p0 + 127;
    const int64_t dlo = (int64_t)t_lo + off, dhi = (int64_t)t_hi + off;
    if (p0 >= skv) return 0;
    if (a.mask != 0 && p0 > dhi) return 0;
    if (a.wl >= 0 && p1 < dlo - a.wl) return 0;
    if (a.wr >= 0 && p0 > dhi + a.wr) return 0;
    bool full = p1 < skv;
    if (a.mask != 0) full = full && (p1 <= dlo);
    if (a.wl >= 0) full = full && (p0 >= dhi - a.wl);
    if (a.wr >= 0) full = full && (p1 <= dlo + a.wr);
    return full ? 1 : 2;
}

__device__ __forceinline__ bool key_visible(const FwdArgs& a, int64_t p, int skv, int64_t d) {
    bool ok = p < skv;
    if (a.mask != 0) ok = ok && (p <= d);
    if (a.wl >= 0) ok = ok && (p >= d - a.wl);
    if (a.wr >= 0) ok = ok && (p <= d + a.wr);
    return ok;
}

// Offset of the causal diagonal: bottom-right (off = kv length - query length) for mask modes
// 0 and 1, top-left (off = 0) for mode 2. Windows are relative to the same diagonal.
__device__ __forceinline__ int diag_off(const FwdArgs& a, int skv, int sq) {
    return a.mask == 2 ? 0 : skv - sq;
}

// ---------------------------------------------------------------------------
// User attention mask: uint8, nonzero = the key is masked out for that query row, indexed by
// the batch-local query row t and the key position p; one [rows, cols] array per sequence or
// one shared by all. Entries outside the extent do not mask.
// ---------------------------------------------------------------------------
struct UMaskRow {
    rsrc_t r;  // the sequence's mask, records = rows x row stride
    int roff;  // byte offset of this lane's row, or -1 (no row, or a row past the extent)
};
__device__ __forceinline__ UMaskRow umask_row(const FwdArgs& a, int b, int t, bool valid) {
    UMaskRow m;
    m.r = make_rsrc(a.umask + (int64_t)b * a.um_bstride, a.um_rows * a.um_rstride);
    m.roff = (valid && t < a.um_rows) ? t * a.um_rstride : -1;
    return m;
}
// Mask bytes of keys p .. p + 3 (p a multiple of 4) in this lane's row, 0 for a visible key.
__device__ __forceinline__ uint32_t umask_word(const FwdArgs& a, const UMaskRow& m, int64_t p) {
    const bool in = m.roff >= 0 && p < a.um_cols;
    const int voff = in ? m.roff + (int)p : 0x7fffffff;  // past the records: reads 0
    uint32_t w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(m.r, voff, 0, 0));
    const int64_t n = (int64_t)a.um_cols - p;  // keys of the group inside the extent
    if (n < 4) w &= (n <= 0) ? 0u : (0xffffffffu >> (32 - 8 * (int)n));
    return w;
}

// Visible key positions of query row d = t + off inside the block starting at p0, as an
// inclusive range of offsets [*lo, *hi] relative to p0 (empty when *lo > *hi).
__device__ __forceinline__ void key_range(const FwdArgs& a, int64_t p0, int skv, int64_t d,
                                          int* lo, int* hi) {
    int64_t l = 0, h = (int64_t)skv - 1;
    if (a.mask != 0) h = min(h, d);
    if (a.wl >= 0) l = max(l, d - a.wl);
    if (a.wr >= 0) h = min(h, d + a.wr);
    l -= p0;
    h -= p0;
    *lo = (int)max((int64_t)0, min(l, (int64_t)128));
    *hi = (int)max((int64_t)-1, min(h, (int64_t)127));
}

// New running max (log2 domain) under lazy rescaling; mx is the block max already scaled.
__device__ __forceinline__ float lazy_max(float mrun, float mx) {
    return (mx > mrun + kLazyMax) ? mx : mrun;
}

}  // namespace gbsa
