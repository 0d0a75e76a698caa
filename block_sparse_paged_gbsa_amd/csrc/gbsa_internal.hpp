// Internal declarations shared by the host entry points and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gbsa {

// Metadata buffer format (1024 int32 words), written by the scheduler kernel:
//   [0] magic  [1] version  [2] P (workers)  [3] U (units)  [4..5] total cost (lo, hi)
//   [6] number of split units  [7] N1 [8] N2 [9] D [10] blockShapeX [11] blockShapeY
//   [12] topK [13] mask_mode [14] quant_mode [15] totalQBlocks [16] B [17] win_left
//   [18] win_right [19] seqused_q given [20] is_packed_gqa [21] kv_layout [22..23] 0
//   [24 + w], w = 0..P: boundary of worker w, packed (unit << 9) | slot; the rest 0.
constexpr int kMetaWords = 1024;
constexpr int kHeaderWords = 24;
constexpr int kSlotBits = 9;
constexpr int kSlotMask = (1 << kSlotBits) - 1;
constexpr uint32_t kMagic = 0x41534247u;  // bytes "GBSA"
constexpr int kVersion = 1;
constexpr int kMaxWorkers = kMetaWords - kHeaderWords - 1;
constexpr int kMaxUnits = 1 << (32 - kSlotBits - 1);
// header words the main kernels compare against their own parameters
constexpr int kCheckFirst = 7, kCheckLast = 21;

enum DType : int { kF16 = 0, kBF16 = 1, kFP8 = 2 };

// Upper bound of the scheduler kernels' static shared variables (bytes); the host sizes their
// dynamic LDS so that both fit in the 160 KiB of a CU.
constexpr int kMetaStaticLds = 512;

struct MetaArgs {
    const int32_t* count;  // [N2, tqb]
    const int64_t* cu;     // [B+1]
    const int32_t* squ;    // [B] or null
    int32_t* meta;         // [1024]
    int32_t B, N2, X, topK, tqb, P;
    int32_t ucap;  // units whose clamped counts the kernel keeps in LDS between its passes
    int32_t header[kHeaderWords];  // words 7..21 prefilled by the host; the rest computed
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* idx;    // [N2, tqb, topK]
    const int32_t* cnt;    // [N2, tqb]
    const int32_t* meta;   // [1024]
    const int64_t* cu;     // [B+1]
    const int32_t* squ;    // [B] or null
    const int32_t* skv;    // [B]; may be null with token-major key/value
    const int32_t* table;  // [B, maxb] (paged key/value) or null (token-major)
    const int64_t* cu_kv;  // [B+1] token-major key/value, else null
    const float* qs;       // [N1] or null
    const float* ks;       // [N2] or null
    const float* vs;       // [N2] or null
    void* out;             // [T, N1, D]
    float* lse;            // [T, N1] or null
    int32_t* ws_status;    // workspace word 0: non-zero = metadata mismatch
    int32_t* ws_arrive;    // [P * nst] arrival counters of split units (left at zero)
    int32_t* ws_queue;     // workspace words 16..48: task queue counters (left at zero)
    int32_t unit_tasks;    // 1: tasks are whole units taken from the queues; 0: worker plan
    int32_t cus;           // compute units of the device
    int32_t half_softmax;  // softmax precision 1 with f16: the 16-bit softmax item
    const float* ps;       // [N1] P quantisation scales (quant 5), or null: P stays 16-bit
    float ps_max;          // largest P * scale: the destination type's max, at most 448
    float* ws_o;           // [2P, M, 128]
    float* ws_m;           // [2P, M]  running max, log2 domain
    float* ws_l;           // [2P, M]  running sum
    int64_t kv_stride;     // elements per storage unit: a page (paged) or a row (token-major)
    int64_t kv_rows;       // token-major: rows of key (= of value); paged: unused
    const uint8_t* umask;  // user attention mask or null: [rows, cols] per sequence or shared
    int64_t um_bstride;    // bytes between sequences' masks (0: shared)
    int32_t um_rstride, um_rows, um_cols;  // row stride (bytes) and extent
    int32_t B, N1, N2, G, X, topK, tqb, maxb, P, M, nst;
    int32_t mask, wl, wr, return_lse;  // mask: 0 none, 1 causal bottom-right, 2 top-left
    float scale_log2;      // softmax scale * log2(e)
    int64_t T;             // rows of query / attention_out / softmax_lse
    uint32_t out_nan2;     // two quiet NaNs of the output type, packed (refused calls)
    int32_t expect[kHeaderWords];  // expected header words (0, 1, 2 and 7..21 are checked)
};

// Arguments of the opt-in value check (gbsa_validate).
struct ValArgs {
    const int64_t* cu;      // [B+1]
    const int32_t* squ;     // [B] or null
    const int32_t* skv;     // [B] or null
    const int64_t* cu_kv;   // [B+1] token-major, else null
    const int32_t* table;   // [B, maxb] paged, else null
    const int32_t* cnt;     // [N2, tqb]
    const int32_t* idx;     // [N2, tqb, topK]
    const uint8_t* umask;   // user mask or null (only its extent is checked)
    int32_t* out;           // device flags
    int64_t total_q, num_pages, kv_rows;
    int32_t B, N2, X, tqb, topK, maxb, um_rows, um_cols;
    int32_t max_sq, max_skv;  // given length bounds, or 0
};

// Workspace layout (byte offsets), a pure function of P and M.
struct WsLayout {
    size_t status, arrive, o, m, l, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline WsLayout ws_layout(int64_t P, int64_t M, int64_t nst) {
    WsLayout w;
    w.status = 0;
    w.arrive = 256;
    w.o = align_up(w.arrive + sizeof(int32_t) * P * nst, 256);
    w.m = align_up(w.o + sizeof(float) * 2 * P * M * 128, 256);
    w.l = align_up(w.m + sizeof(float) * 2 * P * M, 256);
    w.total = align_up(w.l + sizeof(float) * 2 * P * M, 256);
    return w;
}

// Launchers (each defined next to its kernel).
hipError_t launch_metadata(const MetaArgs& a, hipStream_t s);
hipError_t launch_validate(const ValArgs& a, hipStream_t s);
// Main kernel choice: rows per unit M = blockShapeX * G. M <= 16 uses the decode kernel
// (KV slots spread over the waves), larger M the prefill kernel (rows over the waves).
hipError_t launch_decode(const FwdArgs& a, int dtype, int out_dtype, hipStream_t s);
hipError_t launch_prefill(const FwdArgs& a, int dtype, int out_dtype, int rows_per_wg,
                          hipStream_t s);

// Rows a prefill workgroup covers for a given M: 256 (eight waves of 32 rows) above 256,
// else 128 (two groups of four waves sharing the same rows, or eight 16-row waves).
inline int prefill_rows_per_wg(int M) { return M > 256 ? 256 : 128; }
constexpr int kDecodeMaxRows = 16;
// Row subtiles per unit (workgroups per worker) for a given M.
inline int64_t subtiles(int64_t M) {
    if (M <= kDecodeMaxRows) return 1;
    const int r = prefill_rows_per_wg((int)M);
    return (M + r - 1) / r;
}

}  // namespace gbsa
