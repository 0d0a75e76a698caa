// Host entry points of libgbsa: validation, launch planning and kernel launches.
//
// Mirrors the two-stage interface of the GenericBlockSparseAttention article (cf-1.com):
// "two-stage call" (metadata operator, then the main operator), "aclnn API" (first stage
// validates and sizes the workspace, second stage executes on a stream), "general
// constraints" (D = 128, 128-token pages equal to blockShapeY, N1 % N2 == 0, group <= 128,
// topK <= 256, empty tensors rejected, tensor values not checked at this stage), "mask" and
// "quantisation" (mask 1 = causal; quant 0 or 5; scales only with quant 5).
#include <math.h>
#include <mutex>
#include <string.h>

#include "gbsa.h"
#include "gbsa_internal.hpp"

using namespace gbsa;

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int g_cus[kMaxDevices] = {0};

gbsa_status device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GBSA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GBSA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            return GBSA_ERR_HIP;
        g_cus[dev] = n;
    }
    *cus = g_cus[dev];
    return GBSA_OK;
}

int64_t rows_per_unit(const gbsa_params* p) {
    return (int64_t)p->block_x * (p->num_heads_q / p->num_heads_kv);
}

gbsa_status plan_workers(const gbsa_params* p, int* P_out) {
    if (p->num_workers > 0) {
        *P_out = p->num_workers;
        return GBSA_OK;
    }
    int cus = 0;
    gbsa_status st = device_cus(&cus);
    if (st != GBSA_OK) return st;
    const int64_t M = rows_per_unit(p);
    int64_t P;
    if (M <= kDecodeMaxRows) {
        // one decode workgroup per CU: on the gather-bound decode shapes this beat two per CU
        // (fewer, longer gather streams; 3 % on 64 x 16 pages, 12-20 % on the split shapes)
        P = (int64_t)cus;
    } else {
        const int rows = prefill_rows_per_wg((int)M);
        const int64_t nst = (M + rows - 1) / rows;
        P = (2 * (int64_t)cus + nst - 1) / nst;
    }
    if (P < 1) P = 1;
    if (P > kMaxWorkers) P = kMaxWorkers;
    *P_out = (int)P;
    return GBSA_OK;
}

void fill_fingerprint(const gbsa_params* p, int32_t* h) {
    h[7] = p->num_heads_q;
    h[8] = p->num_heads_kv;
    h[9] = p->head_dim;
    h[10] = p->block_x;
    h[11] = p->block_y;
    h[12] = p->top_k;
    h[13] = p->mask_mode;
    h[14] = p->quant_mode;
    h[15] = p->total_q_blocks;
    h[16] = p->batch;
    h[17] = p->win_left;
    h[18] = p->win_right;
    h[19] = p->has_seqused_q;
    h[20] = p->is_packed_gqa;
    h[21] = p->kv_layout;
}

}  // namespace

extern "C" {

gbsa_status gbsa_check_params(const gbsa_params* p) {
    if (p == nullptr) return GBSA_ERR_NULL;
    if (p->kv_layout != GBSA_KV_PA_BBND && p->kv_layout != GBSA_KV_TND)
        return GBSA_ERR_UNSUPPORTED;
    const bool tnd = p->kv_layout == GBSA_KV_TND;
    if (p->batch == 0 || p->num_heads_q == 0 || p->num_heads_kv == 0 || p->head_dim == 0 ||
        p->total_q == 0 || p->total_q_blocks == 0 || p->top_k == 0 || p->block_x == 0 ||
        (!tnd && p->max_blocks_per_seq == 0) || p->num_pages == 0)
        return GBSA_ERR_EMPTY;
    if (p->batch < 0 || p->num_heads_q < 0 || p->num_heads_kv < 0 || p->total_q < 0 ||
        p->total_q_blocks < 0 || p->top_k < 0 || p->block_x < 0 || p->max_blocks_per_seq < 0 ||
        p->num_pages < 0)
        return GBSA_ERR_SHAPE;
    if (p->head_dim != GBSA_HEAD_DIM) return GBSA_ERR_SHAPE;
    if (p->block_y != GBSA_PAGE_SIZE || p->page_size != GBSA_PAGE_SIZE) return GBSA_ERR_SHAPE;
    if (p->num_heads_q % p->num_heads_kv != 0) return GBSA_ERR_SHAPE;
    if (p->num_heads_q / p->num_heads_kv > GBSA_MAX_GROUP) return GBSA_ERR_SHAPE;
    if (p->top_k > GBSA_MAX_TOPK) return GBSA_ERR_SHAPE;
    if (p->win_left < -1 || p->win_right < -1) return GBSA_ERR_SHAPE;
    if (p->num_workers < 0 || p->num_workers > GBSA_MAX_WORKERS) return GBSA_ERR_SHAPE;
    const int64_t page_elems = (int64_t)GBSA_PAGE_SIZE * p->num_heads_kv * p->head_dim;
    if (tnd) {
        // rows are dense; the last block of a sequence must start at an int32 row
        if (p->kv_page_stride != 0 || p->num_pages > GBSA_MAX_KV_ROWS) return GBSA_ERR_SHAPE;
    } else if (p->kv_page_stride != 0 &&
               (p->kv_page_stride < page_elems ||
                p->kv_page_stride % ((int64_t)p->num_heads_kv * p->head_dim) != 0)) {
        return GBSA_ERR_SHAPE;
    }
    if (p->batch > GBSA_MAX_BATCH) return GBSA_ERR_UNSUPPORTED;
    if ((int64_t)p->num_heads_kv * p->total_q_blocks >= kMaxUnits) return GBSA_ERR_UNSUPPORTED;
    if (p->dtype < GBSA_DTYPE_F16 || p->dtype > GBSA_DTYPE_FP8_E4M3) return GBSA_ERR_DTYPE;
    if (p->out_dtype != GBSA_DTYPE_F16 && p->out_dtype != GBSA_DTYPE_BF16) return GBSA_ERR_DTYPE;
    if (p->quant_mode != GBSA_QUANT_NONE && p->quant_mode != GBSA_QUANT_FP8_E4M3)
        return GBSA_ERR_UNSUPPORTED;
    if (p->quant_mode == GBSA_QUANT_FP8_E4M3) {
        if (p->dtype != GBSA_DTYPE_FP8_E4M3) return GBSA_ERR_DTYPE;
    } else {
        if (p->dtype == GBSA_DTYPE_FP8_E4M3) return GBSA_ERR_DTYPE;
        if (p->out_dtype != p->dtype) return GBSA_ERR_DTYPE;
    }
    if (p->mask_mode != GBSA_MASK_NONE && p->mask_mode != GBSA_MASK_CAUSAL &&
        p->mask_mode != GBSA_MASK_CAUSAL_TOP_LEFT)
        return GBSA_ERR_UNSUPPORTED;
    if (p->softmax_precision != 0 && p->softmax_precision != 1) return GBSA_ERR_UNSUPPORTED;
    if (p->is_packed_gqa != 1) return GBSA_ERR_UNSUPPORTED;
    if (p->has_seqused_q != 0 && p->has_seqused_q != 1) return GBSA_ERR_SHAPE;
    if (p->return_lse != 0 && p->return_lse != 1) return GBSA_ERR_SHAPE;
    if (!(p->dst_type_max >= 0.f) || p->dst_type_max > 3.0e38f) return GBSA_ERR_UNSUPPORTED;
    // max_seqlen_q / max_seqlen_kv: -1 or 0 = not given; a given bound must fit the storage
    if (p->max_seqlen_q < -1 || p->max_seqlen_kv < -1) return GBSA_ERR_SHAPE;
    if (p->max_seqlen_q > p->total_q) return GBSA_ERR_SHAPE;
    if (p->max_seqlen_kv > (tnd ? p->num_pages : (int64_t)p->max_blocks_per_seq * GBSA_PAGE_SIZE))
        return GBSA_ERR_SHAPE;
    if (!(p->scale == p->scale)) return GBSA_ERR_SHAPE;  // NaN
    return GBSA_OK;
}

gbsa_status gbsa_num_workers(const gbsa_params* p, int32_t* num_workers) {
    gbsa_status st = gbsa_check_params(p);
    if (st != GBSA_OK) return st;
    if (num_workers == nullptr) return GBSA_ERR_NULL;
    int P = 0;
    st = plan_workers(p, &P);
    if (st != GBSA_OK) return st;
    *num_workers = P;
    return GBSA_OK;
}

gbsa_status gbsa_workspace_size(const gbsa_params* p, size_t* bytes) {
    gbsa_status st = gbsa_check_params(p);
    if (st != GBSA_OK) return st;
    if (bytes == nullptr) return GBSA_ERR_NULL;
    int P = 0;
    st = plan_workers(p, &P);
    if (st != GBSA_OK) return st;
    const int64_t M = rows_per_unit(p);
    *bytes = ws_layout(P, M, subtiles(M)).total;
    return GBSA_OK;
}

gbsa_status gbsa_metadata(const gbsa_params* p, const int32_t* sparse_block_count,
                          const int64_t* cu_seqlens_q, const int32_t* seqused_q,
                          const int32_t* seqused_kv, int32_t* metadata, hipStream_t stream) {
    gbsa_status st = gbsa_check_params(p);
    if (st != GBSA_OK) return st;
    if (sparse_block_count == nullptr || cu_seqlens_q == nullptr) return GBSA_ERR_NULL;
    // "general constraints": PA_BBND requires seqused_kv; with TND it is optional
    if (p->kv_layout == GBSA_KV_PA_BBND && seqused_kv == nullptr) return GBSA_ERR_NULL;
    if ((seqused_q != nullptr) != (p->has_seqused_q == 1)) return GBSA_ERR_NULL;
    if (metadata == nullptr) return GBSA_ERR_METADATA;
    int P = 0;
    st = plan_workers(p, &P);
    if (st != GBSA_OK) return st;
    MetaArgs a;
    memset(&a, 0, sizeof(a));
    a.count = sparse_block_count;
    a.cu = cu_seqlens_q;
    a.squ = seqused_q;
    a.meta = metadata;
    a.B = p->batch;
    a.N2 = p->num_heads_kv;
    a.X = p->block_x;
    a.topK = p->top_k;
    a.tqb = p->total_q_blocks;
    a.P = P;
    {
        // the chunked scheduler's dynamic LDS: two per-sequence tables and the cached counts,
        // next to its own static shared variables (kMetaStaticLds bytes at most)
        const int64_t lds_cap = (160 * 1024 - kMetaStaticLds) / (int64_t)sizeof(int) -
                                2 * ((int64_t)p->batch + 1);
        int64_t ucap = (int64_t)p->num_heads_kv * p->total_q_blocks;
        if (ucap > 16384) ucap = 16384;
        if (ucap > lds_cap) ucap = lds_cap;
        a.ucap = (int32_t)(ucap > 0 ? ucap : 0);
    }
    fill_fingerprint(p, a.header);
    return launch_metadata(a, stream) == hipSuccess ? GBSA_OK : GBSA_ERR_HIP;
}

// ---------------------------------------------------------------------------------------
// Allocation-free variant: the workspace is a fixed device array of the library. Its layout
// does not depend on the call (the arrival counters have a region of their own), so a call
// never finds another call's partial results where it expects zeroed counters.
// ---------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)GBSA_NOALLOC_SCRATCH_BYTES;
constexpr int64_t kScratchCounters = GBSA_NOALLOC_MAX_COUNTERS;
constexpr size_t kScratchCounterBytes = sizeof(int32_t) * (size_t)kScratchCounters;

static __device__ __align__(256) unsigned char scratch[GBSA_NOALLOC_SCRATCH_BYTES];

// scratch: [status word][arrival counters, fixed region][partial O][running max][running sum]
static WsLayout scratch_layout(int64_t P, int64_t M) {
    WsLayout w;
    w.status = 0;
    w.arrive = 256;
    w.o = align_up(w.arrive + kScratchCounterBytes, 256);
    w.m = align_up(w.o + sizeof(float) * 2 * P * M * 128, 256);
    w.l = align_up(w.m + sizeof(float) * 2 * P * M, 256);
    w.total = align_up(w.l + sizeof(float) * 2 * P * M, 256);
    return w;
}

namespace {
// Zeroes `n` words (the status word and the counter region) once per device.
__global__ void clear_words_kernel(int32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0;
}

std::mutex g_scratch_mu;
unsigned char* g_scratch[kMaxDevices] = {nullptr};
}  // namespace

// Device address of this device's copy of `scratch`, looked up once per device with that
// device current (the array's name is a host-side stand-in, not a device address). The first
// call on a device also clears the status word and the counter region on `stream`, with a
// kernel (capturable) rather than a memset.
static gbsa_status scratch_base(hipStream_t stream, unsigned char** base) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GBSA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return GBSA_ERR_HIP;
        const int words = (int)((256 + kScratchCounterBytes) / sizeof(int32_t));
        hipLaunchKernelGGL(clear_words_kernel, dim3(64), dim3(256), 0, stream, (int32_t*)ptr,
                           words);
        if (hipGetLastError() != hipSuccess) return GBSA_ERR_HIP;
        g_scratch[dev] = (unsigned char*)ptr;
    }
    *base = g_scratch[dev];
    return GBSA_OK;
}

// fixed_ws: false = the caller's workspace (args->workspace), true = the array `scratch`.
static gbsa_status forward_impl(const gbsa_params* p, const gbsa_forward_args* g,
                                hipStream_t stream, const bool fixed_ws = false) {
    const void* query = g->query;
    const void* key = g->key;
    const void* value = g->value;
    const int32_t* sparse_block_idx = g->sparse_block_idx;
    const int32_t* sparse_block_count = g->sparse_block_count;
    const int32_t* metadata = g->metadata;
    const int64_t* cu_seqlens_q = g->cu_seqlens_q;
    const int32_t* seqused_q = g->seqused_q;
    const int32_t* seqused_kv = g->seqused_kv;
    const int32_t* block_table = g->block_table;
    const int64_t* cu_seqlens_kv = g->cu_seqlens_kv;
    const float* q_scale = g->q_scale;
    const float* k_scale = g->k_scale;
    const float* v_scale = g->v_scale;
    const float* p_scale = g->p_scale;
    void* attention_out = g->attention_out;
    float* softmax_lse = g->softmax_lse;
    void* workspace = g->workspace;
    const size_t workspace_bytes = g->workspace_bytes;
    gbsa_status st = gbsa_check_params(p);
    if (st != GBSA_OK) return st;
    const bool tnd = p->kv_layout == GBSA_KV_TND;
    if (query == nullptr || key == nullptr || value == nullptr || sparse_block_idx == nullptr ||
        sparse_block_count == nullptr || cu_seqlens_q == nullptr || attention_out == nullptr)
        return GBSA_ERR_NULL;
    if (tnd ? cu_seqlens_kv == nullptr : (seqused_kv == nullptr || block_table == nullptr))
        return GBSA_ERR_NULL;
    if ((seqused_q != nullptr) != (p->has_seqused_q == 1)) return GBSA_ERR_NULL;
    if ((softmax_lse != nullptr) != (p->return_lse == 1)) return GBSA_ERR_NULL;
    if (metadata == nullptr) return GBSA_ERR_METADATA;
    const bool quant = p->quant_mode == GBSA_QUANT_FP8_E4M3;
    if (quant && (q_scale == nullptr || k_scale == nullptr || v_scale == nullptr))
        return GBSA_ERR_DTYPE;
    if (!quant && (q_scale != nullptr || k_scale != nullptr || v_scale != nullptr))
        return GBSA_ERR_DTYPE;
    if (p_scale != nullptr && !quant) return GBSA_ERR_DTYPE;
    if (g->atten_mask != nullptr) {
        const int64_t rs = g->mask_row_stride, bs = g->mask_batch_stride;
        if (((uintptr_t)g->atten_mask & 3) != 0 || g->mask_rows < 0 || g->mask_cols < 0 ||
            rs < g->mask_cols || rs % 4 != 0 || bs < 0 || bs % 4 != 0 ||
            (int64_t)g->mask_rows * rs > 0x7fffffff)
            return GBSA_ERR_SHAPE;
    }
    int P = 0;
    st = plan_workers(p, &P);
    if (st != GBSA_OK) return st;
    const int64_t M = rows_per_unit(p);
    WsLayout L;
    unsigned char* ws = (unsigned char*)workspace;
    if (fixed_ws) {
        // the caller brings no workspace; the shapes must fit the fixed array
        if (workspace != nullptr || workspace_bytes != 0) return GBSA_ERR_WORKSPACE;
        L = scratch_layout(P, M);
        if ((int64_t)P * subtiles(M) > kScratchCounters || L.total > kScratchBytes)
            return GBSA_ERR_WORKSPACE;
        st = scratch_base(stream, &ws);
        if (st != GBSA_OK) return st;
    } else {
        L = ws_layout(P, M, subtiles(M));
        if (workspace == nullptr || workspace_bytes < L.total) return GBSA_ERR_WORKSPACE;
    }

    FwdArgs a;
    memset(&a, 0, sizeof(a));
    a.q = query;
    a.k = key;
    a.v = value;
    a.idx = sparse_block_idx;
    a.cnt = sparse_block_count;
    a.meta = metadata;
    a.cu = cu_seqlens_q;
    a.squ = seqused_q;
    a.skv = seqused_kv;
    a.table = tnd ? nullptr : block_table;
    a.cu_kv = tnd ? cu_seqlens_kv : nullptr;
    a.qs = q_scale;
    a.ks = k_scale;
    a.vs = v_scale;
    a.out = attention_out;
    if (g->atten_mask != nullptr) {
        a.umask = g->atten_mask;
        a.um_bstride = g->mask_batch_stride;
        a.um_rstride = (int32_t)g->mask_row_stride;
        a.um_rows = g->mask_rows;
        a.um_cols = g->mask_cols;
    }
    a.lse = softmax_lse;
    a.ws_status = (int32_t*)(ws + L.status);
    a.ws_arrive = (int32_t*)(ws + L.arrive);
    a.ws_queue = a.ws_status + 16;  // the rest of the zero-filled status page
    a.ws_o = (float*)(ws + L.o);
    a.ws_m = (float*)(ws + L.m);
    a.ws_l = (float*)(ws + L.l);
    const int64_t row_elems = (int64_t)p->num_heads_kv * p->head_dim;
    if (tnd) {
        a.kv_stride = row_elems;  // a storage unit is one token row
        a.kv_rows = p->num_pages;
    } else {
        a.kv_stride = p->kv_page_stride != 0 ? p->kv_page_stride : GBSA_PAGE_SIZE * row_elems;
    }
    a.B = p->batch;
    a.N1 = p->num_heads_q;
    a.N2 = p->num_heads_kv;
    a.G = p->num_heads_q / p->num_heads_kv;
    a.X = p->block_x;
    a.topK = p->top_k;
    a.tqb = p->total_q_blocks;
    a.maxb = p->max_blocks_per_seq;
    a.P = P;
    a.M = (int32_t)M;
    a.mask = p->mask_mode;
    a.wl = p->win_left;
    a.wr = p->win_right;
    a.return_lse = p->return_lse;
    a.half_softmax = p->softmax_precision == 1 && p->dtype == GBSA_DTYPE_F16;
    a.ps = p_scale;
    a.ps_max = (p->dst_type_max > 0.f && p->dst_type_max < 448.f) ? p->dst_type_max : 448.f;
    const double scale = p->scale > 0.f ? (double)p->scale : 1.0 / sqrt((double)p->head_dim);
    a.scale_log2 = (float)(scale * 1.4426950408889634);
    a.T = p->total_q;
    a.out_nan2 = p->out_dtype == GBSA_DTYPE_F16 ? 0x7e007e00u : 0x7fc07fc0u;
    a.expect[0] = (int32_t)kMagic;
    a.expect[1] = kVersion;
    a.expect[2] = P;
    fill_fingerprint(p, a.expect);

    a.nst = (int32_t)subtiles(M);
    int cus = 0;
    st = device_cus(&cus);
    if (st != GBSA_OK) return st;
    a.cus = cus;
    hipError_t e;
    if (M <= kDecodeMaxRows)
        e = launch_decode(a, p->dtype, p->out_dtype, stream);
    else
        e = launch_prefill(a, p->dtype, p->out_dtype, prefill_rows_per_wg((int)M), stream);
    return e == hipSuccess ? GBSA_OK : GBSA_ERR_HIP;
}

gbsa_status gbsa_forward(const gbsa_params* p, const void* query, const void* key,
                         const void* value, const int32_t* sparse_block_idx,
                         const int32_t* sparse_block_count, const int32_t* metadata,
                         const int64_t* cu_seqlens_q, const int32_t* seqused_q,
                         const int32_t* seqused_kv, const int32_t* block_table,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         const float* p_scale, void* attention_out, float* softmax_lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    gbsa_status st = gbsa_check_params(p);
    if (st != GBSA_OK) return st;
    if (p->kv_layout != GBSA_KV_PA_BBND) return GBSA_ERR_UNSUPPORTED;
    gbsa_forward_args g;
    memset(&g, 0, sizeof(g));
    g.query = query;
    g.key = key;
    g.value = value;
    g.sparse_block_idx = sparse_block_idx;
    g.sparse_block_count = sparse_block_count;
    g.metadata = metadata;
    g.cu_seqlens_q = cu_seqlens_q;
    g.seqused_q = seqused_q;
    g.seqused_kv = seqused_kv;
    g.block_table = block_table;
    g.q_scale = q_scale;
    g.k_scale = k_scale;
    g.v_scale = v_scale;
    g.p_scale = p_scale;
    g.attention_out = attention_out;
    g.softmax_lse = softmax_lse;
    g.workspace = workspace;
    g.workspace_bytes = workspace_bytes;
    return forward_impl(p, &g, stream);
}

gbsa_status gbsa_forward_tnd(const gbsa_params* p, const void* query, const void* key,
                             const void* value, const int32_t* sparse_block_idx,
                             const int32_t* sparse_block_count, const int32_t* metadata,
                             const int64_t* cu_seqlens_q, const int32_t* seqused_q,
                             const int64_t* cu_seqlens_kv, const int32_t* seqused_kv,
                             const float* q_scale, const float* k_scale, const float* v_scale,
                             const float* p_scale, void* attention_out, float* softmax_lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    gbsa_status st = gbsa_check_params(p);
    if (st != GBSA_OK) return st;
    if (p->kv_layout != GBSA_KV_TND) return GBSA_ERR_UNSUPPORTED;
    gbsa_forward_args g;
    memset(&g, 0, sizeof(g));
    g.query = query;
    g.key = key;
    g.value = value;
    g.sparse_block_idx = sparse_block_idx;
    g.sparse_block_count = sparse_block_count;
    g.metadata = metadata;
    g.cu_seqlens_q = cu_seqlens_q;
    g.seqused_q = seqused_q;
    g.cu_seqlens_kv = cu_seqlens_kv;
    g.seqused_kv = seqused_kv;
    g.q_scale = q_scale;
    g.k_scale = k_scale;
    g.v_scale = v_scale;
    g.p_scale = p_scale;
    g.attention_out = attention_out;
    g.softmax_lse = softmax_lse;
    g.workspace = workspace;
    g.workspace_bytes = workspace_bytes;
    return forward_impl(p, &g, stream);
}

gbsa_status gbsa_forward_ex(const gbsa_params* p, const gbsa_forward_args* args,
                            hipStream_t stream) {
    gbsa_status st = gbsa_check_params(p);
    if (st != GBSA_OK) return st;
    if (args == nullptr) return GBSA_ERR_NULL;
    // the layout not in use takes no tensors
    if (p->kv_layout == GBSA_KV_TND ? args->block_table != nullptr
                                    : args->cu_seqlens_kv != nullptr)
        return GBSA_ERR_NULL;
    return forward_impl(p, args, stream);
}

gbsa_status gbsa_forward_ex_noalloc(const gbsa_params* p, const gbsa_forward_args* args,
                                    hipStream_t stream) {
    gbsa_status st = gbsa_check_params(p);
    if (st != GBSA_OK) return st;
    if (args == nullptr) return GBSA_ERR_NULL;
    if (p->kv_layout == GBSA_KV_TND ? args->block_table != nullptr
                                    : args->cu_seqlens_kv != nullptr)
        return GBSA_ERR_NULL;
    return forward_impl(p, args, stream, true);
}

gbsa_status gbsa_validate(const gbsa_params* p, const gbsa_forward_args* g,
                          int32_t* violations, hipStream_t stream) {
    gbsa_status st = gbsa_check_params(p);
    if (st != GBSA_OK) return st;
    if (g == nullptr || violations == nullptr) return GBSA_ERR_NULL;
    const bool tnd = p->kv_layout == GBSA_KV_TND;
    if (g->sparse_block_idx == nullptr || g->sparse_block_count == nullptr ||
        g->cu_seqlens_q == nullptr)
        return GBSA_ERR_NULL;
    if (tnd ? (g->cu_seqlens_kv == nullptr || g->block_table != nullptr)
            : (g->seqused_kv == nullptr || g->block_table == nullptr || g->cu_seqlens_kv != nullptr))
        return GBSA_ERR_NULL;
    if ((g->seqused_q != nullptr) != (p->has_seqused_q == 1)) return GBSA_ERR_NULL;
    ValArgs a;
    memset(&a, 0, sizeof(a));
    a.cu = g->cu_seqlens_q;
    a.squ = g->seqused_q;
    a.skv = g->seqused_kv;
    a.cu_kv = tnd ? g->cu_seqlens_kv : nullptr;
    a.table = tnd ? nullptr : g->block_table;
    a.cnt = g->sparse_block_count;
    a.idx = g->sparse_block_idx;
    a.umask = g->atten_mask;
    a.out = violations;
    a.total_q = p->total_q;
    a.num_pages = p->num_pages;
    a.kv_rows = tnd ? p->num_pages : 0;
    a.B = p->batch;
    a.N2 = p->num_heads_kv;
    a.X = p->block_x;
    a.tqb = p->total_q_blocks;
    a.topK = p->top_k;
    a.maxb = tnd ? 0 : p->max_blocks_per_seq;
    a.um_rows = g->atten_mask != nullptr ? g->mask_rows : 0;
    a.um_cols = g->atten_mask != nullptr ? g->mask_cols : 0;
    a.max_sq = p->max_seqlen_q > 0 ? p->max_seqlen_q : 0;
    a.max_skv = p->max_seqlen_kv > 0 ? p->max_seqlen_kv : 0;
    return launch_validate(a, stream) == hipSuccess ? GBSA_OK : GBSA_ERR_HIP;
}

const char* gbsa_status_string(gbsa_status s) {
    switch (s) {
        case GBSA_OK: return "ok";
        case GBSA_ERR_NULL: return "a required pointer is NULL (or an optional one is inconsistent with its flag)";
        case GBSA_ERR_SHAPE: return "a dimension violates a constraint (D=128, page=blockShapeY=128, N1%N2==0, group<=128, topK<=256, strides)";
        case GBSA_ERR_DTYPE: return "unsupported or inconsistent data type or dequant scales";
        case GBSA_ERR_UNSUPPORTED: return "attribute value not supported (mask/quant mode, packed GQA, KV layout or entry point, batch or unit count limits)";
        case GBSA_ERR_EMPTY: return "a required tensor has an empty axis";
        case GBSA_ERR_WORKSPACE: return "workspace missing or smaller than gbsa_workspace_size";
        case GBSA_ERR_METADATA: return "metadata buffer missing";
        case GBSA_ERR_HIP: return "HIP runtime error (device query or kernel launch)";
    }
    return "unknown status";
}

}  // extern "C"
