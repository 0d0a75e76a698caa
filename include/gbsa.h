/*
 * gbsa.h -- block-sparse flash attention over a paged KV cache, for AMD MI355X (gfx950).
 *
 * The operation is the one the GenericBlockSparseAttention article (cf-1.com, CANN
 * ops-transformer GBSA) defines in its "sparse attention mechanism" section:
 *
 *     attention_out = softmax(scale * Q * K_sparse^T + mask) * V_sparse
 *
 * where every Q block of blockShapeX query rows attends only to the 128-token KV blocks
 * that sparse_block_idx / sparse_block_count select for it from a paged KV cache, and the
 * query heads of one KV head share that selection (packed GQA).
 *
 * The interface mirrors the article's two-stage problem statement ("two-stage call"
 * section): gbsa_metadata() first writes the load-balanced task split into a fixed
 * (1024,) int32 buffer; gbsa_forward() consumes it. As in the article's aclnn interface,
 * the main call's workspace size is queried from shapes alone (gbsa_workspace_size).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library never
 *    allocates, frees or synchronises; work is enqueued on `stream` and completes in
 *    stream order. Inputs are only read; outputs and the workspace are written.
 *  - Arguments are validated on the host before any device work; on error nothing is
 *    enqueued and a gbsa_status other than GBSA_OK is returned. Tensor VALUES (lengths,
 *    indices, page-table entries) are not validated on the host ("general constraints":
 *    tiling never reads tensor values); see gbsa_forward for how the kernels treat them.
 *  - Layouts: query TND [T, N1, D] dense; key/value PA_BBND [num_pages, 128, N2, D] where
 *    only the page axis may be strided (kv_page_stride elements between pages), or, with
 *    kv_layout = GBSA_KV_TND (gbsa_forward_tnd), token-major TND [T_kv, N2, D] dense;
 *    sparse_block_idx [N2, total_q_blocks, top_k] and sparse_block_count
 *    [N2, total_q_blocks] dense int32; block_table [B, max_blocks_per_seq] dense int32;
 *    cu_seqlens_q [B+1] int64; seqused_q / seqused_kv [B] int32; attention_out [T, N1, D];
 *    softmax_lse [T, N1] float32 (the article's (T, N1, 1)).
 *  - Thread safety: calls may be made concurrently from several host threads. Two calls
 *    that share a workspace or metadata buffer must be ordered by the caller.
 */
#ifndef GBSA_H_
#define GBSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed metadata size ("two-stage call": a (1024,) int32 tensor). */
#define GBSA_METADATA_SIZE 1024
/* Only D = 128 and 128-token KV pages equal to blockShapeY ("general constraints"). */
#define GBSA_HEAD_DIM 128
#define GBSA_PAGE_SIZE 128
/* topK upper bound and GQA group bound ("general constraints"). */
#define GBSA_MAX_TOPK 256
#define GBSA_MAX_GROUP 128
/* Largest worker count the metadata buffer can describe (24 header words + P+1 bounds). */
#define GBSA_MAX_WORKERS 999
/* Largest batch the scheduler kernel accepts (it keeps two per-sequence tables in LDS). */
#define GBSA_MAX_BATCH 16384

typedef enum gbsa_status {
    GBSA_OK = 0,
    GBSA_ERR_NULL = 1,        /* a required pointer is NULL */
    GBSA_ERR_SHAPE = 2,       /* a dimension violates a constraint */
    GBSA_ERR_DTYPE = 3,       /* unsupported or inconsistent data type */
    GBSA_ERR_UNSUPPORTED = 4, /* attribute value the article lists as unsupported */
    GBSA_ERR_EMPTY = 5,       /* a required tensor has a zero-length axis */
    GBSA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than gbsa_workspace_size */
    GBSA_ERR_METADATA = 7,    /* metadata buffer missing */
    GBSA_ERR_HIP = 8          /* a HIP runtime call failed (device query, launch) */
} gbsa_status;

typedef enum gbsa_dtype {
    GBSA_DTYPE_F16 = 0,
    GBSA_DTYPE_BF16 = 1,
    GBSA_DTYPE_FP8_E4M3 = 2   /* OCP e4m3fn, the article's FP8 E4M3 full-quant path */
} gbsa_dtype;

/* "mask" section: 1 = the built-in causal mask (aligned to the bottom-right corner when query
 * and key lengths differ). 0 = no mask. 2 = causal aligned to the top-left corner (keys
 * p <= t), an addition to the article's single mask type. */
typedef enum gbsa_mask_mode {
    GBSA_MASK_NONE = 0,
    GBSA_MASK_CAUSAL = 1,
    GBSA_MASK_CAUSAL_TOP_LEFT = 2
} gbsa_mask_mode;

/* Key/value layouts ("parameters" section: layoutKv). PA_BBND pages are located through
 * block_table; TND rows through cu_seqlens_kv ("general constraints": dual lengths, which
 * apply to the KV side when layoutKv is TND). */
typedef enum gbsa_kv_layout { GBSA_KV_PA_BBND = 0, GBSA_KV_TND = 1 } gbsa_kv_layout;
/* Rows a TND key/value tensor may hold: the last block of a sequence must start below 2^31. */
#define GBSA_MAX_KV_ROWS 2147483520LL

/* "quantisation" section: 0 NO_QUANT, 5 FP8_E4M3_STATIC_CAST_P (1..4 are rejected). */
typedef enum gbsa_quant_mode { GBSA_QUANT_NONE = 0, GBSA_QUANT_FP8_E4M3 = 5 } gbsa_quant_mode;

/*
 * Shapes and attributes shared by both stages. The article's "parameters" section gives
 * the defaults: block_shape [1, 128], is_packed_gqa 1, layout TND / PA_BBND, scale 0.0,
 * win_left = win_right = -1. Both calls must receive identical values ("general
 * constraints": metadata and main call must agree); gbsa_forward checks the metadata's
 * fingerprint and refuses to compute on a mismatch (see gbsa_forward).
 */
typedef struct gbsa_params {
    int32_t batch;              /* B >= 1, <= GBSA_MAX_BATCH */
    int32_t num_heads_q;        /* N1 */
    int32_t num_heads_kv;       /* N2; N1 % N2 == 0 and N1 / N2 <= 128 */
    int32_t head_dim;           /* D; must be 128 */
    int64_t total_q;            /* T, rows of query and attention_out */
    int32_t total_q_blocks;     /* dim 1 of sparse_block_idx/count = sum ceil(storage_b / X) */
    int32_t top_k;              /* dim 2 of sparse_block_idx, 1..256 */
    int32_t block_x;            /* blockShapeX >= 1 (query rows per Q block) */
    int32_t block_y;            /* blockShapeY; must be 128 */
    int32_t page_size;          /* KV page size; must be 128 */
    int32_t max_blocks_per_seq; /* dim 1 of block_table (PA_BBND; not read with TND) */
    int64_t num_pages;          /* dim 0 of key/value: pages (PA_BBND) or rows T_kv (TND,
                                   at most GBSA_MAX_KV_ROWS) */
    int64_t kv_page_stride;     /* PA_BBND: elements between pages; 0 = dense (128*N2*D);
                                   else >= 128*N2*D and a multiple of N2*D. TND: must be 0 */
    int32_t dtype;              /* gbsa_dtype of query/key/value (must match) */
    int32_t out_dtype;          /* gbsa_dtype of attention_out: F16 or BF16. With quant 0 it
                                   must equal dtype; with quant 5 it is required */
    int32_t mask_mode;          /* gbsa_mask_mode */
    int32_t win_left;           /* -1 unbounded, else keys p >= t + off - win_left (off: see
                                   gbsa_forward; 0 with GBSA_MASK_CAUSAL_TOP_LEFT) */
    int32_t win_right;          /* -1 unbounded, else keys p <= t + off + win_right */
    int32_t quant_mode;         /* gbsa_quant_mode; 5 requires dtype FP8_E4M3 */
    int32_t softmax_precision;  /* 0: fp32 online softmax; 1 ("softmax precision" section):
                                   with f16, the online-softmax stage of the kernels for more
                                   than 64 rows per unit runs in f16 (rescale and row sums in
                                   fp32); bf16, fp8 and the other kernels compute it in fp32 */
    int32_t return_lse;         /* 1: write softmax_lse */
    int32_t is_packed_gqa;      /* must be 1 */
    int32_t has_seqused_q;      /* 1: seqused_q is passed to both calls */
    float scale;                /* softmax scale; <= 0 means 1/sqrt(D) */
    int32_t num_workers;        /* 0 = chosen by the library from the shapes, else 1..999 */
    int32_t kv_layout;          /* gbsa_kv_layout: GBSA_KV_PA_BBND (gbsa_forward) or
                                   GBSA_KV_TND (gbsa_forward_tnd) */
    int32_t max_seqlen_q;       /* -1 or 0: not given (the article's default -1). Else an
                                   upper bound on every sequence's query storage length
                                   (cu_seqlens_q[b+1] - cu_seqlens_q[b]); at most total_q */
    int32_t max_seqlen_kv;      /* -1 or 0: not given. Else an upper bound on every
                                   sequence's visible KV length (seqused_kv, or the TND
                                   storage length without it); at most what the KV storage
                                   holds (max_blocks_per_seq * 128, or T_kv with TND).
                                   Both bounds are the metadata operator's max_seqlen_q /
                                   max_seqlen_kv ("PyTorch API" section); the kernels need
                                   neither, gbsa_validate checks them against the tensors */
    float dst_type_max;         /* quant 5 with p_scale: the largest value P * p_scale may take
                                   before P is cast to e4m3 ("aclnn API" section's dstTypeMax);
                                   0 = the type's max, 448; larger values are taken as 448.
                                   Must be finite and >= 0 */
} gbsa_params;

/*
 * Check a parameter block without touching any device. Returns the status that
 * gbsa_metadata / gbsa_forward would return for these attributes.
 */
gbsa_status gbsa_check_params(const gbsa_params* params);

/*
 * Number of workers (task-split segments) the two calls will use on the current device:
 * params->num_workers if set, else one per compute unit for units of at most 16 packed rows
 * (decode shapes) and two per compute unit divided by the workgroups per unit otherwise
 * (at most GBSA_MAX_WORKERS). Depends only on the shapes and the device's compute-unit count.
 * Errors: any gbsa_check_params error; GBSA_ERR_HIP when the device cannot be queried.
 */
gbsa_status gbsa_num_workers(const gbsa_params* params, int32_t* num_workers);

/*
 * Stage 1 ("two-stage call" section; the article's metadata operator).
 * Enqueues the scheduler kernel, which writes the task split into `metadata`
 * (GBSA_METADATA_SIZE int32 on the device). Work units are (b, kv head, active q-block)
 * in that order; a q-block is active when it starts below seqused_q[b] (or the storage
 * length cu_seqlens_q[b+1]-cu_seqlens_q[b] when seqused_q is NULL) ("general constraints":
 * the task space follows seqused). Unit cost = clamp(count, 0, top_k) + 1; the units' kv
 * slots are split into num_workers contiguous segments of equal cost.
 *   sparse_block_count  [N2, total_q_blocks] int32, device
 *   cu_seqlens_q        [B+1] int64, device (storage lengths of the TND query)
 *   seqused_q           [B] int32, device, or NULL (must be non-NULL iff has_seqused_q)
 *   seqused_kv          [B] int32, device: required with PA_BBND, optional (NULL) with TND;
 *                       not read here (the task split does not depend on KV lengths)
 *   metadata            [1024] int32, device, written
 * Errors: gbsa_check_params errors; GBSA_ERR_NULL; GBSA_ERR_METADATA (metadata NULL);
 * GBSA_ERR_HIP on a failed launch.
 */
gbsa_status gbsa_metadata(const gbsa_params* params, const int32_t* sparse_block_count,
                          const int64_t* cu_seqlens_q, const int32_t* seqused_q,
                          const int32_t* seqused_kv, int32_t* metadata, hipStream_t stream);

/*
 * Workspace bytes gbsa_forward needs, from shapes only (the aclnn GetWorkspaceSize
 * stage). It holds a status word, the counters from which the prefill workgroups take their
 * tasks, per-worker split-KV partial results (O, running max, running sum) and the arrival
 * counters of split units.
 * A workspace must be zero-filled before its first use (e.g. hipMemsetAsync to 0). Every
 * call leaves its task and arrival counters at zero again, so later calls with the same
 * worker count and rows per unit (block_x * N1 / N2) can reuse it as it is, in stream order;
 * the counter region grows with both, so after a call with other values zero-fill it again. The status
 * word (word 0) is sticky: once a call sets it, it stays set until the caller clears it.
 */
gbsa_status gbsa_workspace_size(const gbsa_params* params, size_t* bytes);

/*
 * Stage 2 (the main operator, "sparse attention mechanism" formula), PA_BBND key/value
 * (params->kv_layout must be GBSA_KV_PA_BBND).
 *   query        [T, N1, 128]            dtype
 *   key, value   [num_pages, 128, N2, 128] dtype, page axis stride kv_page_stride
 *   sparse_block_idx   [N2, total_q_blocks, top_k] int32: LOGICAL block numbers j of the
 *                      sequence (keys 128*j .. 128*j+127); slots >= count are ignored
 *   sparse_block_count [N2, total_q_blocks] int32 (clamped to [0, top_k])
 *   metadata     written by gbsa_metadata with the same params and inputs
 *   cu_seqlens_q [B+1] int64; seqused_q [B] int32 or NULL; seqused_kv [B] int32
 *   block_table  [B, max_blocks_per_seq] int32: physical page of logical block j
 *   q_scale [N1], k_scale [N2], v_scale [N2] float32 dequant scales: required with quant 5,
 *                must be NULL with quant 0
 *   p_scale [N1] float32 or NULL: quant 5 only ("quantisation" section, FP8_E4M3_STATIC_CAST_P:
 *                the softmax probabilities P of query head h, in [0, 1], are cast to e4m3 after
 *                scaling by min(p_scale[h], dst_type_max) and P·V runs on fp8; O is divided
 *                by the scale again). Used by the kernels for more than 64 rows per unit
 *                without a user mask; the others, and every kernel when p_scale is NULL, keep
 *                P in bf16 (the more precise form of the same result)
 *   attention_out [T, N1, 128] out_dtype; rows t >= seqused_q[b] are not written
 *   softmax_lse   [T, N1] float32 natural-log LSE of the scaled logits, -inf for a row
 *                 with no visible key (whose output row is 0); required iff return_lse
 *   workspace / workspace_bytes: device buffer of at least gbsa_workspace_size bytes
 * Visibility of key position p = 128*j + r from batch-local query row t: p < seqused_kv[b];
 * causal: p <= t + off; window: t + off - win_left <= p <= t + off + win_right, with
 * off = seqused_kv[b] - (seqused_q[b] or the storage length), or off = 0 with
 * GBSA_MASK_CAUSAL_TOP_LEFT (whose causal rule is then p <= t).
 * Values the caller must guarantee (not checked, as in the article): lengths within
 * storage, block_table entries in [0, num_pages) for every selected block below
 * seqused_kv. The kernels skip a slot whose index is negative or whose block starts at or
 * beyond seqused_kv[b], and never read past the selection arrays.
 * If the metadata's magic, worker count or parameter fingerprint do not match these
 * params, the kernels compute nothing: they fill attention_out (all T x N1 x 128 entries)
 * and softmax_lse with NaN and set word 0 of the workspace to a non-zero value (readable by
 * the caller after the stream completes).
 * Errors: gbsa_check_params errors; GBSA_ERR_NULL; GBSA_ERR_METADATA; GBSA_ERR_WORKSPACE;
 * GBSA_ERR_DTYPE (scales inconsistent with quant_mode); GBSA_ERR_UNSUPPORTED (kv_layout is
 * not PA_BBND); GBSA_ERR_HIP on a failed launch.
 */
gbsa_status gbsa_forward(const gbsa_params* params, const void* query, const void* key,
                         const void* value, const int32_t* sparse_block_idx,
                         const int32_t* sparse_block_count, const int32_t* metadata,
                         const int64_t* cu_seqlens_q, const int32_t* seqused_q,
                         const int32_t* seqused_kv, const int32_t* block_table,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         const float* p_scale, void* attention_out, float* softmax_lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Stage 2 with token-major TND key/value (params->kv_layout must be GBSA_KV_TND): the
 * article's layoutKv "TND" with cu_seqlens_kv and the dual-length rule of its "general
 * constraints" section applied to the KV side. Same computation and arguments as
 * gbsa_forward except:
 *   key, value     [T_kv, N2, 128] dtype, dense; T_kv = params->num_pages
 *   cu_seqlens_kv  [B+1] int64: sequence b owns rows cu_seqlens_kv[b] .. cu_seqlens_kv[b+1]-1
 *                  (its KV storage length); logical block j is rows cu_seqlens_kv[b] + 128*j
 *                  .. +127 of that sequence
 *   seqused_kv     [B] int32 or NULL: visible KV length of each sequence; NULL means the
 *                  storage length. Values above the storage length are clamped to it.
 * Key position p of sequence b is visible iff p < kv_len[b] (kv_len = seqused_kv or storage)
 * and the mask keeps it, with off = kv_len[b] - (seqused_q[b] or the q storage length).
 * cu_seqlens_kv should be non-decreasing with cu_seqlens_kv[B] <= T_kv; the kernels clamp
 * each sequence's row range into [0, T_kv], so no load leaves the tensor. The rows a block
 * spans past kv_len (the next sequence's, or past the tensor's end) read as zeros without a
 * memory access, as do page-tail rows past seqused_kv in gbsa_forward: cached rows beyond
 * the visible length never reach the output, whatever they hold.
 * Errors: as gbsa_forward; GBSA_ERR_UNSUPPORTED if kv_layout is not TND.
 */
gbsa_status gbsa_forward_tnd(const gbsa_params* params, const void* query, const void* key,
                             const void* value, const int32_t* sparse_block_idx,
                             const int32_t* sparse_block_count, const int32_t* metadata,
                             const int64_t* cu_seqlens_q, const int32_t* seqused_q,
                             const int64_t* cu_seqlens_kv, const int32_t* seqused_kv,
                             const float* q_scale, const float* k_scale, const float* v_scale,
                             const float* p_scale, void* attention_out, float* softmax_lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Every tensor of the main call in one block: the article's aclnn form, one call taking all
 * optional tensors ("aclnn API" section), including the user attention mask it lists as
 * attenMaskOptional. Pointers that do not apply must be NULL.
 */
typedef struct gbsa_forward_args {
    const void* query;                 /* [T, N1, 128] dtype */
    const void* key;                   /* PA_BBND [num_pages, 128, N2, 128] or TND [T_kv, N2, 128] */
    const void* value;                 /* same layout as key */
    const int32_t* sparse_block_idx;   /* [N2, total_q_blocks, top_k] */
    const int32_t* sparse_block_count; /* [N2, total_q_blocks] */
    const int32_t* metadata;           /* [1024] from gbsa_metadata */
    const int64_t* cu_seqlens_q;       /* [B+1] */
    const int32_t* seqused_q;          /* [B] or NULL (must match has_seqused_q) */
    const int64_t* cu_seqlens_kv;      /* [B+1], TND only */
    const int32_t* seqused_kv;         /* [B]: required with PA_BBND, optional with TND */
    const int32_t* block_table;        /* [B, max_blocks_per_seq], PA_BBND only */
    const float* q_scale;              /* dequant scales, quant 5 only (see gbsa_forward) */
    const float* k_scale;
    const float* v_scale;
    const float* p_scale;              /* [N1] or NULL, as in gbsa_forward */
    /* User attention mask, uint8, or NULL. Entry [t][p] nonzero removes key position p for
     * the batch-local query row t of every head of a sequence, on top of every other rule;
     * entries outside rows x cols do not mask. Layout: entry (b, t, p) at byte
     * b * mask_batch_stride + t * mask_row_stride + p (mask_batch_stride 0: one mask shared
     * by all sequences). The base must be 4-byte aligned, mask_row_stride and
     * mask_batch_stride multiples of 4, mask_row_stride >= mask_cols, and one sequence's
     * rows x mask_row_stride below 2^31 (else GBSA_ERR_SHAPE). The fields are ignored when
     * atten_mask is NULL. */
    const uint8_t* atten_mask;
    int64_t mask_batch_stride;
    int64_t mask_row_stride;
    int32_t mask_rows;
    int32_t mask_cols;
    void* attention_out;               /* [T, N1, 128] out_dtype */
    float* softmax_lse;                /* [T, N1] or NULL (must match return_lse) */
    void* workspace;
    size_t workspace_bytes;
} gbsa_forward_args;

/*
 * Stage 2 with every option: either KV layout (params->kv_layout), an optional user
 * attention mask, any mask mode. Same computation, validation and device-side behaviour as
 * gbsa_forward / gbsa_forward_tnd, which are this call with atten_mask NULL.
 * Errors: those of gbsa_forward; GBSA_ERR_NULL if args is NULL; GBSA_ERR_SHAPE for a mask
 * whose alignment, strides or extent break the rules above.
 */
gbsa_status gbsa_forward_ex(const gbsa_params* params, const gbsa_forward_args* args,
                            hipStream_t stream);

/*
 * gbsa_forward_ex for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. The call allocates nothing
 * and needs no workspace: the split-KV partial results, the arrival counters and the status
 * word live in a fixed device array of the library (one per GPU, held until the process
 * ends) of GBSA_NOALLOC_SCRATCH_BYTES bytes. args->workspace must be NULL and
 * args->workspace_bytes 0; every other argument is that of gbsa_forward_ex, and the result
 * is the same, bit for bit.
 * Limits: the workspace gbsa_workspace_size would report for these params (partial results
 * of 2 x workers x rows per unit, rows per unit = block_x * N1 / N2) must fit the array, and
 * workers x row subtiles (ceil(rows per unit / 256) above 16 rows, else 1) must not exceed
 * GBSA_NOALLOC_MAX_COUNTERS; otherwise GBSA_ERR_WORKSPACE is returned and nothing is
 * enqueued. Choose num_workers to fit (the decode shapes fit with the default count).
 * Sharing: all calls on one GPU use the same array. Calls that overlap on one GPU (on
 * different streams, or from several host threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe. Every call leaves the arrival counters at
 * zero for the next; the first call on a GPU also clears them (and the status word) with a
 * small kernel on its stream. A refused call (metadata mismatch) fills attention_out and
 * softmax_lse with NaN, as gbsa_forward does; its status word is not readable by the caller.
 * Errors: those of gbsa_forward_ex; GBSA_ERR_WORKSPACE as above; GBSA_ERR_HIP if the array's
 * device address cannot be obtained.
 */
#define GBSA_NOALLOC_SCRATCH_BYTES (32u << 20)
#define GBSA_NOALLOC_MAX_COUNTERS 16384
gbsa_status gbsa_forward_ex_noalloc(const gbsa_params* params, const gbsa_forward_args* args,
                                    hipStream_t stream);

/*
 * Opt-in check of the tensor VALUES that the forward calls take on trust (the article's
 * "general constraints": tiling reads no tensor values, so the caller guarantees them). Runs
 * one small kernel over the same argument block as gbsa_forward_ex and ORs into *violations
 * (device int32, which the caller zeroes beforehand) one bit per broken rule:
 */
#define GBSA_BAD_CU_SEQLENS_Q 0x01  /* cu_seqlens_q: negative start, decreasing, past total_q,
                                       or implying another total_q_blocks */
#define GBSA_BAD_SEQUSED_Q 0x02     /* seqused_q[b] outside [0, q storage length of b] */
#define GBSA_BAD_KV_LENGTH 0x04     /* seqused_kv[b] < 0, or above the KV storage (PA_BBND:
                                       max_blocks_per_seq * 128; TND: cu_seqlens_kv span) */
#define GBSA_BAD_CU_SEQLENS_KV 0x08 /* TND: cu_seqlens_kv negative, decreasing or past T_kv */
#define GBSA_BAD_BLOCK_TABLE 0x10   /* PA_BBND: a page of a visible block outside
                                       [0, num_pages) */
#define GBSA_BAD_COUNT 0x20         /* sparse_block_count outside [0, top_k] (clamped) */
#define GBSA_BAD_SELECTION 0x40     /* a selected index (slot < count, >= 0) past the
                                       sequence's visible KV blocks (skipped by the kernels) */
#define GBSA_BAD_MASK_EXTENT 0x80   /* user mask rows/cols do not cover every active query row
                                       and visible key (the uncovered ones are not masked) */
#define GBSA_BAD_MAX_SEQLEN 0x100   /* a sequence longer than params->max_seqlen_q (query
                                       storage) or max_seqlen_kv (visible KV), when given */
/*
 * Rules 0x20, 0x40, 0x80 and 0x100 describe inputs the kernels handle in a defined way (clamp,
 * skip, leave unmasked, bounds unused); the others make the forward read undefined data. Errors (returned, nothing
 * enqueued): as gbsa_forward_ex, minus the metadata/workspace/output pointers, which are not
 * needed here; GBSA_ERR_NULL if violations is NULL.
 */
gbsa_status gbsa_validate(const gbsa_params* params, const gbsa_forward_args* args,
                          int32_t* violations, hipStream_t stream);

/*
 * Human-readable text for a status (static storage, never NULL; unknown values give
 * "unknown status"). The article's "aclnn API" section has the first stage validate its
 * arguments and answer with a status code; its code table is not on the page, so the codes
 * and their texts are this library's own (gbsa_status above).
 */
const char* gbsa_status_string(gbsa_status status);

#ifdef __cplusplus
}
#endif

#endif /* GBSA_H_ */
