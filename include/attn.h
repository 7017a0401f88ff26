/*
 * attn.h - C ABI of the MI355X (gfx950) speculative-verify attention library (libattn.so).
 *
 * Operation. For every request slot b of a batch, with L = seq_lens[b], every verify query
 * token t in [0, q_len) and every query head h in [0, Hq), with G = Hq / Hkv and the KV head
 * g = h / G:
 *
 *     out[b][t][h][:] = sum_j softmax_j( sm_scale * <Q[b][t][h][:], k_scale * K_j> ) * v_scale * V_j
 *
 * over the keys j the token sees: j <= L - q_len + t when causal (the verify tokens are the
 * last q_len positions of the sequence), every j < L otherwise. A row that sees no key (L == 0,
 * padded slots, or t < q_len - L) is written as +0. K_j / V_j are the elements of KV head g
 * of logical token j, stored in physical page block_table[b][j / page_size] at slot
 * j % page_size, decoded from E4M3 bytes (OCP E4M3 without infinities, bias 7), E5M2 bytes
 * (OCP E5M2, bias 15) or FP16. The pages name E5M2 and FP16 KV as the other cache formats the
 * backend serves ("DFlash2 ...", same section below).
 *
 * Sources (pages of the method):
 *  - "DFlash2 concurrent long-context attention, 2026-09-27" (design note), section "Why the
 *    single-request optimization was missing from concurrent decode": q8 verify batches of
 *    B2..B16 over a paged E4M3 cache, FP16 queries, D = 256, six query heads per KV head,
 *    per-request lengths, per-request FP32 max/sum workspace panels, safe zero-length rows and
 *    padded requests, a reported batch capacity, workspaces shared per device/stream/contract
 *    that only grow. Section "Operator validation": batched results are bitwise equal to
 *    independent single-request execution; graph replay may change Q and lengths.
 *  - "SM70 attention and quantized projection coverage across TP sizes", section "Scope":
 *    admission by dtype, head grouping, dimensions and alignment; FP16 operands, and both
 *    the score and the value products accumulate in FP32; section "Compiled-library
 *    precision admission": the library reports its accumulation width (32); section
 *    "Additional findings": any positive page size that is a multiple of 16 is admitted;
 *    section "Graph replay and long-prefill follow-up": captured launches take values as
 *    kernel arguments, never host stack addresses.
 *  - "perf(fa2): port decode GQA group-swap into d128 varlen launcher" (PR #48), description:
 *    the query heads of one KV group are packed into one block so KV is read once per group;
 *    split partials are merged by a log-sum-exp combine.
 *
 * Execution model. attn_run launches one split-KV kernel: two waves per (slot, KV head,
 * split) read that split's token range once for all q_len*G packed rows and write an FP32
 * partial (running max, running sum, unnormalised output) into the caller's workspace.
 * attn_combine then merges the splits of each (slot, KV head) in split order and writes FP16.
 * The split count of a row depends only on its own length and on the plan (never on the batch
 * or on other rows), so a request's output bits do not depend on what it is batched with.
 *
 * Threading and ownership. A plan is immutable host memory; it may be shared by threads and
 * streams. The library never allocates, frees or synchronises device memory; every device
 * buffer is owned by the caller. Calls on one stream are ordered; two streams must not share
 * a workspace. No function throws or aborts; errors are returned as attn_status.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 1u

#if defined(__GNUC__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_E_INVALID = 1,      /* bad argument: null pointer, size, alignment, range, ABI mismatch */
    ATTN_E_UNSUPPORTED = 2,  /* well-formed but outside the implemented geometries / dtypes */
    ATTN_E_HIP = 3,          /* a HIP runtime call failed (device query or kernel launch) */
    ATTN_E_WORKSPACE = 4,    /* workspace pointer null or smaller than the plan requires */
    ATTN_E_STATIC_WORKSPACE = 5  /* attn_run_static: the batch needs more than ATTN_STATIC_WORKSPACE_BYTES */
} attn_status;

typedef enum attn_kv_dtype {
    ATTN_KV_E4M3 = 1,        /* one byte per element, OCP E4M3 (no infinities, NaN = S.1111.111) */
    ATTN_KV_FP16 = 2,        /* IEEE binary16 */
    ATTN_KV_E5M2 = 3         /* one byte per element, OCP E5M2 (the upper byte of an FP16 value) */
} attn_kv_dtype;

/* One supported (kv_dtype, head_dim) combination and its row limits. */
typedef struct attn_geometry {
    int32_t kv_dtype;        /* attn_kv_dtype */
    int32_t head_dim;
    int32_t max_q_len;       /* q_len in [1, max_q_len] */
    int32_t max_rows;        /* q_len * (Hq / Hkv) <= max_rows (rows packed per KV read) */
} attn_geometry;

#define ATTN_MAX_GEOMETRIES 8

typedef struct attn_caps {
    uint32_t abi_version;        /* ATTN_ABI_VERSION of the loaded library */
    int32_t max_batch;           /* largest batch_capacity a plan admits */
    int32_t accumulation_bits;   /* 32: QK^T and PV accumulate in FP32 */
    int32_t page_alignment;      /* page_size must be a positive multiple of this (16) */
    int32_t stride_alignment;    /* K/V bases and byte strides must be multiples of this (8) */
    int32_t max_seq_len;         /* largest max_seq_len a plan admits (262144) */
    int32_t num_geometries;
    attn_geometry geometries[ATTN_MAX_GEOMETRIES];
} attn_caps;

/* Static description of one attention contract; input to attn_plan. */
typedef struct attn_desc {
    uint32_t abi_version;        /* must be ATTN_ABI_VERSION */
    int32_t kv_dtype;            /* attn_kv_dtype */
    int32_t q_len;               /* verify tokens per request (8 for q8 verify) */
    int32_t num_q_heads;         /* Hq */
    int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0, query head h uses KV head h / (Hq/Hkv) */
    int32_t head_dim;            /* D */
    int32_t page_size;           /* tokens per page, > 0 and % 16 == 0 */
    int32_t max_pages_per_seq;   /* row length of the block table; >= ceil(max_seq_len / page_size) */
    int32_t max_seq_len;         /* longest seq_len any row may have; seq_lens are clamped to it */
    int32_t batch_capacity;      /* largest batch passed to attn_run / attn_combine */
    /* Byte strides of the K and V caches: element (page, slot, kv_head, d) is at
     * base + page*page_stride + slot*token_stride + kv_head*head_stride + d*elem_bytes.
     * Interleaved K/V layouts are expressed by the two bases and these strides. */
    int64_t k_page_stride, k_token_stride, k_head_stride;
    int64_t v_page_stride, v_token_stride, v_head_stride;
    float sm_scale;              /* softmax scale; 0 selects 1/sqrt(head_dim); must be finite, >= 0 */
    int32_t causal;              /* 1: bottom-right causal verify tail; 0: every key visible */
} attn_desc;

typedef struct attn_plan_s* attn_plan_t;

/* Pass as `device` to attn_plan for a host-only plan: it assumes the 256 compute units of an
 * MI355X, answers attn_plan_get_info / attn_plan_splits, and is refused by attn_run. */
#define ATTN_DEVICE_HOST_ONLY (-1)

typedef struct attn_plan_info {
    int32_t num_cus;             /* compute units the split policy was sized for */
    int32_t split_cap;           /* splits per (slot, KV head) for rows of up to 131072 tokens */
    int32_t partition_max;       /* longer rows: partitions of at most this many tokens, more splits
                                    (never more than 64 splits per row) */
    int32_t partition_min;       /* shortest token partition of a split */
    int32_t partition_align;     /* partitions are multiples of this many tokens */
    int32_t grid_splits;         /* splits per (slot, KV head) in the launch grid (= max over lengths) */
    int32_t rows;                /* q_len * Hq / Hkv packed rows per (slot, KV head) */
    size_t split_bytes;          /* workspace bytes of one split partial */
    size_t workspace_bytes;      /* bytes for batch_capacity slots */
} attn_plan_info;

/* Per-call device buffers. */
typedef struct attn_args {
    const void* q;               /* FP16 [batch][q_len][Hq][D], contiguous */
    const void* k_cache;         /* K cache base (see the strides in attn_desc) */
    const void* v_cache;         /* V cache base */
    int64_t num_pages;           /* pages addressable from both bases; block-table entries are
                                    clamped into [0, num_pages) so that no access leaves the caches */
    const int32_t* block_table;  /* int32 [batch][max_pages_per_seq]; only entries of pages holding
                                    tokens < seq_lens[b] are read */
    const int32_t* seq_lens;     /* int32 [batch]; clamped to [0, max_seq_len]; 0 = empty or padded */
    const float* k_scale;        /* device FP32 scalar (per-tensor K scale) */
    const float* v_scale;        /* device FP32 scalar (per-tensor V scale) */
    void* workspace;             /* FP32 split workspace, >= workspace_bytes_for(batch) bytes, 256-B aligned */
    size_t workspace_bytes;
    void* out;                   /* FP16 [batch][q_len][Hq][D], contiguous */
    int32_t batch;               /* slots in this call, 1 <= batch <= batch_capacity */
} attn_args;

/* Library capabilities: batch capacity, accumulation width, page alignment and the supported
 * geometries ("DFlash2 ...", section "Why the single-request optimization was missing from
 * concurrent decode": the library reports its batch capacity; "SM70 ...", section
 * "Compiled-library precision admission": it reports 32-bit accumulation).
 * Errors: ATTN_E_INVALID if caps is NULL. */
ATTN_API attn_status attn_get_capabilities(attn_caps* caps);

/* Admission ("SM70 ...", sections "Scope" and "Additional findings": by dtype, head grouping,
 * dimensions, alignment and page size, never by a tensor-parallel size) and the split policy.
 * Validate a contract and build an immutable host plan for HIP device `device` (or
 * ATTN_DEVICE_HOST_ONLY). Writes the plan to *plan and, if workspace_bytes is not NULL, the
 * workspace size for batch_capacity slots. No device memory is allocated or read.
 * Errors: ATTN_E_INVALID (null pointers, ABI mismatch, page_size % 16, Hq % Hkv, misaligned
 * strides, non-positive sizes, max_seq_len > caps.max_seq_len, block table too short,
 * batch_capacity out of range), ATTN_E_UNSUPPORTED (dtype / head_dim / rows outside
 * caps.geometries), ATTN_E_HIP (device query failed). On error *plan is set to NULL. */
ATTN_API attn_status attn_plan(const attn_desc* desc, int device, attn_plan_t* plan, size_t* workspace_bytes);

/* Release a plan (NULL is ignored). The caller must not use it afterwards. */
ATTN_API void attn_plan_destroy(attn_plan_t plan);

/* Plan facts. Errors: ATTN_E_INVALID (null pointer). */
ATTN_API attn_status attn_plan_get_info(attn_plan_t plan, attn_plan_info* info);

/* Workspace bytes attn_run needs for `batch` slots (request-major panels). 0 on bad input. */
ATTN_API size_t attn_plan_workspace_bytes(attn_plan_t plan, int32_t batch);

/* Split policy of the plan for one row length: number of splits and tokens per split (the last
 * split may be shorter). seq_len is clamped to [0, max_seq_len]. Errors: ATTN_E_INVALID. */
ATTN_API attn_status attn_plan_splits(attn_plan_t plan, int32_t seq_len, int32_t* num_splits, int32_t* partition_len);

/* Split-KV attention over the paged cache ("DFlash2 ...", section "Why the single-request
 * optimization was missing from concurrent decode": one launch for a whole verify batch with
 * per-request lengths and FP32 max/sum panels; "perf(fa2) ... PR #48", description: the query
 * heads of a KV group share one KV read).
 * Writes the FP32 partial of every (slot, KV head, split) to the workspace.
 * `stream` is a hipStream_t (NULL = the null stream of the current device) and must belong to
 * the plan's device. Asynchronous and capturable into a hipGraph: kernel arguments are values
 * and device pointers only, lengths/scales/queries/tables are read on the device at run time.
 * Errors: ATTN_E_INVALID (null plan/args/pointers, batch out of range, host-only plan, stream on
 * another device), ATTN_E_WORKSPACE, ATTN_E_HIP (launch failed). */
ATTN_API attn_status attn_run(attn_plan_t plan, const attn_args* args, void* stream);

/* The log-sum-exp merge of split partials ("perf(fa2) ... PR #48", description).
 * Log-sum-exp combine of the splits written by attn_run (same args, same stream, after it):
 * writes every output row of the `batch` slots, +0 for rows that see no key. Same errors. */
ATTN_API attn_status attn_combine(attn_plan_t plan, const attn_args* args, void* stream);

/* Static text for a status code (never NULL). */
ATTN_API const char* attn_status_string(attn_status status);

/*
 * Allocation-free attention, for callers that cannot allocate device memory or pass a workspace:
 * code under hipGraph stream capture, tight serving loops, harnesses that forbid allocation.
 * Same result as attn_run followed by attn_combine with the same plan and args (the same
 * kernels, so the same bits), but the split workspace is a static device array inside the
 * library instead of args->workspace (args->workspace and args->workspace_bytes are ignored).
 *
 * The array holds ATTN_STATIC_WORKSPACE_BYTES (64 MiB) on every GPU the library runs on, until
 * the process ends; its device address is looked up once per device, on the first call there.
 * A call needs attn_plan_workspace_bytes(plan, args->batch) bytes of it (25.4 MB for 8 rows of
 * 131072 tokens at Hkv 4, D 256, 48 packed rows); larger batches are refused with
 * ATTN_E_STATIC_WORKSPACE before anything is launched. Nothing in the array needs to start at
 * any value: every panel the combine reads is written by the same call's split launch.
 * Every call on one GPU shares that GPU's array: calls that may overlap on one GPU (two streams,
 * two threads) race on it and must be serialised by the caller.
 * Errors: as attn_run, plus ATTN_E_STATIC_WORKSPACE; ATTN_E_HIP if the array's address cannot be
 * obtained. No HIP allocation, free or synchronisation is made.
 */
#define ATTN_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
ATTN_API attn_status attn_run_static(attn_plan_t plan, const attn_args* args, void* stream);

/*
 * Long prefill. Causal attention of a chunk of q_len query tokens against a kv_len-token
 * sequence whose last q_len positions they are: query token t of head h sees keys
 * j <= kv_len - q_len + t (every key when causal == 0), K/V head g = h / (Hq / Hkv). FP16 Q, K,
 * V and output, D = 256, FP32 accumulation for QK and PV. Source: "SM70 attention and
 * quantized projection coverage across TP sizes", sections "Scope" and "Accumulation audit and
 * rejected tuning" (the Q8192 x KV262144 prefill of six query heads per KV head, a full prefix
 * plus a causal triangular tail, FP32 accumulation in both products).
 *
 * Layout: element (token, head, d) of Q / K / V / out is at base + token * token_stride +
 * head * head_stride + d (strides in elements, multiples of 8; bases 16-byte aligned; K/V tokens
 * contiguous in one buffer per tensor). Errors: ATTN_E_INVALID for null pointers, bad strides,
 * sizes or ABI version; ATTN_E_UNSUPPORTED unless head_dim == 256 and Hq / Hkv divides 12;
 * ATTN_E_HIP if the launch fails. Stateless: no plan, no workspace; the library allocates
 * nothing and does not synchronise. Rows that see no key are +0.
 */
typedef struct attn_prefill_desc {
    uint32_t abi_version;        /* ATTN_ABI_VERSION */
    int32_t q_len;               /* query tokens (>= 1) */
    int32_t kv_len;              /* keys (>= 1); queries are its last q_len positions */
    int32_t num_q_heads;         /* Hq */
    int32_t num_kv_heads;        /* Hkv, Hq % Hkv == 0 */
    int32_t head_dim;            /* 256 */
    int64_t q_token_stride, q_head_stride;   /* elements */
    int64_t k_token_stride, k_head_stride;
    int64_t v_token_stride, v_head_stride;
    int64_t o_token_stride, o_head_stride;
    float sm_scale;              /* 0 selects 1 / sqrt(head_dim) */
    int32_t causal;              /* 1 or 0 */
} attn_prefill_desc;

ATTN_API attn_status attn_prefill(const attn_prefill_desc* desc, const void* q, const void* k, const void* v,
                                  void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
