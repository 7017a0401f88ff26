// attn_plan.cpp - host side of the C ABI: capabilities, contract validation (admission), the
// split policy, workspace sizing and argument checks. No device memory is touched here.
//
// Admission follows the pages: dispatch is decided by dtype, head grouping, dimensions and
// alignment, not by a tensor-parallel size ("SM70 attention and quantized projection coverage
// across TP sizes", section "Scope"); any positive page size that is a multiple of 16 is
// admitted (same page, section "Additional findings"); the library reports its batch capacity
// and FP32 accumulation ("DFlash2 concurrent long-context attention", section "Why the
// single-request optimization was missing from concurrent decode"; SM70 coverage page,
// section "Compiled-library precision admission").
#include <math.h>
#include <stdint.h>
#include <new>
#include <string.h>

#include "attn_internal.h"

namespace {

constexpr int kNominalCUs = 256;   // MI355X: 256 compute units in 8 XCDs

struct Geometry {
    int32_t kv_dtype, head_dim, max_q_len, max_rows;
};

// The kernels compiled into this library.
constexpr Geometry kGeometries[] = {
    {ATTN_KV_E4M3, 256, 8, attn::kMaxRows},
    {ATTN_KV_FP16, 128, 8, attn::kMaxRows},
    {ATTN_KV_E5M2, 256, 8, attn::kMaxRows},
    {ATTN_KV_FP16, 256, 8, attn::kMaxRows},
    {ATTN_KV_E4M3, 128, 8, attn::kMaxRows},
};
constexpr int kNumGeometries = sizeof(kGeometries) / sizeof(kGeometries[0]);

bool aligned(int64_t v, int64_t a) { return v > 0 && v % a == 0; }

attn::SplitPolicy policy_for(int num_cus, int num_kv_heads, int waves_per_simd) {
    attn::SplitPolicy p;
    // Aim waves_per_simd waves at every SIMD (two per split) for a typical batch of 8 long rows:
    // cap = 2 * waves_per_simd * CUs / (8 * Hkv) splits per (slot, KV head), i.e. 16 at Hkv 4
    // and 8 at Hkv 8 on 256 CUs with one wave per SIMD (32 and 16 for the E4M3 D128 kernel,
    // which runs two per SIMD). The cap depends on the device and the head geometry only -
    // never on the batch - so a request's partitions, and its output bits, are the same alone
    // or batched. Clamped to [8, 64]: partitions stay <= 131072 / 8 = 16384 tokens (the kernel
    // stages a split's block-table entries in LDS) and >= 512 tokens (part_min) keep partial
    // traffic small. Rows longer than 131072 tokens keep that row's partition length (part_max:
    // 8192 tokens at Hkv 4) and get up to 64 splits: in a batch of mixed lengths up to 262144,
    // halving the longest rows' partitions shortens the run by 14%, at a cost of 6% for a batch
    // whose rows are all 262144 tokens long (more, shorter workgroups per CU).
    const int cap = num_cus * 2 * waves_per_simd / (8 * num_kv_heads);
    p.split_cap = cap < 8 ? 8 : (cap > 64 ? 64 : cap);
    p.part_max = attn::kLongLen / p.split_cap;
    p.part_min = 512;
    p.part_align = 256;
    return p;
}

}  // namespace

extern "C" {

attn_status attn_get_capabilities(attn_caps* caps) {
    if (!caps) return ATTN_E_INVALID;
    memset(caps, 0, sizeof(*caps));
    caps->abi_version = ATTN_ABI_VERSION;
    caps->max_batch = attn::kMaxBatch;
    caps->accumulation_bits = 32;
    caps->page_alignment = attn::kPageAlign;
    caps->stride_alignment = attn::kStrideAlign;
    caps->max_seq_len = attn::kMaxSeqLen;
    caps->num_geometries = kNumGeometries;
    for (int i = 0; i < kNumGeometries; ++i) {
        caps->geometries[i].kv_dtype = kGeometries[i].kv_dtype;
        caps->geometries[i].head_dim = kGeometries[i].head_dim;
        caps->geometries[i].max_q_len = kGeometries[i].max_q_len;
        caps->geometries[i].max_rows = kGeometries[i].max_rows;
    }
    return ATTN_OK;
}

attn_status attn_plan(const attn_desc* d, int device, attn_plan_t* out, size_t* workspace_bytes) {
    if (out) *out = nullptr;
    if (!d || !out) return ATTN_E_INVALID;
    if (d->abi_version != ATTN_ABI_VERSION) return ATTN_E_INVALID;
    if (d->kv_dtype != ATTN_KV_E4M3 && d->kv_dtype != ATTN_KV_FP16 && d->kv_dtype != ATTN_KV_E5M2)
        return ATTN_E_INVALID;
    if (d->q_len < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1) return ATTN_E_INVALID;
    if (d->num_q_heads % d->num_kv_heads != 0) return ATTN_E_INVALID;
    if (d->page_size < 1 || d->page_size % attn::kPageAlign != 0) return ATTN_E_INVALID;
    if (d->max_seq_len < 1 || d->max_seq_len > attn::kMaxSeqLen) return ATTN_E_INVALID;
    if ((int64_t)d->max_pages_per_seq * d->page_size < d->max_seq_len) return ATTN_E_INVALID;
    if (d->batch_capacity < 1 || d->batch_capacity > attn::kMaxBatch) return ATTN_E_INVALID;
    const int64_t strides[6] = {d->k_page_stride, d->k_token_stride, d->k_head_stride,
                                d->v_page_stride, d->v_token_stride, d->v_head_stride};
    for (int64_t s : strides)
        if (!aligned(s, attn::kStrideAlign)) return ATTN_E_INVALID;
    // The kernel addresses a 16-token granule with 32-bit lane offsets from its first token.
    if (16 * d->k_token_stride + 4096 > INT32_MAX || 16 * d->v_token_stride + 4096 > INT32_MAX) return ATTN_E_INVALID;
    if (!(d->sm_scale >= 0.0f) || isinf(d->sm_scale)) return ATTN_E_INVALID;   // also rejects NaN
    if (d->causal != 0 && d->causal != 1) return ATTN_E_INVALID;

    const int32_t group = d->num_q_heads / d->num_kv_heads;
    const int64_t rows = (int64_t)d->q_len * group;
    bool supported = false;
    for (const Geometry& g : kGeometries)
        if (g.kv_dtype == d->kv_dtype && g.head_dim == d->head_dim && d->q_len <= g.max_q_len &&
            rows <= g.max_rows)
            supported = true;
    if (!supported) return ATTN_E_UNSUPPORTED;

    int num_cus = kNominalCUs;
    if (device != ATTN_DEVICE_HOST_ONLY) {
        if (device < 0) return ATTN_E_INVALID;
        attn_status st = attn_device_cus(device, &num_cus);
        if (st != ATTN_OK) return st;
    }

    attn_plan_s* p = new (std::nothrow) attn_plan_s;
    if (!p) return ATTN_E_INVALID;
    p->desc = *d;
    p->device = device;
    p->num_cus = num_cus;
    p->policy = policy_for(num_cus, d->num_kv_heads, attn_split_waves_per_simd(d->kv_dtype, d->head_dim));
    int32_t gs = 0;
    for (int32_t L = 1; L <= d->max_seq_len; ++L) {
        const int32_t s = attn::num_splits(L, p->policy);
        if (s > gs) gs = s;
    }
    p->grid_splits = gs;
    p->rows = (int32_t)rows;
    p->sm_scale = d->sm_scale > 0.0f ? d->sm_scale : (float)(1.0 / sqrt((double)d->head_dim));
    p->rows_alloc = (int32_t)((rows + 15) / 16 * 16);
    const size_t floats = (size_t)p->rows_alloc * d->head_dim + 2 * (size_t)p->rows_alloc;
    const size_t align_f = attn::kWorkspaceAlign / sizeof(float);
    p->split_floats = (floats + align_f - 1) / align_f * align_f;
    p->split_bytes = p->split_floats * sizeof(float);
    p->workspace_bytes = (size_t)d->batch_capacity * d->num_kv_heads * gs * p->split_bytes;
    if (workspace_bytes) *workspace_bytes = p->workspace_bytes;
    *out = p;
    return ATTN_OK;
}

void attn_plan_destroy(attn_plan_t plan) { delete plan; }

attn_status attn_plan_get_info(attn_plan_t p, attn_plan_info* info) {
    if (!p || !info) return ATTN_E_INVALID;
    info->num_cus = p->num_cus;
    info->split_cap = p->policy.split_cap;
    info->partition_max = p->policy.part_max;
    info->partition_min = p->policy.part_min;
    info->partition_align = p->policy.part_align;
    info->grid_splits = p->grid_splits;
    info->rows = p->rows;
    info->split_bytes = p->split_bytes;
    info->workspace_bytes = p->workspace_bytes;
    return ATTN_OK;
}

size_t attn_plan_workspace_bytes(attn_plan_t p, int32_t batch) {
    if (!p || batch < 1 || batch > p->desc.batch_capacity) return 0;
    return (size_t)batch * p->desc.num_kv_heads * p->grid_splits * p->split_bytes;
}

attn_status attn_plan_splits(attn_plan_t p, int32_t seq_len, int32_t* num_splits, int32_t* partition_len) {
    if (!p || !num_splits || !partition_len) return ATTN_E_INVALID;
    int32_t L = seq_len < 0 ? 0 : (seq_len > p->desc.max_seq_len ? p->desc.max_seq_len : seq_len);
    *num_splits = attn::num_splits(L, p->policy);
    *partition_len = L > 0 ? attn::partition_len(L, p->policy) : 0;
    return ATTN_OK;
}

const char* attn_status_string(attn_status s) {
    switch (s) {
        case ATTN_OK: return "ok";
        case ATTN_E_INVALID: return "invalid argument";
        case ATTN_E_UNSUPPORTED: return "unsupported geometry or dtype";
        case ATTN_E_HIP: return "HIP runtime error";
        case ATTN_E_WORKSPACE: return "workspace missing or too small";
        case ATTN_E_STATIC_WORKSPACE: return "batch needs more workspace than the library's static array holds";
    }
    return "unknown status";
}

}  // extern "C"

// Shared by attn_run / attn_combine / attn_run_static: O(1) host checks, then the parameter block.
attn_status attn_prepare(attn_plan_t p, const attn_args* a, void* stream, attn::RunParams* rp) {
    if (!p || !a || !rp) return ATTN_E_INVALID;
    if (p->device == ATTN_DEVICE_HOST_ONLY) return ATTN_E_INVALID;
    if (a->batch < 1 || a->batch > p->desc.batch_capacity) return ATTN_E_INVALID;
    if (!a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->seq_lens || !a->k_scale ||
        !a->v_scale || !a->out)
        return ATTN_E_INVALID;
    if (a->num_pages < 1) return ATTN_E_INVALID;
    if (((uintptr_t)a->k_cache % attn::kStrideAlign) || ((uintptr_t)a->v_cache % attn::kStrideAlign) ||
        ((uintptr_t)a->q % 16) || ((uintptr_t)a->out % 16) || ((uintptr_t)a->block_table % 4) ||
        ((uintptr_t)a->seq_lens % 4) || ((uintptr_t)a->k_scale % 4) || ((uintptr_t)a->v_scale % 4))
        return ATTN_E_INVALID;
    if (!a->workspace || ((uintptr_t)a->workspace % attn::kWorkspaceAlign)) return ATTN_E_WORKSPACE;
    if (a->workspace_bytes < attn_plan_workspace_bytes(p, a->batch)) return ATTN_E_WORKSPACE;
    int dev = -1;
    attn_status st = attn_stream_device(stream, &dev);
    if (st != ATTN_OK) return st;
    if (dev != p->device) return ATTN_E_INVALID;

    const attn_desc& d = p->desc;
    rp->q = (const uint16_t*)a->q;
    rp->k = (const uint8_t*)a->k_cache;
    rp->v = (const uint8_t*)a->v_cache;
    rp->block_table = a->block_table;
    rp->seq_lens = a->seq_lens;
    rp->k_scale = a->k_scale;
    rp->v_scale = a->v_scale;
    rp->ws = (float*)a->workspace;
    rp->out = (uint16_t*)a->out;
    rp->k_page_stride = d.k_page_stride;
    rp->k_token_stride = d.k_token_stride;
    rp->k_head_stride = d.k_head_stride;
    rp->v_page_stride = d.v_page_stride;
    rp->v_token_stride = d.v_token_stride;
    rp->v_head_stride = d.v_head_stride;
    rp->num_pages = a->num_pages;
    rp->bt_stride = d.max_pages_per_seq;
    rp->page_size = d.page_size;
    rp->page_magic = ((1ull << 40) + (uint64_t)d.page_size - 1) / (uint64_t)d.page_size;
    rp->max_seq_len = d.max_seq_len;
    rp->q_len = d.q_len;
    rp->num_q_heads = d.num_q_heads;
    rp->num_kv_heads = d.num_kv_heads;
    rp->group = d.num_q_heads / d.num_kv_heads;
    rp->rows = p->rows;
    rp->rows_alloc = p->rows_alloc;
    rp->grid_splits = p->grid_splits;
    rp->causal = d.causal;
    rp->split_floats = (int32_t)p->split_floats;
    rp->batch = a->batch;
    rp->order_by_work = a->batch >= 2 && a->batch <= attn::kOrderMaxBatch;
    rp->sm_scale = p->sm_scale;
    rp->policy = p->policy;
    return ATTN_OK;
}

extern "C" {

attn_status attn_run(attn_plan_t p, const attn_args* a, void* stream) {
    attn::RunParams rp;
    attn_status st = attn_prepare(p, a, stream, &rp);
    if (st != ATTN_OK) return st;
    return attn_launch_split(p, rp, stream);
}

attn_status attn_combine(attn_plan_t p, const attn_args* a, void* stream) {
    attn::RunParams rp;
    attn_status st = attn_prepare(p, a, stream, &rp);
    if (st != ATTN_OK) return st;
    return attn_launch_combine(p, rp, stream);
}

}  // extern "C"
