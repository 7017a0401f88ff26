// attn_internal.h - plan layout, split policy and kernel parameters shared by the host plan
// code (attn_plan.cpp) and the kernels (attn_kernels.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "attn.h"

#if defined(__HIP__)
#define ATTN_HD static inline __host__ __device__
#else
#define ATTN_HD static inline
#endif

namespace attn {

// Packed rows (q_len * G) are processed in tiles of 16, at most 3 tiles (48 rows).
constexpr int kMaxRowTiles = 3;
constexpr int kMaxRows = 16 * kMaxRowTiles;
constexpr int kTileTokens = 32;        // tokens per inner iteration of one wave
constexpr int kMaxBatch = 256;
constexpr int kMaxSeqLen = 262144;
constexpr int kPageAlign = 16;
constexpr int kStrideAlign = 8;
constexpr int kWorkspaceAlign = 256;

// Split policy: a row of length L is cut into S(L) token partitions of P(L) tokens (the last
// one shorter). P depends only on L and on plan constants, never on the batch or other rows,
// so a request's partial sums - and therefore its output bits - are the same whether it runs
// alone or batched (the bitwise batched == single requirement of the DFlash2 long-batch note,
// "Operator validation"). P is a multiple of the kernel tile so tiles never straddle splits.
// Rows up to kLongLen tokens get split_cap splits; longer rows keep the partition length of a
// kLongLen row (part_max) and get more splits instead, up to kMaxSplits, so that in a batch of
// mixed lengths the longest rows do not leave a few long workgroups running alone at the end.
constexpr int kMaxSplits = 64;         // the combine kernel holds one split per lane
constexpr int kOrderMaxBatch = 64;     // batches the split kernel orders by work (one slot per lane)
constexpr int kLongLen = 131072;

struct SplitPolicy {
    int32_t split_cap;     // splits per (slot, KV head) for rows of up to kLongLen tokens
    int32_t part_max;      // longer rows: partitions of at most this many tokens (but <= kMaxSplits splits)
    int32_t part_min;      // shortest partition
    int32_t part_align;    // partitions are multiples of this (a multiple of kTileTokens)
};

ATTN_HD int32_t partition_len(int32_t L, SplitPolicy p) {
    int32_t want = (L + p.split_cap - 1) / p.split_cap;
    if (want > p.part_max) {
        const int32_t fewest = (L + kMaxSplits - 1) / kMaxSplits;
        want = p.part_max > fewest ? p.part_max : fewest;
    }
    want = ((want + p.part_align - 1) / p.part_align) * p.part_align;
    return want < p.part_min ? p.part_min : want;
}

ATTN_HD int32_t num_splits(int32_t L, SplitPolicy p) {
    if (L <= 0) return 0;
    const int32_t P = partition_len(L, p);
    return (L + P - 1) / P;
}

// 64-bit value from two 32-bit words. Both parameters are unsigned, so a low word with bit 31
// set is never sign-extended into the high half (the wave-uniform copies of a pointer made with
// readfirstlane come back as signed ints).
ATTN_HD uint64_t join_words(uint32_t hi, uint32_t lo) { return ((uint64_t)hi << 32) | (uint64_t)lo; }

// Kernel parameters, passed by value (a captured hipGraph keeps a copy; nothing points at
// host memory).
struct RunParams {
    const uint16_t* q;            // FP16 bits [batch][q_len][Hq][D]
    const uint8_t* k;             // cache bases (byte addressed)
    const uint8_t* v;
    const int32_t* block_table;   // [batch][bt_stride]
    const int32_t* seq_lens;      // [batch]
    const float* k_scale;
    const float* v_scale;
    float* ws;                    // split panels
    uint16_t* out;                // FP16 bits [batch][q_len][Hq][D]
    int64_t k_page_stride, k_token_stride, k_head_stride;
    int64_t v_page_stride, v_token_stride, v_head_stride;
    int64_t num_pages;
    int32_t bt_stride;
    int32_t page_size;
    uint64_t page_magic;          // ceil(2^40 / page_size): j / page_size = (j * page_magic) >> 40
    int32_t max_seq_len;
    int32_t q_len;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;                // Hq / Hkv
    int32_t rows;                 // q_len * group
    int32_t rows_alloc;           // 16 * row tiles: rows held in a split panel
    int32_t grid_splits;          // splits per (slot, KV head) in the grid
    int32_t causal;
    int32_t split_floats;         // floats per split panel
    int32_t batch;
    int32_t order_by_work;        // 1: split workgroups take slots longest partition first
    float sm_scale;
    SplitPolicy policy;
};

}  // namespace attn

struct attn_plan_s {
    attn_desc desc;
    int device;                    // HIP ordinal, or ATTN_DEVICE_HOST_ONLY
    int num_cus;
    attn::SplitPolicy policy;
    int32_t grid_splits;
    int32_t rows;
    int32_t rows_alloc;
    float sm_scale;
    size_t split_floats;
    size_t split_bytes;
    size_t workspace_bytes;        // for desc.batch_capacity slots
};

// O(1) host checks of a call and its kernel parameter block (attn_plan.cpp).
attn_status attn_prepare(attn_plan_t p, const attn_args* a, void* stream, attn::RunParams* rp);

// Launchers implemented in attn_kernels.hip (host side of the HIP translation unit).
attn_status attn_launch_split(const attn_plan_s* plan, const attn::RunParams& p, void* stream);
attn_status attn_launch_combine(const attn_plan_s* plan, const attn::RunParams& p, void* stream);
attn_status attn_device_cus(int device, int* num_cus);
// Waves per SIMD the split kernel of a (KV dtype, head dim) runs at: 2 for E4M3 at D128, else 1.
int attn_split_waves_per_simd(int kv_dtype, int head_dim);
attn_status attn_stream_device(void* stream, int* device);
