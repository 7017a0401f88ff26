// prefill_internal.h - kernel arguments of the long-prefill kernel (not part of the ABI).
#pragma once

#include <stdint.h>

#include "attn.h"

namespace attn {

struct PrefillParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    int64_t q_token_stride, q_head_stride;   // elements
    int64_t k_token_stride, k_head_stride;
    int64_t v_token_stride, v_head_stride;
    int64_t o_token_stride, o_head_stride;
    int32_t q_len, kv_len;
    int32_t num_q_heads, num_kv_heads, group;
    int32_t tokens_per_wg;                   // 16 * 12 / group query tokens per workgroup
    int32_t causal;
    float c;                                 // sm_scale * log2(e), > 0
};

}  // namespace attn

attn_status attn_launch_prefill(const attn::PrefillParams& p, void* stream);
