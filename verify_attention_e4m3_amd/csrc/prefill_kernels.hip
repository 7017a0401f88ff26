// prefill_kernels.hip - causal long-prefill attention for gfx950 (CDNA4), FP16 Q/K/V, D = 256.
//
// What is computed (see include/attn.h, attn_prefill): for query token t in [0, q_len) of head
// h, with G = Hq / Hkv and KV head g = h / G, softmax(sm_scale * q.K^T) V over the keys the
// token sees - with the queries being the last q_len positions of a kv_len-token sequence,
// token t sees keys j <= kv_len - q_len + t (every key when not causal). The long prefill of
// "SM70 attention and quantized projection coverage across TP sizes" (sections "Scope" and
// "Accumulation audit and rejected tuning": a Q8192 chunk against a 262144-token context,
// D = 256, six query heads per KV head, FP16 operands with both products summed in FP32, a
// full-width prefix plus a causal triangular tail).
//
// Kernel design (an MFMA-bound dense contraction, unlike the HBM-bound verify kernel):
//  * A workgroup of 4 waves (one per SIMD) owns 12 row tiles of 16 query rows: 16 consecutive
//    tokens of one query head each, all heads of one KV head group, so every K/V byte brought
//    into LDS serves 192 query rows. Wave w owns row tiles 3w .. 3w+2.
//  * Keys stream in blocks of 32 through a four-stage LDS ring (K and V, 16 KB each per stage):
//    right after the one barrier of an iteration all four waves issue direct global -> LDS loads
//    three blocks ahead. The loop is software-pipelined: iteration b computes S of block b+1,
//    whose MFMAs do not depend on (and so overlap) the softmax VALU work of block b, then block
//    b's softmax and PV. The 16-byte chunks of a K row are XOR-swizzled by token (chunk ^
//    token % 16), so the MFMA-order LDS reads of 16 lanes hit 16 different bank groups; V rows
//    swizzle whole 32-byte chunk pairs (pair ^ token % 16) for the transposed reads below.
//  * S^T = K . Q^T and O^T += V^T . P^T on v_mfma_f32_16x16x32_f16 with the query rows on the
//    N dimension: a lane holds one query row in both products, so softmax statistics stay
//    lane-local apart from a reduction over the 4 lanes of a row, and P feeds the second MFMA
//    from registers (the PV contraction visits keys in the order S^T holds them). The PV A
//    operand (16 dims x 8 keys per lane group) comes straight from the row-major V block through
//    gfx950's transposed LDS read (ds_read_b64_tr_b16), two reads per dim tile.
//  * Softmax in log2 units against a fixed per-row reference (the maximum of block 0, the first
//    block of every row that sees a key), so the O accumulators are only ever touched by MFMAs
//    and later blocks need no row maximum at all: the loop only keeps the largest exponential.
//    A later score may exceed the reference by up to 2^10 (exact range in FP16 and FP32); if any
//    exponential of the workgroup exceeds 2^10, it recomputes with each row's exact maximum
//    from a QK-only pass. Both passes depend only on the data, so results are deterministic.
//  * Q (3 row tiles x 256 dims) stays in registers for the whole key loop; O^T (3 x 256 x 16
//    FP32 per wave) lives in accumulation registers.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_internal.h"
#include "prefill_internal.h"

namespace attn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfWaves = 4;
constexpr int kPfRowTilesPerWave = 3;
constexpr int kPfBlock = 32;                                 // keys per block: two granules of 16
constexpr int kPfStages = 4;
constexpr int kPfD = 256;
constexpr int kPfRowBytes = kPfD * 2;                        // one token row of one head
constexpr int kPfStageBytes = kPfBlock * kPfRowBytes;        // 16 KB: one K (or V) block
constexpr int kPfLoadsPerWave = kPfStageBytes / 1024 / kPfWaves;   // 4 K + 4 V per wave and block
constexpr float kPfSlackFactor = 1024.0f;                    // 2^10: headroom over the reference

// Max over lanes l, l^16, l^32, l^48 (one MFMA column's four quarter-wave partials) with the
// gfx950 lane swaps (v_permlane32_swap: l <-> l^32, v_permlane16_swap: l <-> l^16), VALU only.
__device__ __forceinline__ float pf_quad_max(float m) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ uint32_t pf_lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global -> LDS load of 16 bytes per lane from base + voff into lds + 16*lane. Inline asm
// so that the compiler does not wait for it before every LDS read; the key loop waits
// explicitly. No streaming hint: every K/V block is read by all workgroups of its KV head.
__device__ __forceinline__ void pf_dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
    const uint64_t b64 = (uint64_t)base;
    const uint64_t sbase = join_words((uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32)),
                                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                 "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

struct PrefillLds {
    __attribute__((aligned(16))) uint8_t k[kPfStages][kPfStageBytes];
    __attribute__((aligned(16))) uint8_t v[kPfStages][kPfStageBytes];
};

// Loads of one key block: 16 instructions for K and 16 for V, each covering two 512-byte token
// rows; wave w issues instructions 4w .. 4w+3 of both. Lane l of instruction i writes LDS row
// 2i + l/32, slot l%32, and fetches that row's 16-byte chunk (l%32) ^ (row%16) for K and
// (l%32) ^ 2*(row%16) for V (V is read in 32-byte pieces, so its swizzle moves whole pairs of
// chunks). Rows past the sequence re-read its last token (they are masked).
// Per-lane byte offsets of a full block's loads (row 2i + l/32 of the block and its chunk), fixed
// for the kernel.
struct PfLoadOffs {
    uint32_t k[kPfLoadsPerWave];
    uint32_t v[kPfLoadsPerWave];
};

__device__ __forceinline__ PfLoadOffs pf_load_offsets(const PrefillParams& p, int wave, int lane) {
    PfLoadOffs lo;
    const int slot = lane & 31;
#pragma unroll
    for (int u = 0; u < kPfLoadsPerWave; ++u) {
        const int row = 2 * (wave * kPfLoadsPerWave + u) + (lane >> 5);
        lo.k[u] = (uint32_t)(row * p.k_token_stride * 2) + (uint32_t)(slot ^ (row & 15)) * 16;
        lo.v[u] = (uint32_t)(row * p.v_token_stride * 2) + (uint32_t)(slot ^ (2 * (row & 15))) * 16;
    }
    return lo;
}

__device__ __forceinline__ void pf_issue_block(const PrefillParams& p, const uint8_t* kbase, const uint8_t* vbase,
                                               int32_t blk, uint32_t k_stage, uint32_t v_stage, int wave,
                                               int lane, const PfLoadOffs& lo) {
    const int32_t key0 = blk * kPfBlock;
    const uint8_t* kb = kbase + (int64_t)key0 * p.k_token_stride * 2;
    const uint8_t* vb = vbase + (int64_t)key0 * p.v_token_stride * 2;
    if (key0 + kPfBlock <= p.kv_len) {                       // a full block: the fixed offsets
#pragma unroll
        for (int u = 0; u < kPfLoadsPerWave; ++u) {
            const int i = wave * kPfLoadsPerWave + u;
            pf_dma16(kb, lo.k[u], k_stage + i * 1024);
            pf_dma16(vb, lo.v[u], v_stage + i * 1024);
        }
        return;
    }
    const int32_t last = p.kv_len - 1 - key0;                // last valid row of this block
    const int slot = lane & 31;
#pragma unroll
    for (int u = 0; u < kPfLoadsPerWave; ++u) {
        const int i = wave * kPfLoadsPerWave + u;
        const int row = 2 * i + (lane >> 5);
        const int src_row = min(row, last);
        const uint32_t kchunk = (uint32_t)(slot ^ (row & 15)) * 16;
        const uint32_t vchunk = (uint32_t)(slot ^ (2 * (row & 15))) * 16;
        pf_dma16(kb, (uint32_t)(src_row * p.k_token_stride * 2) + kchunk, k_stage + i * 1024);
        pf_dma16(vb, (uint32_t)(src_row * p.v_token_stride * 2) + vchunk, v_stage + i * 1024);
    }
}

// Wait until at most `blocks` newer blocks' loads (8 per wave and block) are still in flight.
__device__ __forceinline__ void pf_wait_loads(int blocks) {
    if (blocks >= 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (blocks == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool kLongestFirst>
__global__ __launch_bounds__(64 * kPfWaves) void prefill_kernel(PrefillParams p) {
    constexpr int RT = kPfRowTilesPerWave;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;         // MFMA column: query row within a row tile
    const int qd = lane >> 4;        // quarter of the wave

    // Workgroup order: KV head fastest, then query tile - in descending order with kLongestFirst
    // (causal tiles see more keys the later their tokens, so the longest go first and the short
    // ones fill in behind them when the grid takes several rounds of the CUs).
    const int g = blockIdx.x % p.num_kv_heads;
    const int qi = blockIdx.x / p.num_kv_heads;
    const int qt = kLongestFirst ? (p.q_len + p.tokens_per_wg - 1) / p.tokens_per_wg - 1 - qi : qi;
    const int32_t t0 = qt * p.tokens_per_wg;

    // Row tile r (0..11) of the workgroup: query tokens t0 + 16*(r / G) + 0..15 of head g*G + r%G.
    half8 qop[RT][8];
    int32_t lim[RT];                 // keys j < lim[rt] are visible to this lane's row
    int32_t tok[RT], head[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = wave * RT + rt;
        const int tg = r / p.group;
        head[rt] = g * p.group + (r - tg * p.group);
        tok[rt] = t0 + 16 * tg + n;
        const bool live = tok[rt] < p.q_len;
        const uint16_t* qrow =
            p.q + (int64_t)(live ? tok[rt] : 0) * p.q_token_stride + (int64_t)head[rt] * p.q_head_stride;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const half8 v = *reinterpret_cast<const half8*>(qrow + 32 * ks + 8 * qd);
            qop[rt][ks] = live ? v : half8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        const int32_t vis = p.causal ? p.kv_len - p.q_len + tok[rt] + 1 : p.kv_len;
        lim[rt] = live ? max(0, min(vis, p.kv_len)) : 0;
    }
    // Make the Q loads land before the ring is primed (their waits would otherwise count the
    // ring's loads).
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ks = 0; ks < 8; ks += 2) asm volatile("" ::"v"(qop[rt][ks]), "v"(qop[rt][ks + 1]));

    // Keys the workgroup needs: up to the last visible key of its last live token. Blocks that
    // end below every row's limit need no mask.
    const int32_t t_last = min(t0 + p.tokens_per_wg, p.q_len) - 1;
    const int32_t key_end = p.causal ? min(p.kv_len, p.kv_len - p.q_len + t_last + 1) : p.kv_len;
    const int32_t nblk = key_end > 0 ? (key_end + kPfBlock - 1) / kPfBlock : 0;
    const int32_t mask_from = p.causal ? max(0, min(p.kv_len, p.kv_len - p.q_len + t0 + 1)) : p.kv_len;

    __shared__ PrefillLds lds;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k + (int64_t)g * p.k_head_stride);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v + (int64_t)g * p.v_head_stride);
    const uint32_t k0 = pf_lds_addr(&lds.k[0][0]);
    const uint32_t v0 = pf_lds_addr(&lds.v[0][0]);
    const float c = p.c;

    float4v o[RT][16];
    float m_ref[RT], l_run[RT];
    const PfLoadOffs lo = pf_load_offsets(p, wave, lane);

    auto stage_k = [&](int32_t blk) { return &lds.k[blk % kPfStages][0]; };
    auto issue = [&](int32_t blk) {
        const int sn = blk % kPfStages;
        pf_issue_block(p, kbase, vbase, blk, k0 + sn * kPfStageBytes, v0 + sn * kPfStageBytes, wave, lane, lo);
    };
    auto qk = [&](int32_t blk, float4v (&sacc)[2][RT]) {
        const uint8_t* kst = stage_k(blk);
        // K operands are read PD k-steps ahead of their MFMAs (a fence keeps the reads there;
        // left alone, the scheduler moves each read next to its use): 1-2% faster than one
        // step ahead.
        constexpr int PD = 4;
        auto kread = [&](int ks, int gr) {
            const int row = 16 * gr + n;
            const int chunk = (4 * ks + qd) ^ (row & 15);
            return *reinterpret_cast<const half8*>(kst + row * kPfRowBytes + chunk * 16);
        };
        half8 ka[PD + 1][2];
#pragma unroll
        for (int ks = 0; ks < PD; ++ks)
#pragma unroll
            for (int gr = 0; gr < 2; ++gr) ka[ks][gr] = kread(ks, gr);
#pragma unroll
        for (int gr = 0; gr < 2; ++gr)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sacc[gr][rt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (ks + PD < 8) {
#pragma unroll
                for (int gr = 0; gr < 2; ++gr) ka[(ks + PD) % (PD + 1)][gr] = kread(ks + PD, gr);
            }
            // keep the reads ahead of this k-step's MFMAs (VALU and SALU may still move)
            __builtin_amdgcn_sched_barrier(0x406);
#pragma unroll
            for (int gr = 0; gr < 2; ++gr) {
                const half8 a = ka[ks % (PD + 1)][gr];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    sacc[gr][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qop[rt][ks], sacc[gr][rt], 0, 0, 0);
            }
        }
    };
    // Row maximum of a block's scores (masked keys excluded), scaled to log2 units; lane (n, qd)
    // holds keys key0 + 16*gr + 4*qd + i of its row, the other three quarters the rest.
    auto row_max = [&](int32_t blk, const float4v (&sacc)[2][RT], int rt, bool masked) {
        const int32_t key0 = blk * kPfBlock;
        float mx = -INFINITY;
#pragma unroll
        for (int gr = 0; gr < 2; ++gr)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = sacc[gr][rt][i];
                mx = fmaxf(mx, (!masked || (key0 + 16 * gr + 4 * qd + i) < lim[rt]) ? x : -INFINITY);
            }
        return pf_quad_max(mx) * c;
    };
    // Exponentials against the fixed references, row sums, and P for the PV product. `emax`
    // keeps the largest exponential: one above kPfSlackFactor (2^10) means some score exceeded
    // its reference by more than 10 log2 units.
    float emax = 0.0f;
    auto softmax = [&](int32_t blk, const float4v (&sacc)[2][RT], half8 (&pop)[RT], auto masked_tag) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        const int32_t key0 = blk * kPfBlock;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float neg = -m_ref[rt];
            float e[8];
#pragma unroll
            for (int gr = 0; gr < 2; ++gr)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[gr][rt][i], c, neg));
                    // a row without a visible key has reference -inf and only masked blocks
                    if constexpr (kMasked) v = (key0 + 16 * gr + 4 * qd + i) < lim[rt] ? v : 0.0f;
                    e[4 * gr + i] = v;
                }
#pragma unroll
            for (int k = 0; k < 8; ++k) l_run[rt] += e[k];
            emax = fmaxf(fmaxf(emax, fmaxf(e[0], e[1])), fmaxf(fmaxf(e[2], e[3]), fmaxf(e[4], e[5])));
            emax = fmaxf(emax, fmaxf(e[6], e[7]));
#pragma unroll
            for (int k = 0; k < 8; ++k) pop[rt][k] = (_Float16)e[k];
        }
    };
    auto pv = [&](int32_t blk, const half8 (&pop)[RT]) {
        // O^T += V^T . P^T over the block's keys in the order 4*qd + e (e < 4) of granule 0,
        // then 16 + 4*qd + e - 4 (e >= 4), as P holds them. The V^T operand of dim tile jd
        // (dims 16*jd + 0..15) comes from two transposed LDS reads (ds_read_b64_tr_b16): in
        // each 16-lane group, lane n points at 4 dims (16*jd + 4*(n%4) ..) of key base + n/4,
        // and lane n receives dim 16*jd + n of the group's 4 keys. Group qd reads keys 4*qd..
        // (base 0) and 16 + 4*qd.. (base 16, 8 KB further in the stage).
        const uint8_t* vst = &lds.v[blk % kPfStages][0];
        const int vrow = 4 * qd + (n >> 2);                  // < 16: row % 16 of both reads
        const uint32_t vlane = (uint32_t)(vrow * kPfRowBytes + 8 * (n & 3));
#pragma unroll
        for (int jd = 0; jd < 16; ++jd) {
            const uint8_t* a0 = vst + vlane + (uint32_t)(32 * (jd ^ vrow));
            const short4v lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(__attribute__((address_space(3))) const void*)a0);
            const short4v hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(__attribute__((address_space(3))) const void*)(
                    a0 + 16 * kPfRowBytes));
            const half8 ah = __builtin_bit_cast(half8, short8v{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                o[rt][jd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, pop[rt], o[rt][jd], 0, 0, 0);
        }
    };

    // Blocks that end at or below every row's visible limit need no mask; the rest (the causal
    // tail and the ragged end of the keys) run the masked copy of the loop body.
    const int32_t nfull = min(nblk, mask_from / kPfBlock);
    // One pass over the key blocks, software-pipelined: iteration b computes S of block b+1 (its
    // MFMAs are independent of, and so overlap, the VALU work on block b), then consumes block b
    // (`consume(b, S, masked)`). Block i lives in ring stage i % 4; at iteration b the ring holds
    // K of b+1, V of b, block b+2 in flight and the stage of b+3 being loaded. `first(S)` sees
    // block 0's scores before the loop.
    auto run_pass = [&](auto consume, auto first) {
        float4v s_cur[2][RT];
        for (int32_t i = 0; i < min(nblk, kPfStages - 1); ++i) issue(i);
        if (nblk > 0) {
            pf_wait_loads(min(nblk, kPfStages - 1) - 1);      // block 0 of this wave has landed
            __syncthreads();
            qk(0, s_cur);
            first(s_cur);
        }
        auto iteration = [&](int32_t b, auto masked_tag) {
            // Block b+1 (if any) has landed everywhere, and iteration b-1 is done everywhere, so
            // the stage of block b-1 = b+3 may be refilled.
            pf_wait_loads(b + 2 < nblk ? 1 : 0);
            __syncthreads();
            if (b + kPfStages - 1 < nblk) issue(b + kPfStages - 1);
            float4v s_next[2][RT];
            qk(b + 1 < nblk ? b + 1 : b, s_next);             // past the end: a discarded re-read
            consume(b, s_cur, masked_tag);
#pragma unroll
            for (int gr = 0; gr < 2; ++gr)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) s_cur[gr][rt] = s_next[gr][rt];
        };
        for (int32_t b = 0; b < nfull; ++b) iteration(b, std::false_type{});
        for (int32_t b = nfull; b < nblk; ++b) iteration(b, std::true_type{});
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // no load may still write the ring
    };
    auto accumulate = [&](int32_t b, const float4v (&sacc)[2][RT], auto masked_tag) {
        half8 pop[RT];
        softmax(b, sacc, pop, masked_tag);
        pv(b, pop);
    };
    auto clear = [&]() {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            l_run[rt] = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) o[rt][j] = float4v{0.f, 0.f, 0.f, 0.f};
        }
    };

    // The first pass: each row's reference is the maximum of block 0 (every row that sees a key
    // sees key 0, so this is its first visible block; a row that sees none keeps -inf and only
    // has masked blocks).
    clear();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) m_ref[rt] = -INFINITY;
    run_pass(accumulate, [&](const float4v (&s0)[2][RT]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) m_ref[rt] = row_max(0, s0, rt, nfull == 0);
    });
    // Some score above its reference by more than the slack, anywhere in the workgroup: a QK-only
    // pass takes each row's exact maximum as its reference, and the accumulation runs again (it
    // cannot exceed those maxima). The barrier also frees the ring for a next pass.
    if (__syncthreads_or(emax > kPfSlackFactor) != 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) m_ref[rt] = -INFINITY;
        run_pass(
            [&](int32_t b, const float4v (&sacc)[2][RT], auto masked_tag) {
                constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) m_ref[rt] = fmaxf(m_ref[rt], row_max(b, sacc, rt, kMasked));
            },
            [](const float4v (&)[2][RT]) {});
        __syncthreads();
        clear();
        run_pass(accumulate, [](const float4v (&)[2][RT]) {});
    }

    // Normalise and store: O^T tile j element i of lane (n, qd) is dim 16*j + 4*qd + i of the
    // lane's row.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float l = l_run[rt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (tok[rt] >= p.q_len) continue;
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        uint16_t* orow = p.out + (int64_t)tok[rt] * p.o_token_stride + (int64_t)head[rt] * p.o_head_stride;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            half4v v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = l > 0.0f ? (_Float16)(o[rt][j][i] * inv) : (_Float16)0.0f;
            *reinterpret_cast<half4v*>(orow + 16 * j + 4 * qd) = v;
        }
    }
}

}  // namespace
}  // namespace attn

attn_status attn_launch_prefill(const attn::PrefillParams& p, void* stream) {
    attn::PrefillParams args = p;
    void* kargs[] = {&args};
    const unsigned q_tiles = (unsigned)((p.q_len + p.tokens_per_wg - 1) / p.tokens_per_wg);
    const unsigned grid = q_tiles * (unsigned)p.num_kv_heads;
    if (grid == 0) return ATTN_OK;
    // Longest tiles first when the causal grid takes three or more rounds of the CUs (one
    // workgroup per CU at a time); with one or two rounds the ascending order ends sooner.
    int dev = 0, cus = 0;
    const bool rounds3 = hipGetDevice(&dev) == hipSuccess && attn_device_cus(dev, &cus) == ATTN_OK &&
                         grid >= 3u * (unsigned)cus;
    const void* fn = p.causal && rounds3 ? (const void*)attn::prefill_kernel<true> : (const void*)attn::prefill_kernel<false>;
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(64 * attn::kPfWaves), kargs, 0, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

// ---- C ABI ----

extern "C" ATTN_API attn_status attn_prefill(const attn_prefill_desc* d, const void* q, const void* k, const void* v,
                                             void* out, void* stream) {
    if (!d || !q || !k || !v || !out) return ATTN_E_INVALID;
    if (d->abi_version != ATTN_ABI_VERSION) return ATTN_E_INVALID;
    if (d->q_len < 1 || d->kv_len < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1) return ATTN_E_INVALID;
    if (d->num_q_heads % d->num_kv_heads != 0) return ATTN_E_INVALID;
    if (d->causal != 0 && d->causal != 1) return ATTN_E_INVALID;
    if (!(d->sm_scale >= 0.0f) || d->sm_scale > 3.0e38f) return ATTN_E_INVALID;   // NaN, negative, inf
    const int64_t strides[8] = {d->q_token_stride, d->q_head_stride, d->k_token_stride, d->k_head_stride,
                                d->v_token_stride, d->v_head_stride, d->o_token_stride, d->o_head_stride};
    for (int64_t s : strides)
        if (s < 0 || s % 8 != 0) return ATTN_E_INVALID;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16 != 0) return ATTN_E_INVALID;
    // Per-lane 32-bit offsets address one 64-key block from its first key.
    if (64 * (d->k_token_stride * 2) + 1024 > INT32_MAX || 64 * (d->v_token_stride * 2) + 1024 > INT32_MAX)
        return ATTN_E_INVALID;
    const int group = d->num_q_heads / d->num_kv_heads;
    if (d->head_dim != 256 || 12 % group != 0) return ATTN_E_UNSUPPORTED;

    attn::PrefillParams p{};
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.out = (uint16_t*)out;
    p.q_token_stride = d->q_token_stride;
    p.q_head_stride = d->q_head_stride;
    p.k_token_stride = d->k_token_stride;
    p.k_head_stride = d->k_head_stride;
    p.v_token_stride = d->v_token_stride;
    p.v_head_stride = d->v_head_stride;
    p.o_token_stride = d->o_token_stride;
    p.o_head_stride = d->o_head_stride;
    p.q_len = d->q_len;
    p.kv_len = d->kv_len;
    p.num_q_heads = d->num_q_heads;
    p.num_kv_heads = d->num_kv_heads;
    p.group = group;
    p.tokens_per_wg = 16 * (12 / group);
    p.causal = d->causal;
    const float sm = d->sm_scale > 0.0f ? d->sm_scale : 1.0f / sqrtf((float)d->head_dim);
    p.c = fmaxf(sm * 1.4426950408889634f, 1.17549435e-38f);
    return attn_launch_prefill(p, stream);
}
