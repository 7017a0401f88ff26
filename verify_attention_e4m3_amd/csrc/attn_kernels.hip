// attn_kernels.hip - split-KV verify attention and log-sum-exp combine for gfx950 (CDNA4).
//
// What is computed (see include/attn.h): for every slot b, KV head g and packed row
// r = t*G + j (query token t, query head g*G + j), softmax(sm_scale * q.(k_scale*K)^T) over the
// keys the verify token sees, times v_scale*V. Sources: "DFlash2 concurrent long-context
// attention, 2026-09-27" (q8 verify over a paged E4M3 cache, D = 256, six query heads per KV
// head, per-request FP32 max/sum workspace panels, safe zero-length and padded rows);
// "perf(fa2): port decode GQA group-swap into d128 varlen launcher" PR #48 (pack the query
// heads of a KV group so KV is read once per group; merge split partials with a log-sum-exp
// combine); "SM70 attention and quantized projection coverage across TP sizes", section
// "Scope" (FP16 operands, FP32 accumulation for QK and PV) and "Implementation and validation
// in progress" (exact E4M3 -> FP16 conversion).
//
// Kernel design (one 64-lane wave per workgroup and per (slot, KV head, split)):
//  * The 48 packed rows (8 verify tokens x 6 heads) are the N dimension of every MFMA, so one
//    wave reads each K/V byte of its token range exactly once for all rows.
//  * S^T = K . Q^T on v_mfma_f32_16x16x32_f16: A = 16 tokens x 32 dims of K, B = 32 dims x 16
//    rows of Q (Q stays in registers for the whole split). The dims are visited in a
//    permuted order shared by A and B, chosen so each lane's K bytes are 4 contiguous 16-byte
//    loads; a contraction is indifferent to the order.
//  * O^T += V^T . P^T on the same MFMA: A = 16 dims x 32 tokens of V, B = 32 tokens x 16 rows
//    of P. The token order is the one the S^T accumulators already hold, so P feeds the
//    second MFMA straight from registers; MFMA j of a lane covers dims 16*m + j, so each lane
//    loads 16 contiguous V bytes per token and a byte permute regroups them per dim.
//  * Row ownership is identical in both products (row = lane % 16), so the running max/sum
//    and the O rescale stay lane-local; the max is reduced across the 4 lanes of a row.
//  * E4M3 -> FP16 is exact (every finite E4M3 value is an FP16 value); k_scale is folded into
//    the FP32 score scale and v_scale is applied once in the combine.
//  * Each split writes an FP32 panel {O[48][D], m[48], l[48]} (m in log2 units of the scaled
//    score). The combine merges a row's splits in split order - no atomics, so results are
//    bitwise reproducible and independent of the batch a request is in.
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kD = 256;

// Four E4M3 byte pairs -> eight FP16 values, byte k of (lo, hi) -> element k.
__device__ __forceinline__ half8 e4m3x8(uint32_t lo, uint32_t hi) {
    const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    return half8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max of three floats in one v_max3_f32. fmaxf would first quiet each operand (IEEE mode);
// the scores here are finite or -inf, so no quieting is needed.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ int32_t clamp_len(int32_t L, int32_t max_len) {
    return L < 0 ? 0 : (L > max_len ? max_len : L);
}

constexpr float kRefSlack = 10.0f;
// Block-table entries one split can touch: partitions are at most 8192 tokens and pages hold
// at least 16 tokens, so a split spans at most 8192/16 + 1 pages.
constexpr int kMaxSplitPages = 8192 / 16 + 2;

// One 32-token tile as each lane holds it. K: granule tt (tokens j0 + 16*tt + n), dims
// 64*i + 16*qd + 0..15. V: slot e = token 4*qd + (e & 3) of granule e >> 2, dims 16*n + 0..15.
struct TileK { u32x4 k[2][4]; };
struct TileV { u32x4 v[8]; };

// Page and slot of logical token j (a granule start): j / page_size by a multiply-shift with
// the host-computed reciprocal ceil(2^40 / page_size), exact for j < 2^20 and page_size < 2^20.
__device__ __forceinline__ void locate(int32_t j, const RunParams& p, int32_t& page_idx, int32_t& slot) {
    page_idx = (int32_t)(((uint64_t)(uint32_t)j * p.page_magic) >> 40);
    slot = j - page_idx * p.page_size;
}

// Per-lane byte offsets of a full tile within its two granules, fixed for the whole split.
// Every load instruction reads whole 256-byte token rows, 16 lanes per row, 4 rows per
// instruction, so each one is eight 128-byte lines.
// K: instruction i (0..7) covers tokens 16*(i/4) + 4*(i%4) + (lane/16) of the tile; lane l
//    fetches 16-byte chunk (l%16) ^ (token%16) of its row into LDS slot l%16. The XOR swizzle
//    lets the MFMA-order reads of the consumer (16 lanes = 16 tokens, same chunk) hit 16
//    different LDS bank groups.
// V: slot e of lane (n, qd) is token 4*qd + (e&3) of granule e>>2, dims 16*n + 0..15 - the
//    lane that loads a chunk is the lane that consumes it.
struct LaneOffs {
    uint32_t k[4];
    uint32_t v[4];
};

__device__ __forceinline__ LaneOffs lane_offsets(const RunParams& p, int lane, int n, int qd) {
    LaneOffs o;
    const int tr = lane >> 4, slot = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = 4 * i + tr;                    // token within the granule
        o.k[i] = (uint32_t)(tok * p.k_token_stride + 16 * (slot ^ tok));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) o.v[e] = (uint32_t)((4 * qd + e) * p.v_token_stride + 16 * n);
    return o;
}

// Uniform byte addresses of the first tokens of a tile's two granules (A at j0, B at gsB) in
// the K and V caches of this KV head.
struct Granules {
    const uint8_t* kA;
    const uint8_t* kB;
    const uint8_t* vA;
    const uint8_t* vB;
    int32_t j0, gsB;
};

__device__ __forceinline__ Granules granules(int32_t j0, int32_t last, const int32_t* pages, int32_t pg0,
                                             const uint8_t* kbase, const uint8_t* vbase, const RunParams& p) {
    Granules gr;
    gr.j0 = j0;
    gr.gsB = min(j0 + 16, last & ~15);
    int32_t ia, sa, ib, sb;
    locate(j0, p, ia, sa);
    locate(gr.gsB, p, ib, sb);
    const int64_t pageA = __builtin_amdgcn_readfirstlane(pages[ia - pg0]);
    const int64_t pageB = __builtin_amdgcn_readfirstlane(pages[ib - pg0]);
    gr.kA = kbase + pageA * p.k_page_stride + (int64_t)sa * p.k_token_stride;
    gr.kB = kbase + pageB * p.k_page_stride + (int64_t)sb * p.k_token_stride;
    gr.vA = vbase + pageA * p.v_page_stride + (int64_t)sa * p.v_token_stride;
    gr.vB = vbase + pageB * p.v_page_stride + (int64_t)sb * p.v_token_stride;
    return gr;
}

// Direct global -> LDS load of 16 bytes per lane from base + voff: lane l's bytes land at
// lds + 16*l. Issued as inline asm so that the compiler's wait-count pass, which cannot tell
// the two ring stages apart and would wait for every LDS load before any LDS read, leaves the
// waiting to the explicit vmcnt waits of the tile loop. The KV cache is read exactly once, so
// the loads carry the non-temporal (streaming) hint.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// A ring stage holds one tile: 16 rows of 64 lanes x 16 bytes (rows 0..7 K, 8..15 V).
constexpr int kStageRows = 16;
constexpr int kStageBytes = kStageRows * 64 * 16;

// A tile whose 32 tokens all precede `last` uses the split's fixed lane offsets; the tail tile
// clamps each lane's token to `last` (whose page exists; the extra tokens are masked).
__device__ __forceinline__ void issue_k(const Granules& gr, int32_t last, const LaneOffs& lo, uint32_t stage,
                                        const RunParams& p, int lane) {
    if (gr.j0 + kTileTokens - 1 <= last) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(gr.kA, lo.k[i], stage + i * 1024);
            dma16(gr.kB, lo.k[i], stage + (4 + i) * 1024);
        }
    } else {
        const int tr = lane >> 4, slot = lane & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 4 * i + tr;
            const uint32_t oa = (uint32_t)((min(gr.j0 + tok, last) - gr.j0) * p.k_token_stride + 16 * (slot ^ tok));
            const uint32_t ob =
                (uint32_t)((min(gr.j0 + 16 + tok, last) - gr.gsB) * p.k_token_stride + 16 * (slot ^ tok));
            dma16(gr.kA, oa, stage + i * 1024);
            dma16(gr.kB, ob, stage + (4 + i) * 1024);
        }
    }
}

__device__ __forceinline__ void issue_v(const Granules& gr, int32_t last, const LaneOffs& lo, uint32_t stage,
                                        const RunParams& p, int n, int qd) {
    if (gr.j0 + kTileTokens - 1 <= last) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dma16(gr.vA, lo.v[e], stage + (8 + e) * 1024);
            dma16(gr.vB, lo.v[e], stage + (12 + e) * 1024);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rel = 4 * qd + e;
            const uint32_t oa = (uint32_t)((min(gr.j0 + rel, last) - gr.j0) * p.v_token_stride + 16 * n);
            const uint32_t ob = (uint32_t)((min(gr.j0 + 16 + rel, last) - gr.gsB) * p.v_token_stride + 16 * n);
            dma16(gr.vA, oa, stage + (8 + e) * 1024);
            dma16(gr.vB, ob, stage + (12 + e) * 1024);
        }
    }
}

__device__ __forceinline__ void vm_wait_tile() { asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); }
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// S^T = K . Q^T for the tile's two 16-token granules and the three row tiles.
__device__ __forceinline__ void qk_tile(const TileK& t, float4v (&sacc)[2][kRowTiles],
                                        const half8 (&qop)[kRowTiles][8]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) sacc[tt][rt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const u32x4 w = t.k[tt][ks >> 1];
            const half8 a = (ks & 1) ? e4m3x8(w[2], w[3]) : e4m3x8(w[0], w[1]);
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt)
                sacc[tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qop[rt][ks], sacc[tt][rt], 0, 0, 0);
        }
    }
}

// Softmax step of one tile: masked raw scores (lane holds row n's tokens j0 + 16*tt + 4*qd + i),
// exponentials exp2(c*x - m) against the row references (c > 0, log2 units), P^T in FP16.
// Returns true (uniformly) when a row's tile max exceeds its reference by more than kRefSlack;
// the references are then raised and nothing was accumulated.
__device__ __forceinline__ bool softmax_tile(const float4v (&sacc)[2][kRowTiles], int32_t j0, int32_t mask_from,
                                             const int32_t (&lim)[kRowTiles], float c, float (&m_ref)[kRowTiles],
                                             float (&l_run)[kRowTiles], half8 (&pop)[kRowTiles], int qd) {
    float x[kRowTiles][8];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[rt][tt * 4 + i] = sacc[tt][rt][i];
    if (j0 + kTileTokens > mask_from) {      // only tiles at the causal tail or the row end
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    x[rt][tt * 4 + i] = (j0 + 16 * tt + 4 * qd + i) < lim[rt] ? x[rt][tt * 4 + i] : -INFINITY;
    }
    float mx[kRowTiles];
    bool over = false;
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        float m = max3f(max3f(x[rt][0], x[rt][1], x[rt][2]), max3f(x[rt][3], x[rt][4], x[rt][5]),
                        max3f(x[rt][6], x[rt][7], x[rt][7]));
        const float m16 = __shfl_xor(m, 16);
        m = max3f(m, m16, m16);
        const float m32 = __shfl_xor(m, 32);
        m = max3f(m, m32, m32);
        m *= c;                                      // c > 0: max commutes with the scale
        mx[rt] = m;
        over |= m > m_ref[rt] + kRefSlack && m_ref[rt] != -INFINITY;
    }
    if (__any(over)) {
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) m_ref[rt] = fmaxf(m_ref[rt], mx[rt]);
        return true;
    }
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        if (m_ref[rt] == -INFINITY) m_ref[rt] = mx[rt];        // first tile with a visible key
        const float neg_m = m_ref[rt] == -INFINITY ? 0.0f : -m_ref[rt];
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(__builtin_fmaf(x[rt][e], c, neg_m));
        l_run[rt] += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
#pragma unroll
        for (int e = 0; e < 8; ++e) pop[rt][e] = (_Float16)pe[e];
    }
    return false;
}

// O^T += V^T . P^T. For dword w of the lane's 16 V bytes and byte pair (2cp, 2cp+1), a byte
// permute regroups tokens (2pp, 2pp+1) of dims 16*n + 4*w + 2*cp + {0,1} into 16-bit words,
// which convert to the FP16 pairs of the A operand.
__device__ __forceinline__ void pv_tile(const TileV& t, const half8 (&pop)[kRowTiles], float4v (&o)[kRowTiles][16]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int cp = 0; cp < 2; ++cp) {
            const uint32_t sel = cp ? 0x07030602u : 0x05010400u;
            half8 a0, a1;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const uint32_t pr = __builtin_amdgcn_perm(t.v[2 * pp + 1][w], t.v[2 * pp][w], sel);
                const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pr, 1.0f, false);
                const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pr, 1.0f, true);
                a0[2 * pp] = lo[0];
                a0[2 * pp + 1] = lo[1];
                a1[2 * pp] = hi[0];
                a1[2 * pp + 1] = hi[1];
            }
            const int jd = 4 * w + 2 * cp;
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
                o[rt][jd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, pop[rt], o[rt][jd], 0, 0, 0);
                o[rt][jd + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, pop[rt], o[rt][jd + 1], 0, 0, 0);
            }
        }
    }
}

// Exact maximum of every row's scaled, masked scores over the split (log2 units; -inf for a
// row that sees no key in it). Used only by the rare recompute of a split; plain global loads.
__device__ __forceinline__ void split_row_max(float (&m)[kRowTiles], int32_t j_begin, int32_t j_end, int32_t mask_from,
                                              const int32_t (&lim)[kRowTiles], float c, const int32_t* pages,
                                              int32_t pg0, const uint8_t* kbase, const uint8_t* vbase, const RunParams& p,
                                              const half8 (&qop)[kRowTiles][8], int n, int qd) {
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) m[rt] = -INFINITY;
    const int32_t last = j_end - 1;
    for (int32_t j0 = j_begin; j0 < j_end; j0 += kTileTokens) {
        const Granules gr = granules(j0, last, pages, pg0, kbase, vbase, p);
        const uint8_t* rowA = gr.kA + (int64_t)(min(j0 + n, last) - j0) * p.k_token_stride + 16 * qd;
        const uint8_t* rowB = gr.kB + (int64_t)(min(j0 + 16 + n, last) - gr.gsB) * p.k_token_stride + 16 * qd;
        TileK t;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t.k[0][i] = *reinterpret_cast<const u32x4*>(rowA + 64 * i);
            t.k[1][i] = *reinterpret_cast<const u32x4*>(rowB + 64 * i);
        }
        float4v sacc[2][kRowTiles];
        qk_tile(t, sacc, qop);
        const bool need_mask = j0 + kTileTokens > mask_from;
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = sacc[tt][rt][i];
                    if (need_mask) v = (j0 + 16 * tt + 4 * qd + i) < lim[rt] ? v : -INFINITY;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            m[rt] = fmaxf(m[rt], mx * c);
        }
    }
}

__global__ __launch_bounds__(64) void split_kernel_e4m3_d256(RunParams p) {
    const int lane = threadIdx.x;
    const int n = lane & 15;       // MFMA column = packed row within a row tile
    const int qd = lane >> 4;      // quarter of the wave

    // Workgroup order: KV head fastest, then split, then slot. The KV heads of one token are
    // adjacent in the cache (token stride = Hkv * head stride), so the workgroups that read the
    // same tokens' rows are dispatched together and stream through the same DRAM pages at
    // about the same time.
    int wg = blockIdx.x;
    const int g = wg % p.num_kv_heads;
    wg /= p.num_kv_heads;
    const int s = wg % p.grid_splits;
    const int b = wg / p.grid_splits;

    const int32_t L = clamp_len(p.seq_lens[b], p.max_seq_len);
    const int32_t S = num_splits(L, p.policy);
    if (s >= S) return;
    const int32_t P = partition_len(L, p.policy);
    const int32_t j_begin = s * P;
    const int32_t j_end = min(j_begin + P, L);
    const int32_t last = j_end - 1;
    const int32_t last_tile = j_begin + (last - j_begin) / kTileTokens * kTileTokens;

    // Q^T operands stay in registers for the whole split: entry (rt, ks) holds dims
    // 64*(ks/2) + 16*qd + 8*(ks%2) + 0..7 of packed row rt*16 + n (zeros past q_len*G) - the
    // dim order of the K operand, so the contraction pairs matching dims.
    half8 qop[kRowTiles][8];
    int32_t lim[kRowTiles];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        const int r = rt * 16 + n;
        const int t = r / p.group;
        const int h = g * p.group + (r - t * p.group);
        const bool live = r < p.rows;
        const uint16_t* qrow = p.q + (((int64_t)b * p.q_len + (live ? t : 0)) * p.num_q_heads + (live ? h : 0)) * kD;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int d0 = 64 * (ks >> 1) + 16 * qd + 8 * (ks & 1);
            const half8 v = *reinterpret_cast<const half8*>(qrow + d0);
            qop[rt][ks] = live ? v : half8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        // Keys j < lim are visible to this row: the verify token t sits at position L - q_len + t.
        const int32_t lr = p.causal ? (L - p.q_len + 1 + t) : L;
        lim[rt] = min(lr, j_end);
    }
    // Score scale in log2 units, c = sm_scale * k_scale * log2(e). The softmax takes the max of
    // the raw scores and scales it, which needs c > 0: a negative k_scale is moved into Q
    // (negating FP16 is exact) and c = 0 is raised to the smallest normal float, which leaves
    // every exp2 argument unchanged (|score| * 2^-126 rounds away) but keeps -inf * c = -inf.
    float c = p.sm_scale * (*p.k_scale) * kLog2e;
    if (c < 0.0f) {
        c = -c;
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) qop[rt][ks] = -qop[rt][ks];
    }
    c = fmaxf(c, 1.17549435e-38f);
    // Make the Q loads land before the ring is primed: otherwise the compiler's waits for them,
    // placed at their first use, would count the ring loads issued in between and wait for those.
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
        for (int ks = 0; ks < 8; ks += 2) asm volatile("" ::"v"(qop[rt][ks]), "v"(qop[rt][ks + 1]));
    const int32_t mask_from = p.causal ? min(j_end, L - p.q_len + 1) : j_end;

    const uint8_t* kbase = p.k + (int64_t)g * p.k_head_stride;
    const uint8_t* vbase = p.v + (int64_t)g * p.v_head_stride;
    // The split's block-table entries, clamped into the caches, staged once in LDS: the tile
    // loop then issues no compiler-visible global load (whose wait would also drain the ring).
    __shared__ int32_t pages[kMaxSplitPages];
    int32_t pg0, pg_last, unused_slot;
    locate(j_begin, p, pg0, unused_slot);
    locate(last, p, pg_last, unused_slot);
    {
        const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
        for (int i = lane; i <= pg_last - pg0; i += 64) {
            const int32_t v = bt[pg0 + i];
            pages[i] = v < 0 ? 0 : (v >= p.num_pages ? (int32_t)(p.num_pages - 1) : v);
        }
    }
    __syncthreads();

    // Two-stage LDS ring: tile i lives in stage i % 2. Tiles i+1 and i+2 are in flight while
    // tile i is computed: tile i+2's K (V) loads are issued into stage i % 2 as soon as tile
    // i's K (V) has been read into registers. Past the split's end the last tile is loaded
    // again, so every iteration issues the same 16 loads and `vmcnt(16)` always means "tile i
    // has landed".
    __shared__ __attribute__((aligned(16))) uint8_t ring[2 * kStageBytes];
    const uint32_t ring0 = lds_addr(ring);
    const u32x4* ring_lane = reinterpret_cast<const u32x4*>(ring) + lane;
    const LaneOffs lo = lane_offsets(p, lane, n, qd);
    // LDS byte offsets of the consumer's K chunks: token n of granule tt at row 16*tt + n,
    // chunk 4*i + qd (dims 64*i + 16*qd + 0..15) in slot chunk ^ n.
    uint32_t k_rd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) k_rd[i] = n * 256 + 16 * ((4 * i + qd) ^ n);

    // Per-row reference max (log2 units). A row's reference is the max of the first tile in
    // which it sees a key; exponentials are taken against it, so O and l never need
    // rescaling and the O accumulators are touched only by MFMAs. A later tile may exceed the
    // reference by up to kRefSlack (P <= 2^kRefSlack, exact range in FP16 and FP32). If one
    // exceeds it by more, the split is recomputed once with each row's exact maximum over the
    // split as its reference (then no tile can exceed it). Both passes depend only on the
    // split's own data, so the result is deterministic.
    float m_ref[kRowTiles];
    float l_run[kRowTiles];
    float4v o[kRowTiles][16];

    auto run_pass = [&]() -> bool {
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
            l_run[rt] = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) o[rt][j] = float4v{0.f, 0.f, 0.f, 0.f};
        }
        {
            const Granules g0 = granules(j_begin, last, pages, pg0, kbase, vbase, p);
            issue_k(g0, last, lo, ring0, p, lane);
            issue_v(g0, last, lo, ring0, p, n, qd);
            const Granules g1 = granules(min(j_begin + kTileTokens, last_tile), last, pages, pg0, kbase, vbase, p);
            issue_k(g1, last, lo, ring0 + kStageBytes, p, lane);
            issue_v(g1, last, lo, ring0 + kStageBytes, p, n, qd);
        }
        bool over = false;
        int32_t j0 = j_begin;
        for (int st = 0;; st ^= 1) {
            const uint32_t stage = ring0 + st * kStageBytes;
            const u32x4* sl = ring_lane + st * (kStageBytes / 16);
            const Granules gn = granules(min(j0 + 2 * kTileTokens, last_tile), last, pages, pg0, kbase, vbase, p);
            vm_wait_tile();
            TileK tk;
            const uint8_t* stage_bytes = ring + st * kStageBytes;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tk.k[tt][i] = *reinterpret_cast<const u32x4*>(stage_bytes + tt * 4096 + k_rd[i]);
            lds_wait_all();
            issue_k(gn, last, lo, stage, p, lane);
            float4v sacc[2][kRowTiles];
            qk_tile(tk, sacc, qop);
            half8 pop[kRowTiles];
            over = softmax_tile(sacc, j0, mask_from, lim, c, m_ref, l_run, pop, qd);
            TileV tv;
#pragma unroll
            for (int e = 0; e < 8; ++e) tv.v[e] = sl[(8 + e) * 64];
            lds_wait_all();
            issue_v(gn, last, lo, stage, p, n, qd);
            if (over) break;
            pv_tile(tv, pop, o);
            j0 += kTileTokens;
            if (j0 > last) break;
        }
        vm_wait_all();   // no load may still be writing the ring when the wave moves on
        return over;
    };

    float* panel = p.ws + ((int64_t)(b * p.num_kv_heads + g) * p.grid_splits + s) * p.split_floats;
    // Split epilogue: O^T tile j holds O[row n][dim 16*(4*qd + i) + j] in element i.
    auto store_panel = [&]() {
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
            const int r = rt * 16 + n;
            float* orow = panel + r * kD + 64 * qd;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    *reinterpret_cast<float4v*>(orow + 16 * i + 4 * c4) =
                        float4v{o[rt][4 * c4][i], o[rt][4 * c4 + 1][i], o[rt][4 * c4 + 2][i], o[rt][4 * c4 + 3][i]};
            float l = l_run[rt];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            if (qd == 0) {
                panel[kRowsAlloc * kD + r] = m_ref[rt];
                panel[kRowsAlloc * kD + kRowsAlloc + r] = l;
            }
        }
    };

#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) m_ref[rt] = -INFINITY;
    const bool over = run_pass();
    store_panel();
    if (over) {
        split_row_max(m_ref, j_begin, j_end, mask_from, lim, c, pages, pg0, kbase, vbase, p, qop, n, qd);
        run_pass();
        store_panel();
    }
}

// Log-sum-exp combine: one wave per packed row. Lane s holds split s's (m, l) (splits past 64
// are folded in by lane s % 64 in order), the max and the denominator are wave reductions, and
// the O sum visits the splits in index order with every lane covering 4 dims; the split order
// is fixed, so the FP32 sums are bitwise reproducible.
__global__ __launch_bounds__(256) void combine_kernel_d256(RunParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row_blocks = (p.rows + 3) / 4;
    int wg = blockIdx.x;
    const int rb = wg % row_blocks;
    wg /= row_blocks;
    const int g = wg % p.num_kv_heads;
    const int b = wg / p.num_kv_heads;
    const int r = rb * 4 + wave;
    if (r >= p.rows) return;
    const int t = r / p.group;
    const int h = g * p.group + (r - t * p.group);

    const int32_t L = clamp_len(p.seq_lens[b], p.max_seq_len);
    const int32_t S = num_splits(L, p.policy);
    const float* panel0 = p.ws + (int64_t)(b * p.num_kv_heads + g) * p.grid_splits * p.split_floats;
    const int64_t m_off = kRowsAlloc * kD + r;
    const int64_t l_off = kRowsAlloc * kD + kRowsAlloc + r;

    float mloc = -INFINITY;
    for (int s = lane; s < S; s += 64) mloc = fmaxf(mloc, panel0[(int64_t)s * p.split_floats + m_off]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    const float M = mloc;

    float4v acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.0f;
    if (M != -INFINITY) {
        // weight and l of split `lane` (and lane + 64, ...), then the denominator
        float dloc = 0.0f;
        for (int s = lane; s < S; s += 64) {
            const float ms = panel0[(int64_t)s * p.split_floats + m_off];
            const float w = ms == -INFINITY ? 0.0f : fast_exp2(ms - M);
            dloc += w * panel0[(int64_t)s * p.split_floats + l_off];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) dloc += __shfl_xor(dloc, off);
        den = dloc;
        const float* orow = panel0 + r * kD + 4 * lane;
        int s = 0;
        for (; s + 4 <= S; s += 4) {
            float4v ov[4];
            float w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ov[u] = *reinterpret_cast<const float4v*>(orow + (int64_t)(s + u) * p.split_floats);
                const float ms = panel0[(int64_t)(s + u) * p.split_floats + m_off];
                w[u] = ms == -INFINITY ? 0.0f : fast_exp2(ms - M);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) acc += w[u] * ov[u];
        }
        for (; s < S; ++s) {
            const float4v ov = *reinterpret_cast<const float4v*>(orow + (int64_t)s * p.split_floats);
            const float ms = panel0[(int64_t)s * p.split_floats + m_off];
            acc += (ms == -INFINITY ? 0.0f : fast_exp2(ms - M)) * ov;
        }
    }
    const float scale = den > 0.0f ? (*p.v_scale) / den : 0.0f;
    uint16_t* out = p.out + (((int64_t)b * p.q_len + t) * p.num_q_heads + h) * kD + 4 * lane;
    typedef _Float16 half4v __attribute__((ext_vector_type(4)));
    half4v res;
#pragma unroll
    for (int i = 0; i < 4; ++i) res[i] = den > 0.0f ? (_Float16)(acc[i] * scale) : (_Float16)0.0f;
    *reinterpret_cast<half4v*>(out) = res;
}

}  // namespace
}  // namespace attn

attn_status attn_launch_split(const attn_plan_s* plan, const attn::RunParams& p, void* stream) {
    attn::RunParams args = p;
    void* kargs[] = {&args};
    const unsigned grid = (unsigned)p.batch * p.num_kv_heads * p.grid_splits;
    hipError_t e = hipLaunchKernel((const void*)attn::split_kernel_e4m3_d256, dim3(grid), dim3(64), kargs, 0,
                                   (hipStream_t)stream);
    (void)plan;
    return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

attn_status attn_launch_combine(const attn_plan_s* plan, const attn::RunParams& p, void* stream) {
    attn::RunParams args = p;
    void* kargs[] = {&args};
    const unsigned grid = (unsigned)p.batch * p.num_kv_heads * ((p.rows + 3) / 4);
    hipError_t e = hipLaunchKernel((const void*)attn::combine_kernel_d256, dim3(grid), dim3(256), kargs, 0,
                                   (hipStream_t)stream);
    (void)plan;
    return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

attn_status attn_device_cus(int device, int* num_cus) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device >= count) return ATTN_E_HIP;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
        return ATTN_E_HIP;
    *num_cus = cus;
    return ATTN_OK;
}

attn_status attn_stream_device(void* stream, int* device) {
    if (stream == nullptr) return hipGetDevice(device) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
    hipDevice_t dev;
    if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return ATTN_E_HIP;
    *device = (int)dev;
    return ATTN_OK;
}
