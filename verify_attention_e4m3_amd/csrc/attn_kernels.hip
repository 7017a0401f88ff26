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
// Kernel design (two 64-lane waves per (slot, KV head, split); one, two or four KV heads per
// workgroup, or, for grids of at most one workgroup per CU, one KV head with its rows split
// over two or three wave pairs):
//  * The packed rows (q_len verify tokens x G heads, up to 48) are the N dimension of every
//    MFMA, so each K/V byte of a token range is read exactly once for all rows (with two row
//    groups, once per group, the second read mostly from L2; with three, into one shared ring).
//  * S^T = K . Q^T on v_mfma_f32_16x16x32_f16: A = 16 tokens x 32 dims of K, B = 32 dims x 16
//    rows of Q (Q stays in registers for the whole split). The dims are visited in a
//    permuted order shared by A and B, chosen so each lane's K bytes are 4 contiguous 16-byte
//    loads; a contraction is indifferent to the order.
//  * O^T += V^T . P^T on the same MFMA: A = 16 dims x 32 tokens of V, B = 32 tokens x 16 rows
//    of P. The token order is the one the S^T accumulators already hold, so P feeds the
//    second MFMA straight from registers; each lane loads 16 contiguous V bytes per token and
//    a byte permute regroups them per dim.
//  * Row ownership is identical in both products (row = lane % 16), so the softmax statistics
//    stay lane-local; the max of a wave's first tile is reduced across the 4 lanes of a row and
//    becomes the row's fixed reference for the split (with a recompute pass if a later score
//    exceeds it by so much that P overflows FP16), so the O accumulators are never rescaled and
//    later tiles take no maximum at all.
//  * E4M3 / E5M2 -> FP16 are exact (every finite value of either is an FP16 value); k_scale is
//    folded into the FP32 score scale and v_scale is applied once in the combine.
//  * Each split writes an FP32 panel {O[rows][D], m[rows], l[rows]} (m in log2 units of the
//    scaled score). The combine merges a row's splits in split order - no atomics, so results
//    are bitwise reproducible and independent of the batch a request is in.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_internal.h"

namespace attn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Four E4M3 byte pairs -> eight FP16 values, byte k of (lo, hi) -> element k.
__device__ __forceinline__ half8 e4m3x8(uint32_t lo, uint32_t hi) {
    const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    return half8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max of three floats. Written with the compiler's own max rather than an inline v_max3_f32: its
// operands are often MFMA results, and the compiler inserts the wait states between an MFMA
// write and a VALU read only for instructions it can see.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Max over lanes l, l^16, l^32, l^48 (the four quarter-wave partials of one MFMA column) with
// the gfx950 lane swaps: v_permlane32_swap pairs lane l with l^32, v_permlane16_swap pairs l with
// l^16. Both are VALU operations, so the reduction takes no LDS round trip.
__device__ __forceinline__ float quad_max(float m) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = max3f(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return max3f(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[1]));
}

__device__ __forceinline__ int32_t clamp_len(int32_t L, int32_t max_len) {
    return L < 0 ? 0 : (L > max_len ? max_len : L);
}

// Block-table entries one split can touch: partitions are at most 32768 tokens and pages hold
// at least 16 tokens, so a split spans at most 32768/16 + 1 pages.
constexpr int kMaxSplitPages = 32768 / 16 + 2;

// One 32-token tile as each lane holds it (see LaneOffs for which bytes).
struct TileK { u32x4 k[2][4]; };
struct TileV { u32x4 v[8]; };

// KV element formats. A tile is two granules of 16 rows of 256 bytes: for E4M3 / E5M2 at D = 256
// and FP16 at D = 128 (256-byte token rows) they are 32 consecutive tokens; for FP16 at D = 256
// (512-byte rows) they are the two 256-byte halves of 16 tokens. All share the gather, the LDS
// ring and the swizzle; they differ in how a lane's 16 bytes become MFMA operands and which
// output dims an accumulator element holds. Traits: TILE tokens per tile, NG granules of scores
// per tile, B_TOK / B_BYTES the token and byte offset of granule B from granule A, ROW the bytes
// of one head's token row (E4M3 at D = 128 has 128-byte rows: see Fmt<kFmtE4M3D128>).
enum KvFormat { kFmtE4M3D256 = 0, kFmtF16D128 = 1, kFmtE5M2D256 = 2, kFmtF16D256 = 3, kFmtE4M3D128 = 4 };

// Byte -> FP16 decoders of the one-byte formats; both are exact.
// E4M3: v_cvt_scalef32_pk_f16_fp8 with scale 1.0 (every finite E4M3 value is an FP16 value).
struct DecE4M3 {
    __device__ static half8 x8(uint32_t lo, uint32_t hi) { return e4m3x8(lo, hi); }
    // Byte pair cp of the dwords a (token 2pp) and b (token 2pp+1): FP16 pairs (a, b) of dims
    // 2cp (d0) and 2cp+1 (d1).
    __device__ static void pair(uint32_t b, uint32_t a, int cp, half2v& d0, half2v& d1) {
        const uint32_t pr = __builtin_amdgcn_perm(b, a, cp ? 0x07030602u : 0x05010400u);
        d0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pr, 1.0f, false);
        d1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pr, 1.0f, true);
    }
};

// E5M2 has FP16's sign, exponent width and bias, so a byte is the upper byte of the FP16 value
// it encodes (subnormals, infinities and NaN included): decoding is a byte permute that puts
// each byte over a zero byte (selector 0x0c yields 0x00).
struct DecE5M2 {
    __device__ static half8 x8(uint32_t lo, uint32_t hi) {
        const u32x4 w = {__builtin_amdgcn_perm(0u, lo, 0x010c000cu), __builtin_amdgcn_perm(0u, lo, 0x030c020cu),
                         __builtin_amdgcn_perm(0u, hi, 0x010c000cu), __builtin_amdgcn_perm(0u, hi, 0x030c020cu)};
        return __builtin_bit_cast(half8, w);
    }
    __device__ static void pair(uint32_t b, uint32_t a, int cp, half2v& d0, half2v& d1) {
        d0 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(b, a, cp ? 0x060c020cu : 0x040c000cu));
        d1 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(b, a, cp ? 0x070c030cu : 0x050c010cu));
    }
};

// One-byte formats, D = 256. K vector i of a lane holds dims 64*i + 16*qd + 0..15 (one byte
// each) and feeds k-steps 2i and 2i+1; PV MFMA j (0..15) covers dims 16*m + j.
// S^T = K . Q^T for the two 16-token granules of a 32-token tile (one accumulator each).
template <class F, int RT>
__device__ __forceinline__ void qk_two_granules(const TileK& t, float4v (&sacc)[2][RT],
                                                const half8 (&qop)[RT][F::KSTEPS]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sacc[tt][rt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const half8 a = F::k_op(t.k[tt], ks);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                sacc[tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qop[rt][ks], sacc[tt][rt], 0, 0, 0);
        }
    }
}

template <class Dec>
struct Fmt8D256 {
    static constexpr int D = 256;
    static constexpr int KSTEPS = 8;
    static constexpr int JT = 16;
    static constexpr int TILE = 32, NG = 2, B_TOK = 16, B_BYTES = 0, ROW = 256;
    // V^T operands come from transposed LDS reads (see read_v); PV accumulator element i of
    // tile j holds dim 16*j + 4*qd + i, so the four elements of a tile are consecutive dims.
    static constexpr bool VTR = true;
    typedef half8 PopT;
    template <int RT>
    __device__ static void qk(const TileK& t, float4v (&sacc)[2][RT], const half8 (&qop)[RT][KSTEPS]) {
        qk_two_granules<Fmt8D256, RT>(t, sacc, qop);
    }
    __device__ static int q_dim(int ks, int qd) { return 64 * (ks >> 1) + 16 * qd + 8 * (ks & 1); }
    __device__ static half8 k_op(const u32x4 (&k)[4], int ks) {
        const u32x4 w = k[ks >> 1];
        return (ks & 1) ? Dec::x8(w[2], w[3]) : Dec::x8(w[0], w[1]);
    }
    __device__ static int o_dim(int qd, int i, int j) { return 16 * j + 4 * qd + i; }
    // O^T += V^T . P^T. Dwords 2*(j%2) and 2*(j%2)+1 of t.v[j/2] hold dim 16*j + lane%16 of the
    // lane's 8 tokens in k order (read_v), so one decode gives MFMA j's A operand.
    template <int RT>
    __device__ static void pv(const TileV& t, const half8 (&pop)[RT], float4v (&o)[RT][JT]) {
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const half8 a = Dec::x8(t.v[j >> 1][2 * (j & 1)], t.v[j >> 1][2 * (j & 1) + 1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                o[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop[rt], o[rt][j], 0, 0, 0);
        }
    }
};

template <int FMT> struct Fmt;
template <> struct Fmt<kFmtE4M3D256> : Fmt8D256<DecE4M3> {};
template <> struct Fmt<kFmtE5M2D256> : Fmt8D256<DecE5M2> {};

// FP16, D = 128. K vector i of a lane holds dims 32*i + 8*qd + 0..7 and is k-step i as it is;
// PV MFMA j (0..7) covers dims 8*m + j.
template <> struct Fmt<kFmtF16D128> {
    static constexpr int D = 128;
    static constexpr int KSTEPS = 4;
    static constexpr int JT = 8;
    static constexpr int TILE = 32, NG = 2, B_TOK = 16, B_BYTES = 0, ROW = 256;
    static constexpr bool VTR = false;
    typedef half8 PopT;
    template <int RT>
    __device__ static void qk(const TileK& t, float4v (&sacc)[2][RT], const half8 (&qop)[RT][KSTEPS]) {
        qk_two_granules<Fmt<kFmtF16D128>, RT>(t, sacc, qop);
    }
    __device__ static int q_dim(int ks, int qd) { return 32 * ks + 8 * qd; }
    __device__ static half8 k_op(const u32x4 (&k)[4], int ks) { return __builtin_bit_cast(half8, k[ks]); }
    __device__ static int o_dim(int qd, int i, int j) { return 8 * (4 * qd + i) + j; }
    // O^T += V^T . P^T. Dword w of the lane's 16 V bytes holds dims 8*n + 2w, 2w+1 of a token;
    // a permute pairs tokens (2pp, 2pp+1) of one of those dims into an FP16 pair.
    template <int RT>
    __device__ static void pv(const TileV& t, const half8 (&pop)[RT], float4v (&o)[RT][JT]) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t sel = h ? 0x07060302u : 0x05040100u;
                u32x4 a;
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) a[pp] = __builtin_amdgcn_perm(t.v[2 * pp + 1][w], t.v[2 * pp][w], sel);
                const half8 ah = __builtin_bit_cast(half8, a);
                const int jd = 2 * w + h;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    o[rt][jd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, pop[rt], o[rt][jd], 0, 0, 0);
            }
        }
    }
};

// FP16, D = 256: 512-byte token rows, so a tile is 16 tokens and its granules A and B are their
// dims 0..127 and 128..255 (granule B = same tokens, 256 bytes on). K vector i of granule tt of
// a lane holds dims 128*tt + 32*i + 8*qd + 0..7 (k-step 4*tt + i as it is); both halves
// accumulate into one score tile. PV runs on v_mfma_f32_16x16x16_f16 over the 16 tokens: lane
// (m, qd) holds dims 8m..8m+7 (slots 0..3) and 128+8m.. (slots 4..7) of tokens 4*qd + 0..3, and
// MFMA j covers dims 8m + j (j < 8) or 128 + 8m + j - 8.
template <> struct Fmt<kFmtF16D256> {
    static constexpr int D = 256;
    static constexpr int KSTEPS = 8;
    static constexpr int JT = 16;
    static constexpr int TILE = 16, NG = 1, B_TOK = 0, B_BYTES = 256, ROW = 256;
    static constexpr bool VTR = false;
    typedef half4 PopT;
    __device__ static int q_dim(int ks, int qd) { return 32 * ks + 8 * qd; }
    __device__ static int o_dim(int qd, int i, int j) { return j < 8 ? 8 * (4 * qd + i) + j : 128 + 8 * (4 * qd + i) + j - 8; }
    template <int RT>
    __device__ static void qk(const TileK& t, float4v (&sacc)[2][RT], const half8 (&qop)[RT][KSTEPS]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sacc[0][rt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const half8 a = __builtin_bit_cast(half8, t.k[tt][ks]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    sacc[0][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qop[rt][4 * tt + ks], sacc[0][rt], 0, 0, 0);
            }
    }
    template <int RT>
    __device__ static void pv(const TileV& t, const half4 (&pop)[RT], float4v (&o)[RT][JT]) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t sel = h ? 0x07060302u : 0x05040100u;
                    const uint32_t a0 = __builtin_amdgcn_perm(t.v[4 * hf + 1][w], t.v[4 * hf][w], sel);
                    const uint32_t a1 = __builtin_amdgcn_perm(t.v[4 * hf + 3][w], t.v[4 * hf + 2][w], sel);
                    const half4 ah = __builtin_bit_cast(half4, (uint32_t __attribute__((ext_vector_type(2)))){a0, a1});
                    const int jd = 8 * hf + 2 * w + h;
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        o[rt][jd] = __builtin_amdgcn_mfma_f32_16x16x16f16(ah, pop[rt], o[rt][jd], 0, 0, 0);
                }
    }
};

// E4M3, D = 128: 128-byte token rows, 32-token tiles of two 16-token granules. K vector i
// (i = 0, 1) of a lane holds dims 64*i + 16*qd + 0..15 and feeds k-steps 2i and 2i+1, as at
// D = 256. PV tile j (0..7) covers dims 16*j .. 16*j + 15, its V^T operand from a transposed
// LDS read (read_v).
template <> struct Fmt<kFmtE4M3D128> {
    static constexpr int D = 128;
    static constexpr int KSTEPS = 4;
    static constexpr int JT = 8;
    static constexpr int TILE = 32, NG = 2, B_TOK = 16, B_BYTES = 0, ROW = 128;
    // V^T operands from transposed LDS reads, as for the one-byte D = 256 formats (read_v).
    static constexpr bool VTR = true;
    typedef half8 PopT;
    __device__ static int q_dim(int ks, int qd) { return 64 * (ks >> 1) + 16 * qd + 8 * (ks & 1); }
    __device__ static half8 k_op(const u32x4 (&k)[4], int ks) {
        const u32x4 w = k[ks >> 1];
        return (ks & 1) ? e4m3x8(w[2], w[3]) : e4m3x8(w[0], w[1]);
    }
    __device__ static int o_dim(int qd, int i, int j) { return 16 * j + 4 * qd + i; }
    template <int RT>
    __device__ static void qk(const TileK& t, float4v (&sacc)[2][RT], const half8 (&qop)[RT][KSTEPS]) {
        qk_two_granules<Fmt<kFmtE4M3D128>, RT>(t, sacc, qop);
    }
    // O^T += V^T . P^T: slot j of the transposed read holds dim 16*j + lane%16 of the lane's 8
    // tokens in k order.
    template <int RT>
    __device__ static void pv(const TileV& t, const half8 (&pop)[RT], float4v (&o)[RT][JT]) {
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const half8 a = e4m3x8(t.v[j >> 1][2 * (j & 1)], t.v[j >> 1][2 * (j & 1) + 1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                o[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop[rt], o[rt][j], 0, 0, 0);
        }
    }
};

// Row geometry of a format: K loads per granule (1 KB each), rows per load, lanes per row, the
// chunk-swizzle key of a token, the V layout, and the LDS ring it implies.
// A wave's ring has 2 stages. 256-byte rows: a tile is 16 KB (K in 1 KB rows 0..7 of its stage,
// V in rows 8..15), 32 KB of ring. 128-byte rows: a tile is 8 KB (K rows 0..3, V rows 4..7),
// 16 KB of ring, so a workgroup of two head pairs fits twice in a CU's LDS and the kernel can be
// held to 256 registers (two waves per SIMD), which keeps the score tiles in VGPRs: in
// accumulation registers every VALU read of them first takes a copy (8% slower at D128).
template <class F>
struct Geo {
    static constexpr int KL = F::ROW / 64;            // 4 (256-byte rows) or 2 (128-byte rows)
    static constexpr int RPI = 1024 / F::ROW;         // token rows per load instruction
    static constexpr int LPR = F::ROW / 16;           // lanes per token row
    static constexpr int CH = F::ROW / 64;            // 16-byte K chunks a lane reads per granule token
    // K chunk c of token t sits in LDS slot c ^ swz(t): with rows 256 bytes apart the 16 lanes of
    // an MFMA-order read (16 tokens, one chunk) then hit 16 bank groups; 128-byte rows pair up.
    __device__ static int swz(int t) { return F::ROW == 256 ? t : (t >> 1); }
    static constexpr int KLOADS = 2 * KL;             // per tile and wave
    static constexpr int VLOADS = 2 * KL;             // V is stored once, like K
    // V load e of a tile lands at vblk(e) bytes from the stage's V region. For transposed V
    // reads the blocks are 1040 bytes apart, so each block's token rows start 16 bytes further
    // along the LDS banks than the previous block's and the eight rows a 16-lane group reads
    // together (one per block) fall on eight different bank groups.
    static constexpr int VBLK = F::VTR ? 1040 : 1024;
    __device__ static constexpr int vblk(int e) { return VBLK * e; }
    static constexpr int STAGE = KLOADS * 1024 + (F::VTR ? VLOADS * 1040 + 128 : VLOADS * 1024);
    static constexpr int VROW = KLOADS;               // first 1 KB row of V in a stage
    static constexpr int NS = 2;                      // ring stages per wave
    static constexpr int RING = NS * STAGE;           // ring bytes per wave
    // 128-byte rows, V: load p (0, 1) of a granule holds, in its 128-byte row q, the granule's
    // token 4*(q/2) + 2*(q%2) + p: the 4 tokens a 16-lane group takes from a granule (4*qd + i,
    // i = 0..3) lie in two loads (i & 1) and two row parities (i >> 1), which with the loads'
    // 16-byte phase steps puts the group's 8 rows on 8 different bank groups.
    __device__ static int vtok128(int q, int p) { return 4 * (q >> 1) + 2 * (q & 1) + p; }
};

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
// V: load e (0..3) of a granule covers tokens 4*q + e of it, quarter q of the load being token
//    4*q + e's row; lane (n, qd) fetches dims 16*n + 0..15 of token 4*qd + e. Without transposed
//    reads the lane that loads a chunk is the lane that consumes it (read_v).
struct LaneOffs {
    uint32_t k[4];
    uint32_t v[4];
};

template <class F>
__device__ __forceinline__ LaneOffs lane_offsets(const RunParams& p, int lane, int n, int qd) {
    using G = Geo<F>;
    LaneOffs o;
    const int tr = lane / G::LPR, slot = lane % G::LPR;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = G::RPI * i + tr;               // token within the granule (i < KL used)
        o.k[i] = (uint32_t)(tok * p.k_token_stride + 16 * (slot ^ G::swz(tok)));
    }
    if constexpr (F::ROW == 256) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o.v[e] = (uint32_t)((4 * qd + e) * p.v_token_stride + 16 * n);
    } else {
#pragma unroll
        for (int e = 0; e < 2; ++e) o.v[e] = (uint32_t)(G::vtok128(lane >> 3, e) * p.v_token_stride + 16 * (lane & 7));
        o.v[2] = o.v[3] = 0;
    }
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
    bool past_end;       // a prefetch beyond the split: every lane re-reads token `last`
};

template <class F>
__device__ __forceinline__ Granules granules(int32_t j0, int32_t last, const int32_t* pages, int32_t pg0,
                                             const uint8_t* kbase, const uint8_t* vbase, const RunParams& p) {
    Granules gr;
    gr.past_end = j0 > last;
    if (gr.past_end) j0 = last & ~15;
    gr.j0 = j0;
    gr.gsB = min(j0 + F::B_TOK, last & ~15);
    int32_t ia, sa, ib, sb;
    locate(j0, p, ia, sa);
    locate(gr.gsB, p, ib, sb);
    const int64_t pageA = __builtin_amdgcn_readfirstlane(pages[ia - pg0]);
    const int64_t pageB = __builtin_amdgcn_readfirstlane(pages[ib - pg0]);
    gr.kA = kbase + pageA * p.k_page_stride + (int64_t)sa * p.k_token_stride;
    gr.kB = kbase + pageB * p.k_page_stride + (int64_t)sb * p.k_token_stride + F::B_BYTES;
    gr.vA = vbase + pageA * p.v_page_stride + (int64_t)sa * p.v_token_stride;
    gr.vB = vbase + pageB * p.v_page_stride + (int64_t)sb * p.v_token_stride + F::B_BYTES;
    return gr;
}

// Direct global -> LDS load of 16 bytes per lane from base + voff: lane l's bytes land at
// lds + 16*l. Issued as inline asm so that the compiler's wait-count pass, which cannot tell
// the two ring stages apart and would wait for every LDS load before any LDS read, leaves the
// waiting to the explicit vmcnt waits of the tile loop. The KV cache is read once, so the loads
// carry the non-temporal (streaming) hint (NT); with two row groups the same bytes are read by
// two waves at about the same time, and plain loads let the second read hit in L2.
template <bool NT>
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
    const uint64_t b64 = (uint64_t)base;
    const uint64_t sbase = join_words((uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32)),
                                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64));
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                     "v"(voff), "s"(sbase)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                     "v"(voff), "s"(sbase)
                     : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Waves per SIMD the compiler is held to: two for 128-byte rows (their 16 KB rings leave room for
// two workgroups per CU), else one.
template <int FMT>
constexpr int split_waves_per_simd() { return Fmt<FMT>::ROW == 128 ? 2 : 1; }

// A tile whose 32 tokens all precede `last` uses the split's fixed lane offsets; the tail tile
// clamps each lane's token to `last` (whose page exists; the extra tokens are masked). A
// prefetch past the split's end keeps the per-tile load count (so the ring's vmcnt accounting
// is the same every iteration) but reads only token `last`'s row, which stays in L2.
template <class F, bool NT>
__device__ __forceinline__ void issue_k(const Granules& gr, int32_t last, const LaneOffs& lo, uint32_t stage,
                                        const RunParams& p, int lane) {
    using G = Geo<F>;
    if (gr.j0 + F::TILE - 1 <= last && !gr.past_end) {
#pragma unroll
        for (int i = 0; i < G::KL; ++i) {
            dma16<NT>(gr.kA, lo.k[i], stage + i * 1024);
            dma16<NT>(gr.kB, lo.k[i], stage + (G::KL + i) * 1024);
        }
    } else {
        const int tr = lane / G::LPR, slot = lane % G::LPR;
        const int32_t cap = gr.past_end ? gr.j0 : last;
#pragma unroll
        for (int i = 0; i < G::KL; ++i) {
            const int tok = G::RPI * i + tr;
            const uint32_t sw = 16 * (slot ^ G::swz(tok));
            const uint32_t oa = (uint32_t)((min(gr.j0 + tok, last) - gr.j0) * p.k_token_stride) + sw;
            const uint32_t ob = (uint32_t)((min(gr.j0 + F::B_TOK + tok, last) - gr.gsB) * p.k_token_stride) + sw;
            const uint32_t oz = (uint32_t)((last - cap) * p.k_token_stride + 16 * slot);
            dma16<NT>(gr.kA, gr.past_end ? oz : oa, stage + i * 1024);
            dma16<NT>(gr.kB, gr.past_end ? oz : ob, stage + (G::KL + i) * 1024);
        }
    }
}

template <class F, bool NT>
__device__ __forceinline__ void issue_v(const Granules& gr, int32_t last, const LaneOffs& lo, uint32_t stage,
                                        const RunParams& p, int n, int qd, int lane) {
    using G = Geo<F>;
    constexpr int VPG = G::VLOADS / 2;                // V loads per granule
    const uint32_t v0 = stage + G::VROW * 1024;
    if (gr.j0 + F::TILE - 1 <= last && !gr.past_end) {
#pragma unroll
        for (int e = 0; e < VPG; ++e) {
            dma16<NT>(gr.vA, lo.v[e], v0 + G::vblk(e));
            dma16<NT>(gr.vB, lo.v[e], v0 + G::vblk(VPG + e));
        }
    } else {
        // 256-byte rows: lane (n, qd) loads dims 16n.. of tokens 4qd + e; 128-byte rows: lane l
        // loads chunk l % 8 of token vtok128(l / 8, e).
        const uint32_t vb = F::ROW == 256 ? 16 * n : 16 * (lane & 7);
#pragma unroll
        for (int e = 0; e < VPG; ++e) {
            const int rel = F::ROW == 256 ? 4 * qd + e : G::vtok128(lane >> 3, e);
            const uint32_t oa = (uint32_t)((min(gr.j0 + rel, last) - gr.j0) * p.v_token_stride + vb);
            const uint32_t ob = (uint32_t)((min(gr.j0 + F::B_TOK + rel, last) - gr.gsB) * p.v_token_stride + vb);
            const uint32_t oz = (uint32_t)((last - gr.j0) * p.v_token_stride + vb);
            dma16<NT>(gr.vA, gr.past_end ? oz : oa, v0 + G::vblk(e));
            dma16<NT>(gr.vB, gr.past_end ? oz : ob, v0 + G::vblk(VPG + e));
        }
    }
}

// The V operand of a tile from its ring stage.
//  * Transposed reads (one-byte formats): for PV tile j (dims 16*j ..), 16-lane group qd needs
//    its 8 tokens 4*qd + (r&3) of granule r>>2 (r = 0..7, the order P holds them) for every dim
//    of the tile. ds_read_b64_tr_b8 takes, in each 16-lane group, an 8 x 16 byte block whose row
//    r is the 8-byte pieces of lanes 2r and 2r+1, and gives lane n column n: so lane n points at
//    row n/2's token, bytes 16*j + 8*(n&1) of it, and slot j of the result holds dim 16*j + n of
//    the 8 tokens in k order (dwords 2*(j&1), 2*(j&1)+1 of v[j/2]). With 256-byte rows, V load e
//    (block vblk(e)) holds in its quarter q the row of token 4*q + (e&3) of granule e>>2, so row
//    r of group qd is block r, quarter qd; with 128-byte rows, token 4*qd + i of granule g is in
//    load 2*g + (i&1), 128-byte row 2*qd + (i>>1) (Geo::vtok128).
//  * 256-byte rows otherwise: slot e of lane (n, qd) is the 16 bytes of dims 16n.. of token
//    4*qd + (e&3) of granule e>>2, stored by this very lane.
template <class F>
__device__ __forceinline__ TileV read_v(const uint8_t* stage, int n, int qd, int lane) {
    using G = Geo<F>;
    TileV tv;
    const uint8_t* v0 = stage + G::VROW * 1024;
    if constexpr (F::VTR) {
        typedef int int2v __attribute__((ext_vector_type(2)));
        const int r = n >> 1;
        const uint8_t* base = F::ROW == 256
                                  ? v0 + G::vblk(r) + 256 * qd + 8 * (n & 1)
                                  : v0 + G::vblk(2 * (r >> 2) + (r & 1)) + 128 * (2 * qd + ((r >> 1) & 1)) + 8 * (n & 1);
#pragma unroll
        for (int j = 0; j < F::JT; ++j) {
            const int2v w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) int2v*)(__attribute__((address_space(3))) const void*)(base + 16 * j));
            tv.v[j >> 1][2 * (j & 1)] = (uint32_t)w[0];
            tv.v[j >> 1][2 * (j & 1) + 1] = (uint32_t)w[1];
        }
    } else {
        static_assert(F::ROW == 256, "128-byte rows take transposed reads");
#pragma unroll
        for (int e = 0; e < 8; ++e) tv.v[e] = *reinterpret_cast<const u32x4*>(v0 + e * 1024 + 16 * lane);
    }
    return tv;
}

// Every tile is KLOADS K loads then (later) VLOADS V loads, and a wave keeps NS tiles in
// flight: when tile k's K is needed, its V and the next NS - 1 tiles' loads may still be
// outstanding; when its V is needed, those tiles' loads and the K loads issued after K(k) was read.
template <int N>
__device__ __forceinline__ void vm_wait_n() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <class F>
__device__ __forceinline__ void vm_wait_tile_k() {
    using G = Geo<F>;
    vm_wait_n<G::VLOADS + (G::NS - 1) * (G::KLOADS + G::VLOADS)>();
}
template <class F>
__device__ __forceinline__ void vm_wait_tile_v() {
    using G = Geo<F>;
    vm_wait_n<(G::NS - 1) * (G::KLOADS + G::VLOADS) + G::KLOADS>();
}
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Softmax step against fixed references, without a row maximum after the first tile. Every row
// that sees a key in a wave's tiles sees the first of them (a row's visible keys are a prefix),
// so that tile sets each row's reference (FIRST; a row without a key keeps -inf and only meets
// masked scores). Later tiles take exp2(c*x - m) directly; a score far above its reference
// makes P overflow FP16, which the row sums of the pass then show as non-finite.
template <int RT, int NG, int TILE, bool FIRST, class PopT>
__device__ __forceinline__ void softmax_fixed(const float4v (&sacc)[2][RT], int32_t j0, int32_t mask_from,
                                              const int32_t (&lim)[RT], float c, float (&m_ref)[RT],
                                              PopT (&pop)[RT], int qd) {
    constexpr int NV = 4 * NG;
    float x[RT][NV];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < NG; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[rt][tt * 4 + i] = sacc[tt][rt][i];
    if (j0 + TILE > mask_from) {             // only tiles at the causal tail or the row end
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int tt = 0; tt < NG; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    x[rt][tt * 4 + i] = (j0 + 16 * tt + 4 * qd + i) < lim[rt] ? x[rt][tt * 4 + i] : -INFINITY;
    }
    if constexpr (FIRST) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float m = NG == 2 ? max3f(max3f(x[rt][0], x[rt][1], x[rt][2]), max3f(x[rt][3], x[rt][4 % NV], x[rt][5 % NV]),
                                      max3f(x[rt][6 % NV], x[rt][7 % NV], x[rt][7 % NV]))
                              : max3f(max3f(x[rt][0], x[rt][1], x[rt][2]), x[rt][3], x[rt][3]);
            m = quad_max(m) * c;
            if (m_ref[rt] == -INFINITY) m_ref[rt] = m;
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float neg_m = m_ref[rt] == -INFINITY ? 0.0f : -m_ref[rt];
#pragma unroll
        for (int e = 0; e < NV; ++e) pop[rt][e] = (_Float16)fast_exp2(__builtin_fmaf(x[rt][e], c, neg_m));
    }
}

// True in every lane when some row sum of this wave is not finite (a P overflowed FP16).
template <int RT>
__device__ __forceinline__ bool sums_overflowed(const float4v (&lsum)[RT]) {
    bool bad = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) bad |= !(lsum[rt][0] <= 3.4028235e38f);
    return __any(bad);
}

// The slot a workgroup's grid position `b` serves and its clamped length. With order_by_work
// (batches of 2 to 64 slots) the positions go to the slots in order of decreasing partition
// length (then slot index), so the longest-running workgroups are dispatched first and the short
// ones fill in behind them; otherwise position b is slot b. Which workgroup serves a (slot,
// split) changes nothing in its arithmetic. Every lane reads one slot's length; `b` is updated
// in place to the slot index (wave-uniform).
__device__ __forceinline__ int32_t slot_for_position(const RunParams& p, int lane, int& b) {
    if (!p.order_by_work) return clamp_len(p.seq_lens[b], p.max_seq_len);
    const int32_t Ll = lane < p.batch ? clamp_len(p.seq_lens[lane], p.max_seq_len) : 0;
    const int32_t wk = lane < p.batch ? (Ll > 0 ? partition_len(Ll, p.policy) : 0) : -1;
    int rank = 0;
    for (int k = 0; k < p.batch; ++k) {
        const int32_t wkk = __builtin_amdgcn_readlane(wk, k);
        rank += (wkk > wk) | ((wkk == wk) & (k < lane));
    }
    const uint64_t hit = __ballot(lane < p.batch && rank == b);   // exactly one lane: ranks are a permutation
    if (hit != 0) b = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
    return __builtin_amdgcn_readlane(Ll, b);
}

// Q^T operands of row tiles rt0 .. rt0+RT-1 of KV head g of slot b, kept in registers for the
// whole split: entry (rt, ks) holds the 8 dims of k-step ks (F::q_dim) of packed row
// (rt0 + rt)*16 + n (zeros past q_len*G) - the dim order of the K operand, so the contraction
// pairs matching dims. lim[rt]: keys j < lim are visible to the row (the verify token t sits at
// position L - q_len + t), capped at the split's end.
template <class F, int RT>
__device__ __forceinline__ void load_q_rows(const RunParams& p, int b, int g, int rt0, int n, int qd, int32_t L,
                                            int32_t j_end, half8 (&qop)[RT][F::KSTEPS], int32_t (&lim)[RT]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = (rt0 + rt) * 16 + n;
        const int t = r / p.group;
        const int h = g * p.group + (r - t * p.group);
        const bool live = r < p.rows;
        const uint16_t* qrow = p.q + (((int64_t)b * p.q_len + (live ? t : 0)) * p.num_q_heads + (live ? h : 0)) * F::D;
#pragma unroll
        for (int ks = 0; ks < F::KSTEPS; ++ks) {
            const half8 v = *reinterpret_cast<const half8*>(qrow + F::q_dim(ks, qd));
            qop[rt][ks] = live ? v : half8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        const int32_t lr = p.causal ? (L - p.q_len + 1 + t) : L;
        lim[rt] = min(lr, j_end);
    }
}

// Stages the block-table entries of the pages that tokens j_begin .. last of slot b touch,
// clamped into the caches, in LDS (`NT` threads share the copy; the caller's barrier publishes
// it), so the tile loops issue no compiler-visible global load, whose wait would also drain the
// ring. Returns the index of the split's first page.
template <int NT>
__device__ __forceinline__ int32_t stage_pages(const RunParams& p, int b, int32_t j_begin, int32_t last,
                                               int32_t* pages) {
    int32_t pg0, pg_last, unused_slot;
    locate(j_begin, p, pg0, unused_slot);
    locate(last, p, pg_last, unused_slot);
    const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
    for (int i = threadIdx.x; i <= pg_last - pg0; i += NT) {
        const int32_t v = bt[pg0 + i];
        pages[i] = v < 0 ? 0 : (v >= p.num_pages ? (int32_t)(p.num_pages - 1) : v);
    }
    return pg0;
}

// Score scale in log2 units, c = sm_scale * k_scale * log2(e). The softmax takes the max of the
// raw scores and scales it, which needs c > 0: a negative k_scale is moved into Q (negating FP16
// is exact) and c = 0 is raised to the smallest normal float, which leaves every exp2 argument
// unchanged (|score| * 2^-126 rounds away) but keeps -inf * c = -inf.
template <int RT, int KS>
__device__ __forceinline__ float score_scale(const RunParams& p, half8 (&qop)[RT][KS]) {
    float c = p.sm_scale * (*p.k_scale) * kLog2e;
    if (c < 0.0f) {
        c = -c;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qop[rt][ks] = -qop[rt][ks];
    }
    return fmaxf(c, 1.17549435e-38f);
}

// Row sums of a tile's P on the matrix cores: a 16 x K block of ones times P^T (K tokens x 16 rows)
// adds, in every element of lane (n, qd)'s accumulator, the sum of packed row n's K weights - one
// MFMA per row tile instead of a VALU add tree, over the same FP16 weights the PV product uses.
template <int RT>
__device__ __forceinline__ void row_sums(const half8 (&pop)[RT], float4v (&lsum)[RT]) {
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pop[rt], lsum[rt], 0, 0, 0);
}
template <int RT>
__device__ __forceinline__ void row_sums(const half4 (&pop)[RT], float4v (&lsum)[RT]) {
    const half4 ones = {1, 1, 1, 1};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, pop[rt], lsum[rt], 0, 0, 0);
}

// a0*x0 + a1*x1 with the rounding spelled out (the first product rounded, the second fused), so
// that every instantiation of the split kernel - whatever its row tiles, heads or row groups -
// merges a row's two halves to the same bits (left to the compiler, the contraction may differ).
__device__ __forceinline__ float merge2(float a0, float x0, float a1, float x1) {
    return __builtin_fmaf(a1, x1, a0 * x0);
}

// Exact maximum of every row's scaled, masked scores over the split (log2 units; -inf for a
// row that sees no key in it). Used only by the rare recompute of a split; plain global loads.
template <int FMT, int RT>
__device__ __forceinline__ void split_row_max(float (&m)[RT], int32_t j_begin, int32_t j_end, int32_t mask_from,
                                              const int32_t (&lim)[RT], float c, const int32_t* pages, int32_t pg0,
                                              const uint8_t* kbase, const uint8_t* vbase, const RunParams& p,
                                              const half8 (&qop)[RT][Fmt<FMT>::KSTEPS], int n, int qd) {
    using F = Fmt<FMT>;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) m[rt] = -INFINITY;
    const int32_t last = j_end - 1;
    for (int32_t j0 = j_begin; j0 < j_end; j0 += F::TILE) {
        const Granules gr = granules<F>(j0, last, pages, pg0, kbase, vbase, p);
        const uint8_t* rowA = gr.kA + (int64_t)(min(j0 + n, last) - j0) * p.k_token_stride + 16 * qd;
        const uint8_t* rowB = gr.kB + (int64_t)(min(j0 + F::B_TOK + n, last) - gr.gsB) * p.k_token_stride + 16 * qd;
        TileK t;
#pragma unroll
        for (int i = 0; i < Geo<F>::CH; ++i) {
            t.k[0][i] = *reinterpret_cast<const u32x4*>(rowA + 64 * i);
            t.k[1][i] = *reinterpret_cast<const u32x4*>(rowB + 64 * i);
        }
        float4v sacc[2][RT];
        F::template qk<RT>(t, sacc, qop);
        const bool need_mask = j0 + F::TILE > mask_from;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < F::NG; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = sacc[tt][rt][i];
                    if (need_mask) v = (j0 + 16 * tt + 4 * qd + i) < lim[rt] ? v : -INFINITY;
                    mx = fmaxf(mx, v);
                }
            mx = quad_max(mx);
            m[rt] = fmaxf(m[rt], mx * c);
        }
    }
}

// Split kernel: a workgroup holds HP KV heads of one (slot, split), two 64-lane waves per head
// and row group, RT row tiles of 16 packed rows per wave. Wave w serves head HP*pair + w % HP and
// streams that head's tiles (w / HP) % 2, (w / HP) % 2 + 2, ... of the split through its own LDS
// ring; at the end the second wave of each pair hands its partial state to the first through
// LDS, which merges the two (always its own first) and writes its rows of the split panel. Two
// waves per split halve the number of splits, and with it the partial traffic, for the same
// number of waves in flight.
// With HP = 2 (even head counts) the waves of a workgroup read neighbouring head rows of the
// same tokens, so one CU streams whole 2*D-byte runs of each token row instead of isolated
// D-byte pieces; on MI355X that raises the sustained read rate of the paged stream by about a
// tenth over one head per workgroup.
// With RG = 2 row groups (HP = 1; grids that give each CU at most one workgroup, which would
// otherwise leave half of its SIMDs idle) a second pair of waves takes row tiles RT .. 2*RT - 1
// of the same head and tokens (past the head's last row tile, rows without a query: zero
// scores, never written), so each wave's tile loop carries fewer rows and every SIMD works.
// Each row's tiles, references, products and merge are the same in both layouts, and a pair
// recomputes with exact row maxima exactly when a row sum of either pair's wave of the same token
// half is not finite (a P overflowed FP16) - the same tokens and rows whose overflow decides the
// recompute of a one-group wave - so the row groups never change a bit of the result.
constexpr int kWavesPerHead = 2;

template <int NW, int RING>
struct SplitLds {
    __attribute__((aligned(16))) uint8_t rings[NW][RING];
    int32_t pages[kMaxSplitPages];
    int32_t over[NW];
};

template <int FMT, int RT, int HP, int RG>
__global__ __launch_bounds__(64 * kWavesPerHead * HP * RG, split_waves_per_simd<FMT>()) void split_kernel(RunParams p) {
    static_assert(RG == 1 || (RG == 2 && HP == 1), "row groups split one head's rows");
    using F = Fmt<FMT>;
    constexpr int D = F::D;
    constexpr int KS = F::KSTEPS;
    constexpr int JT = F::JT;
    constexpr int NW = kWavesPerHead * HP * RG;                  // waves per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform within a wave
    const int hl = wave % HP;                      // head within the workgroup
    const int half = (wave / HP) % kWavesPerHead;  // which of the pair's two waves
    const int rt0 = (wave / (HP * kWavesPerHead)) * RT;   // the wave's first row tile
    const int n = lane & 15;       // MFMA column = packed row within a row tile
    const int qd = lane >> 4;      // quarter of the wave

    // Workgroup order: KV-head group fastest, then split, then slot. The KV heads of one token
    // are adjacent in the cache (token stride = Hkv * head stride), so the workgroups that read
    // the same tokens' rows are dispatched together and stream through the same DRAM pages at
    // about the same time.
    int wg = blockIdx.x;
    const int head_groups = p.num_kv_heads / HP;
    const int g = (wg % head_groups) * HP + hl;
    wg /= head_groups;
    const int s = wg % p.grid_splits;
    int b = wg / p.grid_splits;
    const int32_t L = slot_for_position(p, lane, b);
    const int32_t S = num_splits(L, p.policy);
    if (s >= S) return;                 // uniform over the workgroup
    const int32_t P = partition_len(L, p.policy);
    const int32_t j_begin = s * P;
    const int32_t j_end = min(j_begin + P, L);
    const int32_t last = j_end - 1;

    // Q^T operands and visibility limits of the wave's row tiles.
    half8 qop[RT][KS];
    int32_t lim[RT];
    load_q_rows<F, RT>(p, b, g, rt0, n, qd, L, j_end, qop, lim);
    const float c = score_scale(p, qop);
    // Make the Q loads land before the ring is primed: otherwise the compiler's waits for them,
    // placed at their first use, would count the ring loads issued in between and wait for those.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) asm volatile("" ::"v"(qop[rt][ks]), "v"(qop[rt][ks + 1]));
    const int32_t mask_from = p.causal ? min(j_end, L - p.q_len + 1) : j_end;

    const uint8_t* kbase = p.k + (int64_t)g * p.k_head_stride;
    const uint8_t* vbase = p.v + (int64_t)g * p.v_head_stride;
    // LDS: the waves' rings, then the split's block-table entries (shared by the workgroup's
    // heads), clamped into the caches and staged once: the tile loop then issues no
    // compiler-visible global load (whose wait would also drain the ring).
    __shared__ SplitLds<NW, Geo<F>::RING> lds;
    int32_t* pages = lds.pages;
    const int32_t pg0 = stage_pages<64 * NW>(p, b, j_begin, last, pages);
    __syncthreads();

    // Per-wave LDS ring of NS stages: the wave's k-th tile lives in stage k % NS. Its tiles
    // k+1 .. k+NS are in flight while tile k is computed: tile k+NS's K (V) loads are issued into
    // stage k % NS as soon as tile k's K (V) has been read into registers. Past the split's end
    // the prefetches re-read one row, so every iteration issues the same KLOADS + VLOADS loads
    // and the fixed vmcnt before reading tile k's K (and again before its V) means "that half of
    // tile k has landed". After the tile loops the rings hold the hand-over.
    using G = Geo<F>;
    static_assert(G::NS * G::STAGE <= sizeof(lds.rings[0]), "ring stages must fit in the wave's ring");
    uint8_t* ring = lds.rings[wave];
    const uint32_t ring0 = lds_addr(ring);
    const LaneOffs lo = lane_offsets<F>(p, lane, n, qd);
    // LDS byte offsets of the consumer's K chunks: token n of granule tt at row n of the granule's
    // rows (ROW bytes each), chunk 4*i + qd in slot chunk ^ swz(n).
    uint32_t k_rd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) k_rd[i] = n * F::ROW + 16 * ((4 * i + qd) ^ Geo<F>::swz(n));
    constexpr int32_t kStride = kWavesPerHead * F::TILE;        // tokens between a wave's tiles
    const int32_t first = j_begin + half * F::TILE;              // this wave's first tile

    // Per-row reference max (log2 units). A row's reference is the max of the wave's first tile
    // (a row's visible keys are a prefix, so a row that sees any key of the wave's tiles sees one
    // in the first); exponentials are taken against it, so O and l never need rescaling and the
    // O accumulators are touched only by MFMAs. A later score may exceed the reference by almost
    // 16 log2 units: P then stays a finite FP16 value with FP16's full relative precision, and
    // the FP32 sums of P and P*V stay far from overflow. A score higher still makes its P infinite
    // in FP16, which the row sums show at the end of the pass; the wave (with row groups: every
    // wave of its token half) then recomputes its tiles once with each row's exact maximum over
    // the split as its reference (then no P exceeds 1). Both passes depend only on the split's
    // own data, so the result is deterministic.
    float m_ref[RT];
    float4v lsum[RT];        // row sums of P: every element of lane (n, qd) holds packed row n's
    float4v o[RT][JT];

    auto run_pass = [&]() -> bool {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            lsum[rt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < JT; ++j) o[rt][j] = float4v{0.f, 0.f, 0.f, 0.f};
        }
        if (first > last) return false;          // a short split may leave a second wave no tile
#pragma unroll
        for (int k = 0; k < G::NS; ++k) {
            const Granules gk = granules<F>(first + k * kStride, last, pages, pg0, kbase, vbase, p);
            issue_k<F, RG == 1>(gk, last, lo, ring0 + k * G::STAGE, p, lane);
            issue_v<F, RG == 1>(gk, last, lo, ring0 + k * G::STAGE, p, n, qd, lane);
        }
        int32_t j0 = first;
        int st = 0;
        // Granules of the tile that refills the current stage; the next one is looked up during
        // the current tile's MFMAs, so its block-table read does not stall the loop head.
        Granules gn = granules<F>(first + G::NS * kStride, last, pages, pg0, kbase, vbase, p);
        auto tile = [&](auto first_tag) {
            const uint32_t stage = ring0 + st * G::STAGE;
            const uint8_t* stage_bytes = ring + st * G::STAGE;
            vm_wait_tile_k<F>();                // tile k's K has landed
            TileK tk;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < G::CH; ++i)
                    tk.k[tt][i] = *reinterpret_cast<const u32x4*>(stage_bytes + tt * G::KL * 1024 + k_rd[i]);
            lds_wait_all();
            issue_k<F, RG == 1>(gn, last, lo, stage, p, lane);
            float4v sacc[2][RT];
            F::template qk<RT>(tk, sacc, qop);
            // With 256-byte rows (one wave per SIMD) V is read while the QK MFMAs run, so its LDS
            // latency overlaps them and the softmax; with 128-byte rows (two waves per SIMD, 256
            // registers) after the softmax, where the other wave covers the latency and the
            // scores no longer take registers.
            TileV tv;
            if constexpr (F::ROW == 256) {
                vm_wait_tile_v<F>();            // tile k's V has landed
                tv = read_v<F>(stage_bytes, n, qd, lane);
                lds_wait_all();
                issue_v<F, RG == 1>(gn, last, lo, stage, p, n, qd, lane);
                gn = granules<F>(j0 + (G::NS + 1) * kStride, last, pages, pg0, kbase, vbase, p);
            }
            typename F::PopT pop[RT];
            softmax_fixed<RT, F::NG, F::TILE, decltype(first_tag)::value>(sacc, j0, mask_from, lim, c, m_ref, pop, qd);
            if constexpr (F::ROW == 128) {
                vm_wait_tile_v<F>();
                tv = read_v<F>(stage_bytes, n, qd, lane);
                lds_wait_all();
                issue_v<F, RG == 1>(gn, last, lo, stage, p, n, qd, lane);
                gn = granules<F>(j0 + (G::NS + 1) * kStride, last, pages, pg0, kbase, vbase, p);
            }
            F::template pv<RT>(tv, pop, o);
            row_sums<RT>(pop, lsum);
            j0 += kStride;
            st = (st + 1) % G::NS;
        };
        tile(std::true_type{});
        while (j0 <= last) tile(std::false_type{});
        const bool over = sums_overflowed<RT>(lsum);
        vm_wait_all();   // no load may still be writing the ring when the wave moves on
        return over;
    };

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) m_ref[rt] = -INFINITY;
    bool over = run_pass();
    if constexpr (RG == 1) {
        if (over) {
            split_row_max<FMT, RT>(m_ref, j_begin, j_end, mask_from, lim, c, pages, pg0, kbase, vbase, p, qop, n, qd);
            run_pass();
        }
    } else {
        // The other row group's wave of the same token half (wave ^ 2) covers the rest of the
        // rows over the same tiles: a wave recomputes if either exceeded a reference. The flags
        // are read as wave-uniform values, so every branch here is a scalar one, and the second
        // barrier (the recompute reuses the rings) is taken by every wave or by none.
        if (lane == 0) lds.over[wave] = over ? 1 : 0;
        __syncthreads();
        const bool any = __builtin_amdgcn_readfirstlane(lds.over[0] | lds.over[1] | lds.over[2] | lds.over[3]) != 0;
        if (any) {
            if (__builtin_amdgcn_readfirstlane(lds.over[wave] | lds.over[wave ^ 2]) != 0) {
                split_row_max<FMT, RT>(m_ref, j_begin, j_end, mask_from, lim, c, pages, pg0, kbase, vbase, p, qop, n, qd);
                run_pass();
            }
            __syncthreads();
        }
    }

    // Hand-over: each pair's second wave writes its accumulators (element i of O^T tile (rt, j)
    // as row (rt*JT + j)*4 + i of 64 lanes), its references and its row sums into the
    // pair's region of the rings; the first wave reads the same lane's values back, so both
    // sides are conflict-free.
    constexpr int kXferFloats = (RT * JT * 4 + 2 * RT) * 64;
    static_assert(HP * RG * kXferFloats * 4 <= sizeof(lds.rings), "hand-over must fit in the rings");
    __syncthreads();                         // every wave is done with its ring
    float* xfer = reinterpret_cast<float*>(&lds.rings[0][0]) + (hl + (rt0 / RT) * HP) * kXferFloats;
    if (half == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int j = 0; j < JT; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) xfer[((rt * JT + j) * 4 + i) * 64 + lane] = o[rt][j][i];
            xfer[(RT * JT * 4 + rt) * 64 + lane] = m_ref[rt];
            xfer[(RT * JT * 4 + RT + rt) * 64 + lane] = lsum[rt][0];
        }
    }
    __syncthreads();
    if (half == 1) return;

    // Merge (first wave, then second) and write the head's split panel: O^T tile j holds
    // O[row n][dim F::o_dim(qd, i, j)] in element i; the four elements of a tile (transposed V
    // reads) or, for a fixed i, groups of 4 consecutive j (otherwise) are 4 consecutive dims.
    const int rows_alloc = RG == 1 ? 16 * RT : p.rows_alloc;
    float* panel = p.ws + ((int64_t)(b * p.num_kv_heads + g) * p.grid_splits + s) * p.split_floats;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (RG == 2 && 16 * (rt0 + rt) >= rows_alloc) break;     // past the head's last row tile
        const float m1 = xfer[(RT * JT * 4 + rt) * 64 + lane];
        const float l1 = xfer[(RT * JT * 4 + RT + rt) * 64 + lane];
        const float m0 = m_ref[rt];
        const float M = fmaxf(m0, m1);
        const float a0 = m0 == -INFINITY ? 0.0f : fast_exp2(m0 - M);
        const float a1 = m1 == -INFINITY ? 0.0f : fast_exp2(m1 - M);
        const int r = (rt0 + rt) * 16 + n;
        float* orow = panel + r * D;
        if constexpr (F::VTR) {
            // the four elements of a tile are four consecutive dims
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                float4v v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = merge2(a0, o[rt][j][i], a1, xfer[((rt * JT + j) * 4 + i) * 64 + lane]);
                *reinterpret_cast<float4v*>(orow + F::o_dim(qd, 0, j)) = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c4 = 0; c4 < JT / 4; ++c4) {
                    float4v v;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int j = 4 * c4 + u;
                        v[u] = merge2(a0, o[rt][j][i], a1, xfer[((rt * JT + j) * 4 + i) * 64 + lane]);
                    }
                    *reinterpret_cast<float4v*>(orow + F::o_dim(qd, i, 4 * c4)) = v;
                }
        }
        const float l = merge2(a0, lsum[rt][0], a1, l1);
        if (qd == 0) {
            panel[rows_alloc * D + r] = M;
            panel[rows_alloc * D + rows_alloc + r] = l;
        }
    }
}

// Three row groups (one-byte formats at D = 256, 33 to 48 packed rows, grids of at most one
// workgroup per CU): six waves per (slot, KV head, split), wave w taking row tile w / 2 over the
// tiles of token half w % 2. The three waves of a half share one four-stage LDS ring: the
// second of them (row tile 1; waves 2 and 3, the two waves alone on their SIMDs - waves 4 and 5
// share SIMDs with waves 0 and 1) issues the K and V loads of each tile, and one barrier per
// tile both publishes tile k (the loader has waited for its own loads) and frees the stage of
// tile k-1 (every wave has read it), which then takes tile k+3, so three tiles per half are in
// flight. Per wave this is a third of the rows' MFMA and softmax work of the one-group kernel,
// and six waves keep every SIMD busy. Every wave runs
// the same number of iterations (the shorter half idles through its last one); a half recomputes
// with exact row maxima when a row sum of any of its three waves is not finite - the rows and
// tiles whose overflow decides the recompute of the one-group wave of that half - so the result
// has the same bits as the other layouts.
constexpr int kRg3Waves = 6;
constexpr int kRg3Stages = 4;

template <int FMT>
__global__ __launch_bounds__(64 * kRg3Waves) void split_kernel_rg3(RunParams p) {
    using F = Fmt<FMT>;
    using G = Geo<F>;
    static_assert(F::ROW == 256 && F::VTR && F::NG == 2, "one-byte formats at D = 256");
    constexpr int D = F::D;
    constexpr int KS = F::KSTEPS;
    constexpr int JT = F::JT;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform within a wave
    const int half = wave & 1;                 // token half: tiles half, half + 2, ...
    const int rg = wave >> 1;                  // row tile
    const int n = lane & 15;
    const int qd = lane >> 4;

    // Workgroup order as in split_kernel (one KV head per workgroup).
    int wg = blockIdx.x;
    const int g = wg % p.num_kv_heads;
    wg /= p.num_kv_heads;
    const int s = wg % p.grid_splits;
    int b = wg / p.grid_splits;
    const int32_t L = slot_for_position(p, lane, b);
    const int32_t S = num_splits(L, p.policy);
    if (s >= S) return;                 // uniform over the workgroup
    const int32_t P = partition_len(L, p.policy);
    const int32_t j_begin = s * P;
    const int32_t j_end = min(j_begin + P, L);
    const int32_t last = j_end - 1;

    // Q^T operands and visibility limit of this wave's row tile.
    half8 qop[1][KS];
    int32_t lim[1];
    load_q_rows<F, 1>(p, b, g, rg, n, qd, L, j_end, qop, lim);
    const float c = score_scale(p, qop);
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) asm volatile("" ::"v"(qop[0][ks]), "v"(qop[0][ks + 1]));
    const int32_t mask_from = p.causal ? min(j_end, L - p.q_len + 1) : j_end;

    const uint8_t* kbase = p.k + (int64_t)g * p.k_head_stride;
    const uint8_t* vbase = p.v + (int64_t)g * p.v_head_stride;
    struct Rg3Lds {
        __attribute__((aligned(16))) uint8_t rings[2][kRg3Stages * G::STAGE];
        int32_t pages[kMaxSplitPages];
        int32_t over[kRg3Waves];
    };
    __shared__ Rg3Lds lds;
    int32_t* pages = lds.pages;
    const int32_t pg0 = stage_pages<64 * kRg3Waves>(p, b, j_begin, last, pages);
    __syncthreads();

    uint8_t* ring = lds.rings[half];
    const uint32_t ring0 = lds_addr(ring);
    const LaneOffs lo = lane_offsets<F>(p, lane, n, qd);
    uint32_t k_rd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) k_rd[i] = n * F::ROW + 16 * ((4 * i + qd) ^ G::swz(n));
    constexpr int32_t kStride = 2 * F::TILE;
    const int32_t first = j_begin + half * F::TILE;
    const int32_t ntiles = (j_end - j_begin + F::TILE - 1) / F::TILE;
    const int iters = (ntiles + 1) >> 1;               // the first half's tile count, uniform

    float m_ref[1];
    float4v lsum[1];
    float4v o[1][JT];
    // The loads of the half's tile t, issued by row group 1 (past the split's end: re-reads of the
    // last row, as in split_kernel).
    auto load_tile = [&](int32_t t, int stage) {
        const Granules gr = granules<F>(first + t * kStride, last, pages, pg0, kbase, vbase, p);
        if (rg == 1) {
            issue_k<F, true>(gr, last, lo, ring0 + stage * G::STAGE, p, lane);
            issue_v<F, true>(gr, last, lo, ring0 + stage * G::STAGE, p, n, qd, lane);
        }
    };
    // One pass over the split; every wave runs `iters` iterations with one barrier each. With
    // `compute` false the wave only keeps the ring going (its half needs no recompute).
    auto run_pass = [&](bool compute) -> bool {
        if (compute) {
            lsum[0] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < JT; ++j) o[0][j] = float4v{0.f, 0.f, 0.f, 0.f};
        }
        load_tile(0, 0);
        load_tile(1, 1);
        load_tile(2, 2);
        int32_t j0 = first;
        for (int it = 0; it < iters; ++it) {
            // The loader's loads of tile `it` have landed (tiles it+1 and it+2 may still be in flight).
            if (rg == 1) vm_wait_n<2 * (G::KLOADS + G::VLOADS)>();
            __syncthreads();                   // tile it in LDS for all; tile it-1 read by all
            load_tile(it + 3, (it + 3) % kRg3Stages);
            if (compute && j0 <= last) {
                const uint8_t* stage_bytes = ring + (it % kRg3Stages) * G::STAGE;
                TileK tk;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < G::CH; ++i)
                        tk.k[tt][i] = *reinterpret_cast<const u32x4*>(stage_bytes + tt * G::KL * 1024 + k_rd[i]);
                float4v sacc[2][1];
                F::template qk<1>(tk, sacc, qop);
                const TileV tv = read_v<F>(stage_bytes, n, qd, lane);
                typename F::PopT pop[1];
                if (it == 0) softmax_fixed<1, F::NG, F::TILE, true>(sacc, j0, mask_from, lim, c, m_ref, pop, qd);
                else softmax_fixed<1, F::NG, F::TILE, false>(sacc, j0, mask_from, lim, c, m_ref, pop, qd);
                F::template pv<1>(tv, pop, o);
                row_sums<1>(pop, lsum);
                lds_wait_all();                // this tile's reads are done before the next barrier
            }
            j0 += kStride;
        }
        vm_wait_all();
        return compute && sums_overflowed<1>(lsum);
    };

    m_ref[0] = -INFINITY;
    const bool over1 = run_pass(true);
    if (lane == 0) lds.over[wave] = over1 ? 1 : 0;
    __syncthreads();
    const bool any = __builtin_amdgcn_readfirstlane(lds.over[0] | lds.over[1] | lds.over[2] | lds.over[3] |
                                                     lds.over[4] | lds.over[5]) != 0;
    if (any) {
        // a half recomputes when any of its three waves overflowed; the other half keeps its pass
        const bool redo = __builtin_amdgcn_readfirstlane(lds.over[half] | lds.over[half + 2] | lds.over[half + 4]) != 0;
        if (redo) split_row_max<FMT, 1>(m_ref, j_begin, j_end, mask_from, lim, c, pages, pg0, kbase, vbase, p, qop, n, qd);
        run_pass(redo);
    }

    // Hand-over per row tile (second half to first) and panel rows, as in split_kernel.
    constexpr int kXferFloats = (JT * 4 + 2) * 64;
    static_assert(3 * kXferFloats * 4 <= sizeof(lds.rings), "hand-over must fit in the rings");
    __syncthreads();                         // every wave is done with the rings
    float* xfer = reinterpret_cast<float*>(&lds.rings[0][0]) + rg * kXferFloats;
    if (half == 1) {
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) xfer[(j * 4 + i) * 64 + lane] = o[0][j][i];
        xfer[(JT * 4) * 64 + lane] = m_ref[0];
        xfer[(JT * 4 + 1) * 64 + lane] = lsum[0][0];
    }
    __syncthreads();
    if (half == 1) return;
    constexpr int rows_alloc = 48;
    float* panel = p.ws + ((int64_t)(b * p.num_kv_heads + g) * p.grid_splits + s) * p.split_floats;
    const float m1 = xfer[(JT * 4) * 64 + lane];
    const float l1 = xfer[(JT * 4 + 1) * 64 + lane];
    const float m0 = m_ref[0];
    const float M = fmaxf(m0, m1);
    const float a0 = m0 == -INFINITY ? 0.0f : fast_exp2(m0 - M);
    const float a1 = m1 == -INFINITY ? 0.0f : fast_exp2(m1 - M);
    const int r = rg * 16 + n;
    float* orow = panel + r * D;
#pragma unroll
    for (int j = 0; j < JT; ++j) {
        float4v v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = merge2(a0, o[0][j][i], a1, xfer[(j * 4 + i) * 64 + lane]);
        *reinterpret_cast<float4v*>(orow + F::o_dim(qd, 0, j)) = v;
    }
    const float l = merge2(a0, lsum[0][0], a1, l1);
    if (qd == 0) {
        panel[rows_alloc * D + r] = M;
        panel[rows_alloc * D + rows_alloc + r] = l;
    }
}

// Log-sum-exp combine: one wave per packed row. Lane s loads split s's (m, l) while every lane
// already loads its D/64 dims of the first 16 splits' O, so the row costs about one memory
// round trip; the max and the denominator are wave reductions in a fixed tree, each split's
// weight is broadcast from the lane that owns it, and O is summed in split order - the FP32
// sums are bitwise reproducible.
template <int D, int DS>
__global__ __launch_bounds__(256) void combine_kernel(RunParams p) {
    constexpr int VW = D / (64 * DS);                   // dims per lane; a wave covers D / DS dims
    static_assert(VW >= 1, "at most one dim block per 64 dims");
    constexpr int kChunk = 16;
    typedef float floatv __attribute__((ext_vector_type(VW)));
    typedef _Float16 halfv __attribute__((ext_vector_type(VW)));
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row_blocks = (p.rows + 3) / 4;
    int wg = blockIdx.x;
    const int db = wg % DS;                             // dim block: dims db*D/DS ..
    wg /= DS;
    const int rb = wg % row_blocks;
    wg /= row_blocks;
    const int g = wg % p.num_kv_heads;
    const int b = wg / p.num_kv_heads;
    const int r = rb * 4 + wave;
    if (r >= p.rows) return;
    const int t = r / p.group;
    const int h = g * p.group + (r - t * p.group);

    const int32_t L = clamp_len(p.seq_lens[b], p.max_seq_len);
    const int32_t S = num_splits(L, p.policy);          // <= 64 splits per (slot, KV head)
    const float* panel0 = p.ws + (int64_t)(b * p.num_kv_heads + g) * p.grid_splits * p.split_floats;
    const int64_t m_off = (int64_t)p.rows_alloc * D + r;
    const int64_t l_off = m_off + p.rows_alloc;
    const float* orow = panel0 + r * D + db * (D / DS) + VW * lane;

    // Split indices past S read split S-1's panel (written by this run, so finite) and get
    // weight 0 from their lane, so the sums need no per-split branches.
    const int32_t s_last = S > 0 ? S - 1 : 0;
    floatv ov[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
        ov[u] = *reinterpret_cast<const floatv*>(orow + (int64_t)min(u, s_last) * p.split_floats);
    const float ms = lane < S ? panel0[(int64_t)lane * p.split_floats + m_off] : -INFINITY;
    const float ls = lane < S ? panel0[(int64_t)lane * p.split_floats + l_off] : 0.0f;

    float M = ms;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    floatv acc = {};
    float den = 0.0f;
    if (M != -INFINITY) {
        const float w = ms == -INFINITY ? 0.0f : fast_exp2(ms - M);
        den = w * ls;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
        for (int s0 = 0; s0 < S; s0 += kChunk) {
            if (s0 > 0) {
#pragma unroll
                for (int u = 0; u < kChunk; ++u)
                    ov[u] = *reinterpret_cast<const floatv*>(orow + (int64_t)min(s0 + u, s_last) * p.split_floats);
            }
#pragma unroll
            for (int u = 0; u < kChunk; ++u) {    // lane s0+u < 64 holds split s0+u's weight (0 past S)
                const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), s0 + u));
                // fused multiply-add spelled out, so every dim split (DS) rounds the sum the same way
#pragma unroll
                for (int i = 0; i < VW; ++i) acc[i] = __builtin_fmaf(wu, ov[u][i], acc[i]);
            }
        }
    }
    const float scale = den > 0.0f ? (*p.v_scale) / den : 0.0f;
    uint16_t* out = p.out + (((int64_t)b * p.q_len + t) * p.num_q_heads + h) * D + db * (D / DS) + VW * lane;
    halfv res;
#pragma unroll
    for (int i = 0; i < VW; ++i) res[i] = den > 0.0f ? (_Float16)(acc[i] * scale) : (_Float16)0.0f;
    *reinterpret_cast<halfv*>(out) = res;
}

typedef void (*KernelFn)(RunParams);

template <int FMT, int HP>
KernelFn split_for_rows(int row_tiles) {
    switch (row_tiles) {
        case 1: return split_kernel<FMT, 1, HP, 1>;
        case 2: return split_kernel<FMT, 2, HP, 1>;
        default: return split_kernel<FMT, 3, HP, 1>;
    }
}

// KV heads per split workgroup: the largest group (4 for 128-byte rows, whose 16 KB rings let
// a workgroup of 8 waves fit a CU; 2 otherwise) that divides the head count while the grid
// still gives every CU a workgroup; otherwise one head per workgroup. The heads of a group read
// neighbouring rows of the same tokens, so a CU streams longer runs of each token row (4 heads x
// 128 bytes at E4M3 D128: 4% faster than pairs). Each head's split runs the same waves, tiles
// and merge whatever the group, so the choice never changes a bit of the result.
inline int heads_per_workgroup(int num_kv_heads, int batch, int grid_splits, int num_cus, int max_hp) {
    for (int hp = max_hp; hp > 1; hp /= 2)
        if (num_kv_heads % hp == 0 && (int64_t)batch * (num_kv_heads / hp) * grid_splits >= num_cus) return hp;
    return 1;
}

// Row groups per head: two (a second pair of waves on the second half of the row tiles) for
// one-wave-per-SIMD formats with two or three row tiles when even the full grid of one-head
// workgroups gives each CU at most one, so that its four waves use all of the CU's SIMDs;
// otherwise one. The result does not depend on the choice.
inline int row_groups(bool one_wave_per_simd, int row_tiles, int hp, int batch, int num_kv_heads, int grid_splits,
                      int num_cus) {
    const bool small = (int64_t)batch * num_kv_heads * grid_splits <= num_cus;
    return one_wave_per_simd && row_tiles >= 2 && hp == 1 && small ? 2 : 1;
}

template <int FMT>
KernelFn split_for(int row_tiles, int hp, int rg) {
    if constexpr (Fmt<FMT>::ROW == 128) {
        if (hp == 4) return split_for_rows<FMT, 4>(row_tiles);
    } else {
        // two groups of ceil(row_tiles / 2) row tiles
        if (rg == 2) return row_tiles == 2 ? split_kernel<FMT, 1, 1, 2> : split_kernel<FMT, 2, 1, 2>;
    }
    return hp == 2 ? split_for_rows<FMT, 2>(row_tiles) : split_for_rows<FMT, 1>(row_tiles);
}

}  // namespace
}  // namespace attn

attn_status attn_launch_split(const attn_plan_s* plan, const attn::RunParams& p, void* stream) {
    attn::RunParams args = p;
    void* kargs[] = {&args};
    const int row_tiles = p.rows_alloc / 16;
    const bool rows128 = plan->desc.kv_dtype == ATTN_KV_E4M3 && plan->desc.head_dim == 128;
    const int hp = attn::heads_per_workgroup(p.num_kv_heads, p.batch, p.grid_splits, plan->num_cus, rows128 ? 4 : 2);
    const int rg = attn::row_groups(!rows128, row_tiles, hp, p.batch, p.num_kv_heads, p.grid_splits, plan->num_cus);
    attn::KernelFn fn;
    if (rows128)
        fn = attn::split_for<attn::kFmtE4M3D128>(row_tiles, hp, 1);
    else if (plan->desc.kv_dtype == ATTN_KV_FP16)
        fn = plan->desc.head_dim == 256 ? attn::split_for<attn::kFmtF16D256>(row_tiles, hp, rg)
                                        : attn::split_for<attn::kFmtF16D128>(row_tiles, hp, rg);
    else if (plan->desc.kv_dtype == ATTN_KV_E5M2)
        fn = attn::split_for<attn::kFmtE5M2D256>(row_tiles, hp, rg);
    else
        fn = attn::split_for<attn::kFmtE4M3D256>(row_tiles, hp, rg);
    // Three row groups for the one-byte D256 formats at three row tiles (one row tile per wave).
    int waves = attn::kWavesPerHead * hp * rg;
    if (rg == 2 && row_tiles == 3 && plan->desc.head_dim == 256 &&
        (plan->desc.kv_dtype == ATTN_KV_E4M3 || plan->desc.kv_dtype == ATTN_KV_E5M2)) {
        fn = plan->desc.kv_dtype == ATTN_KV_E4M3 ? attn::split_kernel_rg3<attn::kFmtE4M3D256>
                                                 : attn::split_kernel_rg3<attn::kFmtE5M2D256>;
        waves = attn::kRg3Waves;
    }
    // One workgroup per (slot, split, group of hp KV heads); the kernel decodes the same order.
    const unsigned grid = (unsigned)p.batch * (p.num_kv_heads / hp) * p.grid_splits;
    hipError_t e = hipLaunchKernel((const void*)fn, dim3(grid), dim3(64 * waves), kargs, 0, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_split_waves_per_simd(int kv_dtype, int head_dim) {
    return kv_dtype == ATTN_KV_E4M3 && head_dim == 128 ? attn::split_waves_per_simd<attn::kFmtE4M3D128>()
                                                       : attn::split_waves_per_simd<attn::kFmtE4M3D256>();
}

attn_status attn_launch_combine(const attn_plan_s* plan, const attn::RunParams& p, void* stream) {
    attn::RunParams args = p;
    void* kargs[] = {&args};
    // Grids with fewer row workgroups than CUs (few slots, KV heads or rows) also split each
    // row's dims over 2 or 4 waves (B8 x 131072 at Hkv 1: 7.9 -> 6.9 us; no gain on larger
    // grids). Every wave of a row computes the same weights and sums each of its dims over the
    // splits in the same order, so the dim split never changes a bit.
    const int64_t row_wgs = (int64_t)p.batch * p.num_kv_heads * ((p.rows + 3) / 4);
    const int max_ds = plan->desc.head_dim / 64;
    int ds = 1;
    while (ds < max_ds && row_wgs * ds < plan->num_cus) ds *= 2;
    const void* fn;
    if (plan->desc.head_dim == 128)
        fn = ds == 1 ? (const void*)attn::combine_kernel<128, 1> : (const void*)attn::combine_kernel<128, 2>;
    else
        fn = ds == 1 ? (const void*)attn::combine_kernel<256, 1>
                     : (ds == 2 ? (const void*)attn::combine_kernel<256, 2> : (const void*)attn::combine_kernel<256, 4>);
    const unsigned grid = (unsigned)(row_wgs * ds);
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(256), kargs, 0, (hipStream_t)stream);
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

// ---- attn_run_static: the split workspace in a static device array ----

// Device memory beyond the caller's buffers for callers that cannot allocate: the split panels of
// attn_run_static. The HIP runtime places one copy on every GPU the library runs on, for the life
// of the process. In host code this name is only a host-side stand-in: the array's device address
// on each GPU comes from hipGetSymbolAddress, and only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[ATTN_STATIC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];       // device address of `scratch` per HIP ordinal

// Device address of the static array on `device`, looked up once per device with that device
// current (each GPU holds its own copy at its own address).
attn_status scratch_address(int device, void** out) {
    if (device < 0 || device >= kMaxScratchDevices) return ATTN_E_INVALID;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[device] == nullptr) {
        int prev = -1;
        if (hipGetDevice(&prev) != hipSuccess) return ATTN_E_HIP;
        if (prev != device && hipSetDevice(device) != hipSuccess) return ATTN_E_HIP;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (prev != device && hipSetDevice(prev) != hipSuccess) return ATTN_E_HIP;
        if (e != hipSuccess || ptr == nullptr) return ATTN_E_HIP;
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return ATTN_OK;
}
}  // namespace

extern "C" attn_status attn_run_static(attn_plan_t p, const attn_args* a, void* stream) {
    if (!p || !a) return ATTN_E_INVALID;
    if (p->device == ATTN_DEVICE_HOST_ONLY) return ATTN_E_INVALID;
    if (a->batch < 1 || a->batch > p->desc.batch_capacity) return ATTN_E_INVALID;
    if (attn_plan_workspace_bytes(p, a->batch) > ATTN_STATIC_WORKSPACE_BYTES) return ATTN_E_STATIC_WORKSPACE;
    void* ws = nullptr;
    attn_status st = scratch_address(p->device, &ws);
    if (st != ATTN_OK) return st;
    attn_args local = *a;
    local.workspace = ws;
    local.workspace_bytes = ATTN_STATIC_WORKSPACE_BYTES;
    attn::RunParams rp;
    st = attn_prepare(p, &local, stream, &rp);
    if (st != ATTN_OK) return st;
    st = attn_launch_split(p, rp, stream);
    if (st != ATTN_OK) return st;
    return attn_launch_combine(p, rp, stream);
}
