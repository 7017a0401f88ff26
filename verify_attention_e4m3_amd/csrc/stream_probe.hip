// stream_probe.hip - streaming-read probes used by bench.py to measure the HBM read bandwidth
// this part actually delivers (the practical ceiling next to the 8 TB/s datasheet peak). Not
// part of the attention library or its ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Register path: every lane reads 16-byte chunks in a grid-stride loop, four loads in flight per
// lane, and folds them into one XOR so the loads cannot be removed.
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, size_t n16,
                                                  uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= src[i];
    uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int off = 32; off >= 1; off >>= 1) v ^= __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = v;
}

// LDS-DMA path, the load form the attention kernel uses: one wave per workgroup streams its own
// contiguous chunk through a two-stage LDS ring of 16 KB stages (global_load_lds_dwordx4, 16 per
// stage, streaming hint), reading each landed stage back from LDS before refilling it.
constexpr int kStage = 16384;

__device__ __forceinline__ void dma16(const uint8_t* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                 "v"(g) : "memory", "m0");
}

__global__ __launch_bounds__(64) void stream_read_lds(const uint8_t* __restrict__ src, size_t bytes_per_wave,
                                                      uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[2 * kStage];
    const uint32_t ring0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring;
    const uint8_t* base = src + (size_t)blockIdx.x * bytes_per_wave + threadIdx.x * 16;
    const int tiles = (int)(bytes_per_wave / kStage);          // >= 2, checked by the host
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int t = 0; t < 2; ++t)
        for (int i = 0; i < 16; ++i) dma16(base + (size_t)t * kStage + i * 1024, ring0 + t * kStage + i * 1024);
    for (int t = 0; t < tiles; ++t) {
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");       // stage t has landed, t + 1 in flight
        const int st = t & 1;
        const u32x4* sl = reinterpret_cast<const u32x4*>(ring + st * kStage) + threadIdx.x;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc ^= sl[i * 64];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int tn = min(t + 2, tiles - 1);                    // the last two refills re-read one stage
        for (int i = 0; i < 16; ++i) dma16(base + (size_t)tn * kStage + i * 1024, ring0 + st * kStage + i * 1024);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int off = 32; off >= 1; off >>= 1) v ^= __shfl_xor(v, off);
    if (threadIdx.x == 0) sink[blockIdx.x] = v;
}

extern "C" __attribute__((visibility("default"))) int attn_probe_stream_read(const void* src, size_t bytes,
                                                                              void* sink, int grid, void* stream) {
    if (!src || !sink || grid < 1 || bytes % 16) return 1;
    hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, bytes / 16,
                       (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

// bytes must split into `grid` chunks of whole 16 KB stages, at least two per wave; sink holds
// `grid` words.
extern "C" __attribute__((visibility("default"))) int attn_probe_stream_read_lds(const void* src, size_t bytes,
                                                                                  void* sink, int grid, void* stream) {
    if (!src || !sink || grid < 1) return 1;
    const size_t per_wave = bytes / (size_t)grid;
    if (bytes % (size_t)grid || per_wave % kStage || per_wave < 2 * (size_t)kStage) return 1;
    hipLaunchKernelGGL(stream_read_lds, dim3(grid), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)src, per_wave,
                       (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
