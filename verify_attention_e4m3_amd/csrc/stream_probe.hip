// stream_probe.hip - plain streaming-read probe used by bench.py to measure the HBM read
// bandwidth this box actually delivers (the practical ceiling next to the 8 TB/s datasheet
// peak). Not part of the attention library or its ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every lane reads 16-byte chunks in a grid-stride loop, four loads in flight per lane, and
// folds them into one XOR so the loads cannot be removed; one word per workgroup is written.
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

extern "C" __attribute__((visibility("default"))) int attn_probe_stream_read(const void* src, size_t bytes,
                                                                              void* sink, int grid, void* stream) {
    if (!src || !sink || grid < 1 || bytes % 16) return 1;
    hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, bytes / 16,
                       (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
