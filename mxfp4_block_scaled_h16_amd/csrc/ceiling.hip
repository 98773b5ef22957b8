// Practical ceilings of gfx950 for the two bounds of the library's kernels: HBM streaming
// (read, write, copy) and the scaled FP4 matrix core. Built as its own library so that the
// measured kernels share nothing with the product kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxfp4_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kStreamThreads = 256;
// launch shapes chosen by a sweep on MI355X (1 GiB buffers, 1024-8192 workgroups, 4 or 8 loads
// in flight, plain or nontemporal accesses): nontemporal grid-stride reads and copies with 8192
// workgroups (6.3 and 5.2 TB/s, the copy as fast as the runtime's device-to-device copy) and
// plain stores with 2048 workgroups (4.6 TB/s) were the fastest
constexpr int kReadBlocks = 8192, kWriteBlocks = 2048, kCopyBlocks = 8192;
constexpr int kFmtFp4 = 4;  // E2M1 operand format of the scaled MFMA

// grid-stride over 16-byte words, four loads in flight per lane
__global__ __launch_bounds__(kStreamThreads) void read_kernel(const u32x4 *__restrict__ src, size_t n,
                                                              uint32_t never, uint32_t *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * kStreamThreads;
    size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i), b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n; i += stride) acc ^= src[i];
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == never) sink[0] = x;
}

__global__ __launch_bounds__(kStreamThreads) void write_kernel(u32x4 *__restrict__ dst, size_t n, uint32_t pattern)
{
    const size_t stride = (size_t)gridDim.x * kStreamThreads;
    const u32x4 v = {pattern, pattern, pattern, pattern};
    for (size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += stride) dst[i] = v;
}

__global__ __launch_bounds__(kStreamThreads) void copy_kernel(const u32x4 *__restrict__ src,
                                                              u32x4 *__restrict__ dst, size_t n)
{
    const size_t stride = (size_t)gridDim.x * kStreamThreads;
    size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i), b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        __builtin_nontemporal_store(a, dst + i);
        __builtin_nontemporal_store(b, dst + i + stride);
        __builtin_nontemporal_store(c, dst + i + 2 * stride);
        __builtin_nontemporal_store(d, dst + i + 3 * stride);
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

// 32-bit finaliser of MurmurHash3: seeds the operand bit patterns (any byte is a valid pair of
// E2M1 codes)
__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x85EBCA6Bu;
    x ^= x >> 13;
    x *= 0xC2B2AE35u;
    x ^= x >> 16;
    return x;
}

__device__ __forceinline__ v8i widen(const u32x4 &v)
{
    return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// 8 wavefronts, each with a 4 x 2 set of 32x32 accumulators (the GEMM's wavefront tile);
// 512 threads and more than 128 VGPRs keep it to one workgroup per compute unit
__global__ __launch_bounds__(512, 1) void mfma_kernel(int iters, uint32_t seed, float *__restrict__ sink)
{
    const uint32_t gid = blockIdx.x * 512u + threadIdx.x;
    uint32_t h = mix32(seed ^ mix32(gid + 0x9E3779B9u));
    u32x4 fa[4], fb[2];
    uint32_t sa[4], sb[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fa[i] = u32x4{h = mix32(h + 1u), h = mix32(h + 1u), h = mix32(h + 1u), h = mix32(h + 1u)};
        sa[i] = 120u + (h = mix32(h + 1u)) % 15u;  // scales 2^-7 .. 2^7: finite products
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        fb[j] = u32x4{h = mix32(h + 1u), h = mix32(h + 1u), h = mix32(h + 1u), h = mix32(h + 1u)};
        sb[j] = 120u + (h = mix32(h + 1u)) % 15u;
    }
    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    uint32_t m = mix32(h);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    widen(fb[j]), widen(fa[i]), acc[i][j], kFmtFp4, kFmtFp4, 0, (int)sb[j], 0, (int)sa[i]);
        // new operand bits for the next round (about half of them flip)
        m = m * 1664525u + 1013904223u;
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] ^= m;
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] ^= ~m;
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[i][j][e];
    sink[gid] = s;
}

int launched(hipError_t e) { return e == hipSuccess ? 0 : 3; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int mxfp4_ceiling_read(const void *src, size_t bytes, uint32_t never, uint32_t *sink, void *stream)
{
    if (!src || !sink) return 1;
    if (bytes == 0 || bytes % 16 || !aligned16(src)) return 2;
    read_kernel<<<kReadBlocks, kStreamThreads, 0, (hipStream_t)stream>>>(
        static_cast<const u32x4 *>(src), bytes / 16, never, sink);
    return launched(hipGetLastError());
}

extern "C" int mxfp4_ceiling_write(void *dst, size_t bytes, uint32_t pattern, void *stream)
{
    if (!dst) return 1;
    if (bytes == 0 || bytes % 16 || !aligned16(dst)) return 2;
    write_kernel<<<kWriteBlocks, kStreamThreads, 0, (hipStream_t)stream>>>(static_cast<u32x4 *>(dst), bytes / 16,
                                                                            pattern);
    return launched(hipGetLastError());
}

extern "C" int mxfp4_ceiling_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (!src || !dst) return 1;
    if (bytes == 0 || bytes % 16 || !aligned16(src) || !aligned16(dst)) return 2;
    copy_kernel<<<kCopyBlocks, kStreamThreads, 0, (hipStream_t)stream>>>(
        static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), bytes / 16);
    return launched(hipGetLastError());
}

extern "C" int mxfp4_ceiling_mfma(int workgroups, int iters, uint32_t seed, float *sink, void *stream)
{
    if (!sink) return 1;
    if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 20)) return 2;
    mfma_kernel<<<workgroups, 512, 0, (hipStream_t)stream>>>(iters, seed, sink);
    return launched(hipGetLastError());
}
