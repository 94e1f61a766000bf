// peaks.hip -- unit-throughput loops for gfx950 (include/pisa_peaks.h). Every
// loop keeps enough independent work in flight per wave that, with 8 waves per
// SIMD, the unit under test and not latency sets the rate.
#include <hip/hip_runtime.h>

#include "pisa_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void exp_loop_kernel(float* out, int iters)
{
    const int tid = blockIdx.x * kThreads + threadIdx.x;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = 0.25f + 0.01f * k + 1e-7f * threadIdx.x;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);  // converges near 0.64
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += x[k];
    out[tid] = s;
}

__device__ inline bf16x8 operand(int lane, int salt)
{
    bf16x8 v;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (__bf16)(0.001f * ((lane + k + salt) & 7));
    return v;
}

#define PISA_MFMA(k) acc##k = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a##k, b, acc##k, 0, 0, 0)
#define PISA_EXP(k) x##k = __builtin_amdgcn_exp2f(-x##k)

// Named accumulators (not an array of loop-carried vectors).
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(float* out, int iters)
{
    const int lane = threadIdx.x & 63;
    const bf16x8 b = operand(lane, 2);
    const bf16x8 a0 = operand(lane, 8), a1 = operand(lane, 9), a2 = operand(lane, 10), a3 = operand(lane, 11);
    const bf16x8 a4 = operand(lane, 12), a5 = operand(lane, 13), a6 = operand(lane, 14), a7 = operand(lane, 15);
    // initial values from a runtime quantity: constant ones make the register allocator
    // move half the accumulators around inside the loop
    const float z = 1e-9f * threadIdx.x;
    f32x4 acc0 = {z, z, z, z}, acc1 = acc0 + 1.f, acc2 = acc0 + 2.f, acc3 = acc0 + 3.f;
    f32x4 acc4 = acc0 + 4.f, acc5 = acc0 + 5.f, acc6 = acc0 + 6.f, acc7 = acc0 + 7.f;
    for (int i = 0; i < iters; ++i) {
        PISA_MFMA(0); PISA_MFMA(1); PISA_MFMA(2); PISA_MFMA(3);
        PISA_MFMA(4); PISA_MFMA(5); PISA_MFMA(6); PISA_MFMA(7);
    }
    const f32x4 s = acc0 + acc1 + acc2 + acc3 + acc4 + acc5 + acc6 + acc7;
    out[blockIdx.x * kThreads + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

__global__ __launch_bounds__(kThreads) void mix_loop_kernel(float* out, int iters)
{
    const int lane = threadIdx.x & 63;
    const bf16x8 b = operand(lane, 4);
    const bf16x8 a0 = operand(lane, 16), a1 = operand(lane, 17), a2 = operand(lane, 18), a3 = operand(lane, 19);
    const bf16x8 a4 = operand(lane, 20), a5 = operand(lane, 21), a6 = operand(lane, 22), a7 = operand(lane, 23);
    // initial values from a runtime quantity: constant ones make the register allocator
    // move half the accumulators around inside the loop
    const float z = 1e-9f * threadIdx.x;
    f32x4 acc0 = {z, z, z, z}, acc1 = acc0 + 1.f, acc2 = acc0 + 2.f, acc3 = acc0 + 3.f;
    f32x4 acc4 = acc0 + 4.f, acc5 = acc0 + 5.f, acc6 = acc0 + 6.f, acc7 = acc0 + 7.f;
    const float t = 1e-7f * threadIdx.x;
    float x0 = 0.25f + t, x1 = 0.26f + t, x2 = 0.27f + t, x3 = 0.28f + t;
    float x4 = 0.29f + t, x5 = 0.30f + t, x6 = 0.31f + t, x7 = 0.32f + t;
    for (int i = 0; i < iters; ++i) {
        PISA_MFMA(0); PISA_EXP(0); PISA_MFMA(1); PISA_EXP(1);
        PISA_MFMA(2); PISA_EXP(2); PISA_MFMA(3); PISA_EXP(3);
        PISA_MFMA(4); PISA_EXP(4); PISA_MFMA(5); PISA_EXP(5);
        PISA_MFMA(6); PISA_EXP(6); PISA_MFMA(7); PISA_EXP(7);
    }
    const f32x4 s = acc0 + acc1 + acc2 + acc3 + acc4 + acc5 + acc6 + acc7;
    out[blockIdx.x * kThreads + threadIdx.x] = s[0] + s[1] + s[2] + s[3] + x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7;
}

#undef PISA_MFMA
#undef PISA_EXP

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        size_t n)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Every thread folds its 16-byte pieces of src[0, n) (grid-stride) into one word.
__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ src, size_t n, float* out)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    uint32_t acc = 0;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {  // four loads in flight per thread
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    out[blockIdx.x * kThreads + threadIdx.x] = (float)(acc & 0xffffu);
}

// 32-bit integer hash (the "lowbias32" xorshift-multiply mix published by C. Wellons).
__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// Every wave reads rows_per_wave rows of 1 KiB (64 lanes x 16 bytes), each row drawn by
// hashing (seed, wave, k) into [0, nrows), eight rows in flight at a time.
__global__ __launch_bounds__(kThreads) void gather_kernel(const uint4* __restrict__ src, uint32_t nrows,
                                                          int rows_per_wave, uint32_t seed, float* out)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    uint32_t acc = 0;
    for (int k = 0; k < rows_per_wave; k += 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t r = mix32(seed ^ mix32(wave * (uint32_t)rows_per_wave + (uint32_t)(k + u))) % nrows;
            v[u] = src[(size_t)r * 64 + lane];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[blockIdx.x * kThreads + threadIdx.x] = (float)(acc & 0xffffu);
}

int launched(void) { return hipGetLastError() == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

int pisa_peak_exp(float* out, int32_t blocks, int32_t iters, void* stream)
{
    if (!out || blocks < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(exp_loop_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
    return launched();
}

int pisa_peak_mfma(float* out, int32_t blocks, int32_t iters, void* stream)
{
    if (!out || blocks < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
    return launched();
}

int pisa_peak_mix(float* out, int32_t blocks, int32_t iters, void* stream)
{
    if (!out || blocks < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(mix_loop_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
    return launched();
}

int pisa_peak_read(const void* src, size_t bytes, float* out, void* stream)
{
    if (!src || !out || bytes == 0 || (bytes & 15) || ((uintptr_t)src & 15)) return -1;
    hipLaunchKernelGGL(read_kernel, dim3(2048), dim3(kThreads), 0, (hipStream_t)stream, (const uint4*)src, bytes / 16,
                       out);
    return launched();
}

int pisa_peak_gather(const void* src, size_t bytes, float* out, int32_t blocks, int32_t rows_per_wave,
                     uint32_t seed, void* stream)
{
    if (!src || !out || bytes < 1024 || (bytes >> 10) > 0xffffffffu || ((uintptr_t)src & 15) || blocks < 1 ||
        rows_per_wave < 8 || (rows_per_wave & 7))
        return -1;
    hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, (const uint4*)src,
                       (uint32_t)(bytes >> 10), rows_per_wave, seed, out);
    return launched();
}

int pisa_peak_copy(const void* src, void* dst, size_t bytes, void* stream)
{
    if (!src || !dst || bytes == 0 || (bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
    const size_t n = bytes / 16;
    // a resident grid that strides over the buffer: 256 CUs x 8 workgroups
    hipLaunchKernelGGL(copy_kernel, dim3(2048), dim3(kThreads), 0, (hipStream_t)stream, (const uint4*)src,
                       (uint4*)dst, n);
    return launched();
}

}  // extern "C"
