// pyramid.hip -- mean-pooled key pyramid: build over a prefix and decode-time
// path update ("Block Sparse Attention with Log-Linear Complexity", section
// 3.2 eq 7-15; section 3.3 "Decoding").
//
// Summation order (shared by build and append, so the two agree bit for bit):
//   leaf i   : s = 0; for r in [iC, min(iC+C, n)): s += float(k_r); mean = s / count
//   node j>1 : s = 0; for r in [jg, min(jg+g, M_{l-1})): s += child_r; mean = s / count
// Each thread owns VEC consecutive channels of one KV head, so a row of
// H_kv * d keys is read with coalesced VEC-wide loads.
#include "pisa_device.hpp"
#include "pisa_internal.hpp"

namespace pisa {

constexpr int VEC = 4;

template <typename T> struct Vec4;
template <> struct Vec4<float> {
    __device__ __forceinline__ static f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
};
template <> struct Vec4<bf16> {
    __device__ __forceinline__ static f32x4 load(const bf16* p)
    {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
        f32x4 r;
        r[0] = from_bf16(v[0]); r[1] = from_bf16(v[1]); r[2] = from_bf16(v[2]); r[3] = from_bf16(v[3]);
        return r;
    }
};

// Mean of keys [lo, hi) of one (b, h) channel group; p points at key lo.
template <typename T>
__device__ __forceinline__ f32x4 leaf_mean(const T* p, int64_t row_stride, int64_t lo, int64_t hi)
{
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    int64_t n = hi - lo;
#pragma unroll 8
    for (int64_t r = 0; r < n; ++r) {
        f32x4 v = Vec4<T>::load(p + r * row_stride);
        s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
    }
    float c = (float)n;
    f32x4 m;
    m[0] = s[0] / c; m[1] = s[1] / c; m[2] = s[2] / c; m[3] = s[3] / c;
    return m;
}

// Mean of nodes [lo, hi) of one level; p points at node lo (row stride d).
__device__ __forceinline__ f32x4 node_mean(const float* p, int d, int64_t lo, int64_t hi)
{
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int64_t r = 0; r < hi - lo; ++r) {
        f32x4 v = *reinterpret_cast<const f32x4*>(p + r * d);
        s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
    }
    float c = (float)(hi - lo);
    f32x4 m;
    m[0] = s[0] / c; m[1] = s[1] / c; m[2] = s[2] / c; m[3] = s[3] / c;
    return m;
}

__device__ __forceinline__ void store4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }

// Levels 1 and 2. Block (j, b): leaves [j*g, min(j*g+g, M1)) and, when the
// pyramid has a level 2 for this n, level-2 node j.
template <typename T>
__global__ void build_l12_kernel(PyrArgs a, const T* __restrict__ K, int64_t n)
{
    const int tid = threadIdx.x;
    const int h = (tid * VEC) / a.d;
    const int e = (tid * VEC) % a.d;
    const int64_t j = blockIdx.x;
    const int b = blockIdx.y;
    const int64_t C = a.C, g = a.g;
    const int64_t M1 = (n + C - 1) / C;
    const int64_t row_stride = (int64_t)a.H * a.d;
    const T* kb = K + (int64_t)b * a.N_cap * row_stride + (int64_t)h * a.d + e;
    float* lev1 = a.buf + a.off[1] + (((int64_t)b * a.H + h) * a.M_cap[1]) * a.d + e;
    f32x4 s2 = {0.f, 0.f, 0.f, 0.f};
    int64_t lo_leaf = j * g, hi_leaf = (j * g + g < M1) ? j * g + g : M1;
    for (int64_t i = lo_leaf; i < hi_leaf; ++i) {
        int64_t lo = i * C, hi = (i * C + C < n) ? i * C + C : n;
        f32x4 m = leaf_mean<T>(kb + lo * row_stride, row_stride, lo, hi);
        store4(lev1 + i * a.d, m);
        s2[0] += m[0]; s2[1] += m[1]; s2[2] += m[2]; s2[3] += m[3];
    }
    if (M1 > 1) {
        float c = (float)(hi_leaf - lo_leaf);
        f32x4 m;
        m[0] = s2[0] / c; m[1] = s2[1] / c; m[2] = s2[2] / c; m[3] = s2[3] / c;
        float* lev2 = a.buf + a.off[2] + (((int64_t)b * a.H + h) * a.M_cap[2]) * a.d + e;
        store4(lev2 + j * a.d, m);
    }
}

// Level l >= 3 from level l-1. Block (j, b): node j of level l.
__global__ void build_upper_kernel(PyrArgs a, int l, int64_t n)
{
    const int tid = threadIdx.x;
    const int h = (tid * VEC) / a.d;
    const int e = (tid * VEC) % a.d;
    const int64_t j = blockIdx.x;
    const int b = blockIdx.y;
    const int64_t span_prev = (int64_t)a.C << ((l - 2) * a.g_log2);
    const int64_t M_prev = (n + span_prev - 1) / span_prev;
    const int64_t lo = j * a.g, hi = (j * a.g + a.g < M_prev) ? j * a.g + a.g : M_prev;
    const float* src = a.buf + a.off[l - 1] + (((int64_t)b * a.H + h) * a.M_cap[l - 1]) * a.d + e;
    float* dst = a.buf + a.off[l] + (((int64_t)b * a.H + h) * a.M_cap[l]) * a.d + e;
    store4(dst + j * a.d, node_mean(src + lo * a.d, a.d, lo, hi));
}

// Path update after one appended token per sequence. Block b.
template <typename T>
__global__ void append_kernel(PyrArgs a, const T* __restrict__ K, const int64_t* __restrict__ seqlen)
{
    const int tid = threadIdx.x;
    const int h = (tid * VEC) / a.d;
    const int e = (tid * VEC) % a.d;
    const int b = blockIdx.x;
    const int64_t n = seqlen[b];
    if (n < 1 || n > a.N_cap) return;  // lengths are validated by the caller; never write out of range
    const int64_t C = a.C;
    const int64_t row_stride = (int64_t)a.H * a.d;
    const int64_t c = (n - 1) / C;
    const T* kb = K + (int64_t)b * a.N_cap * row_stride + (int64_t)h * a.d + e;
    const int64_t lo = c * C, hi = (c * C + C < n) ? c * C + C : n;
    float* lev1 = a.buf + a.off[1] + (((int64_t)b * a.H + h) * a.M_cap[1]) * a.d + e;
    store4(lev1 + c * a.d, leaf_mean<T>(kb + lo * row_stride, row_stride, lo, hi));
    for (int l = 2; l <= a.L_cap; ++l) {
        const int64_t span_prev = (int64_t)a.C << ((l - 2) * a.g_log2);
        const int64_t M_prev = (n + span_prev - 1) / span_prev;
        if (M_prev <= 1) break;  // level l - 1 was the top level for this length
        const int64_t node = c >> ((l - 1) * a.g_log2);
        const int64_t clo = node * a.g, chi = (node * a.g + a.g < M_prev) ? node * a.g + a.g : M_prev;
        const float* src = a.buf + a.off[l - 1] + (((int64_t)b * a.H + h) * a.M_cap[l - 1]) * a.d + e;
        float* dst = a.buf + a.off[l] + (((int64_t)b * a.H + h) * a.M_cap[l]) * a.d + e;
        store4(dst + node * a.d, node_mean(src + clo * a.d, a.d, clo, chi));
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_build(const PyrArgs& a, const void* K, int dtype, int64_t n, hipStream_t s)
{
    const int threads = a.H * a.d / VEC;
    const int64_t C = a.C;
    const int64_t M1 = (n + C - 1) / C;
    dim3 g12((unsigned)((M1 + a.g - 1) / a.g), (unsigned)a.B);
    if (dtype == 0)
        hipLaunchKernelGGL(build_l12_kernel<float>, g12, dim3(threads), 0, s, a, (const float*)K, n);
    else
        hipLaunchKernelGGL(build_l12_kernel<bf16>, g12, dim3(threads), 0, s, a, (const bf16*)K, n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    for (int l = 3;; ++l) {
        const int64_t span = C << ((l - 1) * a.g_log2);
        const int64_t span_prev = C << ((l - 2) * a.g_log2);
        const int64_t M_prev = (n + span_prev - 1) / span_prev;
        if (M_prev <= 1) break;  // level l - 1 is the top
        const int64_t M = (n + span - 1) / span;
        hipLaunchKernelGGL(build_upper_kernel, dim3((unsigned)M, (unsigned)a.B), dim3(threads), 0, s, a, l, n);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_append(const PyrArgs& a, const void* K, int dtype, const int64_t* seqlen, hipStream_t s)
{
    const int threads = a.H * a.d / VEC;
    if (dtype == 0)
        hipLaunchKernelGGL(append_kernel<float>, dim3(a.B), dim3(threads), 0, s, a, (const float*)K, seqlen);
    else
        hipLaunchKernelGGL(append_kernel<bf16>, dim3(a.B), dim3(threads), 0, s, a, (const bf16*)K, seqlen);
    return hipGetLastError();
}

}  // namespace pisa
