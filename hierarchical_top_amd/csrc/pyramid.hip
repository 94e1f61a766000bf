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

// node_mean of cnt <= g children with every child's load issued before the sums (g <= 16);
// the sums run in child order, as in node_mean.
__device__ __forceinline__ f32x4 node_mean_unrolled(const float* p, int d, int cnt, int g)
{
    f32x4 v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        if (r < g) v[r] = *reinterpret_cast<const f32x4*>(p + (r < cnt ? r : 0) * d);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r)
        if (r < cnt) { s[0] += v[r][0]; s[1] += v[r][1]; s[2] += v[r][2]; s[3] += v[r][3]; }
    const float c = (float)cnt;
    f32x4 m;
    m[0] = s[0] / c; m[1] = s[1] / c; m[2] = s[2] / c; m[3] = s[3] / c;
    return m;
}

template <typename T> struct Vec8;
template <> struct Vec8<float> {
    __device__ __forceinline__ static f32x8 load(const float* p)
    {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
        return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
};
template <> struct Vec8<bf16> {
    __device__ __forceinline__ static f32x8 load(const bf16* p)
    {
        // keys are read once per build: non-temporal, so they stream past the caches
        const bf16x8 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
        f32x8 r;
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] = from_bf16(v[k]);
        return r;
    }
};

// leaf_mean on 8 channels: the same per-channel order (tokens in increasing order, then
// one division by the count), so build and append agree bit for bit. A full leaf of CF keys
// is one straight-line sequence of loads and adds, which the compiler issues far ahead of
// the adds (a rolled loop drains its loads every few keys); cnt < CF uses the loop.
template <typename T, int CF>
__device__ __forceinline__ f32x8 leaf_mean8(const T* p, int64_t row_stride, int64_t cnt)
{
    f32x8 s = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (cnt == CF) {
#pragma unroll
        for (int r = 0; r < CF; ++r) {
            const f32x8 v = Vec8<T>::load(p + r * row_stride);
#pragma unroll
            for (int k = 0; k < 8; ++k) s[k] += v[k];
        }
    } else {
        for (int64_t r = 0; r < cnt; ++r) {
            const f32x8 v = Vec8<T>::load(p + r * row_stride);
#pragma unroll
            for (int k = 0; k < 8; ++k) s[k] += v[k];
        }
    }
    const float c = (float)cnt;
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = s[k] / c;
    return s;
}

__device__ __forceinline__ void store8(float* p, const f32x8& v)
{
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Levels 1 .. lbl of the pyramid under one level-lbl node per block (lbl = 3 when g * g <= 16
// and the leaf means fit in LDS, else 2, or 1 when even g leaves do not fit). Work item
// (leaf li of the block, channel group cg): the mean of the leaf's keys on channels
// 8 cg .. 8 cg + 7 of the H_kv * d channels of a token row (coalesced 16-byte loads, one
// leaf per wave when H_kv * d = 512). The block's leaf means (and level-2 means) stay in LDS
// for the next level; a node is the mean of its existing children in increasing order.
template <typename T, int CF>
__global__ __launch_bounds__(1024) void build_block_kernel(PyrArgs a, const T* __restrict__ K, int64_t n, int lbl)
{
    extern __shared__ __attribute__((aligned(16))) float s_m[];  // [LB][HD] leaf means, then [g][HD]
    const int HD = a.H * a.d, CG = HD / 8;
    const int g = a.g;
    const int LB = lbl == 3 ? g * g : (lbl == 2 ? g : 1);  // leaves per block
    const int64_t C = a.C;
    const int64_t node = blockIdx.x;
    const int b = blockIdx.y;
    const int64_t M1 = (n + C - 1) / C;
    const int64_t leaf0 = node * LB;
    const int nl = (int)((int64_t)LB < M1 - leaf0 ? (int64_t)LB : M1 - leaf0);  // >= 1
    const T* kb = K + (int64_t)b * a.N_cap * HD;
    for (int it = threadIdx.x; it < nl * CG; it += blockDim.x) {
        const int li = it / CG, ch = (it % CG) * 8;
        const int64_t i = leaf0 + li;
        const int64_t lo = i * C, hi = lo + C < n ? lo + C : n;
        const f32x8 m = leaf_mean8<T, CF>(kb + lo * HD + ch, HD, hi - lo);
        const int h = ch / a.d, e = ch % a.d;
        store8(a.buf + a.off[1] + ((int64_t)b * a.H + h) * a.M_cap[1] * a.d + i * a.d + e, m);
        if (lbl >= 2) store8(s_m + li * HD + ch, m);
    }
    if (lbl < 2 || M1 <= 1) return;  // block-uniform: no level 2 here, or none at this length
    __syncthreads();
    const int64_t M2 = (M1 + g - 1) / g;
    const int n2 = (nl + g - 1) / g;  // level-2 nodes under this block
    float* s2 = s_m + LB * HD;
    for (int it = threadIdx.x; it < n2 * CG; it += blockDim.x) {
        const int q = it / CG, ch = (it % CG) * 8;
        const int c0 = q * g, c1 = c0 + g < nl ? c0 + g : nl;
        f32x8 s = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int r = c0; r < c1; ++r) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(s_m + r * HD + ch);
            const f32x4 y = *reinterpret_cast<const f32x4*>(s_m + r * HD + ch + 4);
            s[0] += x[0]; s[1] += x[1]; s[2] += x[2]; s[3] += x[3];
            s[4] += y[0]; s[5] += y[1]; s[6] += y[2]; s[7] += y[3];
        }
        const float cnt = (float)(c1 - c0);
#pragma unroll
        for (int k = 0; k < 8; ++k) s[k] = s[k] / cnt;
        const int64_t j2 = node * (LB / g) + q;
        const int h = ch / a.d, e = ch % a.d;
        store8(a.buf + a.off[2] + ((int64_t)b * a.H + h) * a.M_cap[2] * a.d + j2 * a.d + e, s);
        if (lbl == 3) store8(s2 + q * HD + ch, s);
    }
    if (lbl < 3 || M2 <= 1) return;
    __syncthreads();
    for (int it = threadIdx.x; it < CG; it += blockDim.x) {  // level-3 node `node`: its n2 children
        const int ch = it * 8;
        f32x8 s = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < n2; ++q) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(s2 + q * HD + ch);
            const f32x4 y = *reinterpret_cast<const f32x4*>(s2 + q * HD + ch + 4);
            s[0] += x[0]; s[1] += x[1]; s[2] += x[2]; s[3] += x[3];
            s[4] += y[0]; s[5] += y[1]; s[6] += y[2]; s[7] += y[3];
        }
        const float cnt = (float)n2;
#pragma unroll
        for (int k = 0; k < 8; ++k) s[k] = s[k] / cnt;
        const int h = ch / a.d, e = ch % a.d;
        store8(a.buf + a.off[3] + ((int64_t)b * a.H + h) * a.M_cap[3] * a.d + node * a.d + e, s);
    }
}

// Levels l0 .. L (every level whose child level has more than one node at length n). The
// channels of a node never mix, so one single-wave block handles one group of VEC channels
// of one (KV head, sequence) through every level; each node is node_mean of its existing
// children. When level l0 fits in LDS (lds_nodes >= its node count) each level stays in LDS
// for the next one and only level l0 reads global memory; otherwise each level reads the
// previous one from global memory (the block's own stores: one wave, one CU).
__global__ __launch_bounds__(64) void build_top_kernel(PyrArgs a, int64_t n, int l0, int lds_nodes)
{
    extern __shared__ __attribute__((aligned(16))) float s_top[];  // [2][lds_nodes][VEC] ping-pong
    const int e = blockIdx.x * VEC, h = blockIdx.y, b = blockIdx.z;
    const bool in_lds = lds_nodes > 0;
    for (int l = l0, buf = 0;; ++l, buf ^= 1) {
        const int64_t span_prev = (int64_t)a.C << ((l - 2) * a.g_log2);
        const int64_t M_prev = (n + span_prev - 1) / span_prev;
        if (M_prev <= 1) break;  // level l - 1 is the top
        const int64_t M = (M_prev + a.g - 1) / a.g;
        const float* src = a.buf + a.off[l - 1] + ((int64_t)b * a.H + h) * a.M_cap[l - 1] * a.d + e;
        const float* lsrc = s_top + (size_t)(buf ^ 1) * lds_nodes * VEC;  // level l - 1 (l > l0)
        float* ldst = s_top + (size_t)buf * lds_nodes * VEC;
        float* dst = a.buf + a.off[l] + ((int64_t)b * a.H + h) * a.M_cap[l] * a.d + e;
        for (int64_t j = threadIdx.x; j < M; j += 64) {
            const int64_t lo = j * a.g, hi = lo + a.g < M_prev ? lo + a.g : M_prev;
            const f32x4 m = (in_lds && l > l0) ? node_mean_unrolled(lsrc + lo * VEC, VEC, (int)(hi - lo), a.g)
                                               : node_mean_unrolled(src + lo * a.d, a.d, (int)(hi - lo), a.g);
            store4(dst + j * a.d, m);
            if (in_lds) store4(ldst + j * VEC, m);
        }
        __syncthreads();
    }
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
    const int64_t C = a.C;
    const int64_t M1 = (n + C - 1) / C;
    const int HD = a.H * a.d;
    // levels built inside a block: as many as the block's means fit in LDS
    const size_t lds_max = 160 * 1024;
    int lbl = 1;
    if ((size_t)(a.g * a.g + a.g) * HD * 4 <= lds_max && a.g * a.g <= 16) lbl = 3;
    else if ((size_t)a.g * HD * 4 <= lds_max) lbl = 2;
    const int LB = lbl == 3 ? a.g * a.g : (lbl == 2 ? a.g : 1);
    const size_t lds = lbl == 1 ? 0 : (size_t)(LB + (lbl == 3 ? a.g : 0)) * HD * 4;
    const int items = LB * (HD / 8);
    const int threads = items >= 1024 ? 1024 : ((items + 63) / 64) * 64;
    const dim3 grid((unsigned)((M1 + LB - 1) / LB), (unsigned)a.B);
    const void* k;
    if (dtype == 0)
        k = a.C == 16 ? (const void*)build_block_kernel<float, 16>
                      : (a.C == 32 ? (const void*)build_block_kernel<float, 32> : (const void*)build_block_kernel<float, 64>);
    else
        k = a.C == 16 ? (const void*)build_block_kernel<bf16, 16>
                      : (a.C == 32 ? (const void*)build_block_kernel<bf16, 32> : (const void*)build_block_kernel<bf16, 64>);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    PyrArgs arg = a;
    int lb = lbl;
    void* args[] = {&arg, const_cast<void**>(&K), &n, &lb};
    hipError_t err = hipLaunchKernel(k, grid, dim3(threads), args, lds, s);
    if (err == hipSuccess) err = hipGetLastError();
    if (err != hipSuccess) return err;
    // the remaining levels, if level lbl + 1 exists at this length (level lbl has > 1 node)
    const int64_t span = C << (lbl - 1) * a.g_log2;
    const int64_t M_lbl = (n + span - 1) / span;
    if (M_lbl > 1) {
        const int64_t M0 = (M_lbl + a.g - 1) / a.g;  // nodes of level lbl + 1
        const size_t top_lds = (size_t)2 * M0 * VEC * 4;
        const int lds_nodes = top_lds <= 64 * 1024 ? (int)M0 : 0;
        hipLaunchKernelGGL(build_top_kernel, dim3((unsigned)(a.d / VEC), (unsigned)a.H, (unsigned)a.B), dim3(64),
                           lds_nodes ? top_lds : 0, s, a, n, lbl + 1, lds_nodes);
        err = hipGetLastError();
    }
    return err;
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
