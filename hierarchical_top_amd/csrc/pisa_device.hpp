// pisa_device.hpp -- device helpers for the gfx950 kernels of libpisa:
// bf16 conversion and hi/lo splitting, the 16x16x32 bf16 MFMA, wavefront
// primitives (shuffles, ballots, rank sorts) and pyramid geometry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pisa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// ---------------------------------------------------------------------------
// bf16: round-to-nearest-even conversion and an exact-to-2^-17 two-term split
// x ~= hi + lo of a float, so that bf16 matrix products of fp32 operands keep
// close to fp32 accuracy (the products are exact, the sums are fp32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }
__device__ __forceinline__ float from_bf16(bf16 x) { return static_cast<float>(x); }

__device__ __forceinline__ void split8(const f32x8& v, bf16x8& hi, bf16x8& lo)
{
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        bf16 h = to_bf16(v[k]);
        hi[k] = h;
        lo[k] = to_bf16(v[k] - from_bf16(h));
    }
}

__device__ __forceinline__ f32x8 load8f(const float* p)
{
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    f32x4 a = q[0], b = q[1];
    f32x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

__device__ __forceinline__ bf16x8 load8h(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ bf16x8 zero8h()
{
    bf16x8 z;
#pragma unroll
    for (int k = 0; k < 8; ++k) z[k] = to_bf16(0.0f);
    return z;
}

// Load 8 consecutive elements of a bf16 or fp32 row as bf16 operand terms.
// TERMS = 1 for bf16 sources (exact), 2 for fp32 sources (hi + lo).
// The load is issued unconditionally and `ok` = false zeroes the result, so
// that no branch (and no wait) surrounds the load: p must point at valid
// memory even when ok is false (callers clamp the row index).
template <typename T> struct Src;
template <> struct Src<bf16> {
    static constexpr int TERMS = 1;
    __device__ __forceinline__ static void load(const bf16* p, bool ok, bf16x8& hi, bf16x8& lo)
    {
        const bf16x8 v = load8h(p);
        hi = ok ? v : zero8h();
        lo = zero8h();
    }
};
template <> struct Src<float> {
    static constexpr int TERMS = 2;
    __device__ __forceinline__ static void load(const float* p, bool ok, bf16x8& hi, bf16x8& lo)
    {
        f32x8 v = load8f(p);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = ok ? v[k] : 0.f;
        split8(v, hi, lo);
    }
};

// D += A * B for one 16x16x32 bf16 tile. Lane l holds A[l%16][k-chunk l/16]
// and B[k-chunk l/16][l%16] (8 consecutive k each); D lane l holds rows
// 4*(l/16) + i, i = 0..3, of column l % 16.
__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Wavefront primitives.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int shfl_xor(int v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, kWave); }
__device__ __forceinline__ int shfl(int v, int src) { return __shfl(v, src, kWave); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int rank_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Move each lane's value to lane dst (a permutation of 0..63).
__device__ __forceinline__ int permute_to(int dst, int v) { return __builtin_amdgcn_ds_permute(dst << 2, v); }
__device__ __forceinline__ float permute_to(int dst, float v)
{
    return __int_as_float(__builtin_amdgcn_ds_permute(dst << 2, __float_as_int(v)));
}

// Stable compaction: lanes with keep=true move, in lane order, to lanes
// 0..count-1; the others fill the remaining lanes. Returns the count.
__device__ __forceinline__ int compact(bool keep, int& a, float& b)
{
    int lane = lane_id();
    uint64_t m = ballot(keep);
    int cnt = __popcll(m);
    int r = rank_below(m);
    int dst = keep ? r : cnt + (lane - r);
    a = permute_to(dst, a);
    b = permute_to(dst, b);
    return cnt;
}

// Cross-lane moves without the LDS crossbar: DPP quad permutes (xor 1, xor 2)
// and gfx950's permlane swaps, which exchange rows of 16 lanes (xor 16) and
// halves of the wave (xor 32) in one VALU instruction each.
__device__ __forceinline__ float dpp_xor1(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// v + v of lane ^ 16, and v + v of lane ^ 32.
__device__ __forceinline__ float add_xor16(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_xor32(float v)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor16(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
// Sum over aligned groups of G adjacent lanes (G a power of two <= 16).
// Adds one to the LDS counter p_mine (= base_arr + P) and returns its old value, with one
// atomic per wave when every active lane targets the same counter (the lanes then take
// consecutive values in lane order).
__device__ __forceinline__ int lds_add(int* p_mine, int P, int* base_arr)
{
    const uint64_t act = ballot(true);
    const int P0 = __builtin_amdgcn_readfirstlane(P);
    if (ballot(P == P0) == act) {
        const int leader = __builtin_ctzll(act);
        int old = 0;
        if (lane_id() == leader) old = atomicAdd(&base_arr[P0], __popcll(act));
        old = __shfl(old, leader, 64);
        return old + rank_below(act);
    }
    return atomicAdd(p_mine, 1);
}

__device__ __forceinline__ float sum_adjacent(float v, int G)
{
    if (G >= 2) v += dpp_xor1(v);
    if (G >= 4) v += dpp_xor2(v);
    for (int o = 4; o < G; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Maximum / sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_max(float x, int width)
{
    for (int o = 1; o < width; o <<= 1) x = fmaxf(x, shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float group_sum(float x, int width)
{
    for (int o = 1; o < width; o <<= 1) x += shfl_xor(x, o);
    return x;
}

// Selection order: higher key first; equal keys -> lower id first.
__device__ __forceinline__ bool before(float ka, int ia, float kb, int ib)
{
    return ka > kb || (ka == kb && ia < ib);
}

// Moves every lane's (key, id) to the lane of its rank in selection order:
// each live lane counts the live lanes before it (scalar reads of their key
// and id, one per live lane), then one permute places all lanes. Live lanes
// come first, in selection order; the others follow in lane order. Ids must be
// distinct among live lanes.
__device__ __forceinline__ void rank_sort(float& key, int& id, uint64_t live)
{
    int rank = 0;
    for (uint64_t m = live; m; m &= m - 1) {
        const int j = __builtin_ctzll(m);
        const float kj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(key), j));
        const int ij = __builtin_amdgcn_readlane(id, j);
        rank += before(kj, ij, key, id) ? 1 : 0;
    }
    if (!((live >> lane_id()) & 1)) rank = __popcll(live) + rank_below(~live);
    key = __int_as_float(__builtin_amdgcn_ds_permute(rank << 2, __float_as_int(key)));
    id = __builtin_amdgcn_ds_permute(rank << 2, id);
}

// The live lanes' ids in ascending order in lanes 0.., carrying a float
// payload (ids distinct among live lanes); the other lanes follow.
__device__ __forceinline__ void rank_sort_ids(int& id, float& val, uint64_t live)
{
    int rank = 0;
    for (uint64_t m = live; m; m &= m - 1) rank += __builtin_amdgcn_readlane(id, __builtin_ctzll(m)) < id ? 1 : 0;
    if (!((live >> lane_id()) & 1)) rank = __popcll(live) + rank_below(~live);
    val = __int_as_float(__builtin_amdgcn_ds_permute(rank << 2, __float_as_int(val)));
    id = __builtin_amdgcn_ds_permute(rank << 2, id);
}

// ---------------------------------------------------------------------------
// Pyramid geometry (C and g are powers of two): a level-l node covers
// C * g^(l-1) tokens; M_l(n) = ceil(n / span_l); the top level L(n) is the
// first level with one node.
// ---------------------------------------------------------------------------
struct Geo {
    int c_log2, g_log2;
    __device__ __forceinline__ int span_log2(int l) const { return c_log2 + (l - 1) * g_log2; }
    __device__ __forceinline__ int64_t nodes(int64_t n, int l) const
    {
        int s = span_log2(l);
        return (n + ((int64_t)1 << s) - 1) >> s;
    }
    __device__ __forceinline__ int top(int64_t n) const
    {
        int l = 1;
        while (nodes(n, l) > 1) ++l;
        return l;
    }
};

}  // namespace pisa
