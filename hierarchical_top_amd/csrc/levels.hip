// levels.hip -- level-synchronous prefill routing ("Block Sparse Attention with
// Log-Linear Complexity", section 3.2 eq 16-22; appendix B, "Causal masking").
//
// All (query, KV head) items advance one level at a time:
//   select (level l+1)  : kept nodes of level l+1 per item; count, per kept
//                         node, the items whose next level is ranked;
//   scan                : cluster offsets and chunk counts;
//   scatter             : cluster entries (t << 6 | slot);
//   score (level l)     : clustered MFMA scoring of the candidates of level l
//                         (levels_impl.hpp);
//   select (level l)    : Select_K of level l, and so on down to the leaves,
//                         whose select writes the ascending output.
// Counting and scatter aggregate per workgroup in LDS, so a node kept by every
// query (block 0 and the current path are forced) costs one global atomic per
// workgroup, not one per query.
#include <string.h>

#include "pisa_device.hpp"
#include "pisa_internal.hpp"

namespace pisa {

constexpr int kSelThreads = 256;
constexpr int kSelItemsPerThread = 1;
// cluster scatter: positions per thread (a workgroup's per-node cursor atomics are amortised
// over kSelThreads * kScatterItemsPerThread positions, which must divide every window)
constexpr int kScatterItemsPerThread = 4;

// Eligible existing children of node P of level lp at level lp - 1, for query t. Positions,
// node ids and counts of the level router fit 32 bits (it takes N < 2^25).
__device__ __forceinline__ int n_children(int P, int g, int M_child, int elig_max_child)
{
    const int lo = P * g;
    int hi = lo + g;
    if (hi > M_child) hi = M_child;
    if (hi > elig_max_child + 1) hi = elig_max_child + 1;
    return hi > lo ? hi - lo : 0;
}

// Forced nodes of level l for a query in leaf c (first, current and previous
// leaf's ancestors), deduplicated; returns the count (0 without causal masking).
__device__ __forceinline__ int forced_nodes(int c, int shl, bool causal, int F[3])
{
    // constant indices only, so that F stays in registers
    const int fc = c >> shl;
    const int fp = c >= 1 ? (c - 1) >> shl : 0;
    const bool hc = fc != 0;
    const bool hp = c >= 1 && fp != 0 && fp != fc;
    F[0] = 0;
    F[1] = hc ? fc : fp;
    F[2] = fp;
    return causal ? 1 + (hc ? 1 : 0) + (hp ? 1 : 0) : 0;
}

__device__ __forceinline__ bool in3(int x, const int F[3], int nF)
{
    return (nF > 0 && x == F[0]) || (nF > 1 && x == F[1]) || (nF > 2 && x == F[2]);
}

// Select_K of one level, one item per thread. KMAX >= K_top; GB = g when the
// item's candidate scores are loaded into registers up front (g in {2, 4}),
// 0 to read them from memory as they are needed (larger g).
constexpr int kSelItemsPerBlock = kSelThreads * kSelItemsPerThread;

template <int KMAX, int GB>
__device__ __forceinline__ void select_item(const SelectArgs& a, int64_t bh, int64_t t, int* s_hist, bool use_lds)
{
    const int64_t i = bh * a.N + t;
    const int K = a.K_top, g = GB ? GB : 1 << a.g_log2;
    const int l = a.level;
    const int c = (int)(t >> a.c_log2);
    const bool causal = a.causal != 0;
    const int shl = (l - 1) * a.g_log2;
    const int span_log2 = a.c_log2 + shl;
    const int M_l = (int)((a.N + ((int64_t)1 << span_log2) - 1) >> span_log2);
    const int elig_max = causal ? (int)(t >> span_log2) : M_l - 1;

    // kept nodes of level l + 1 (the parents of this level's candidates)
    int kin[KMAX];
#pragma unroll
    for (int s = 0; s < KMAX; ++s) kin[s] = -1;
    int nA = 0;
    if (a.init) {
        nA = elig_max + 1 < M_l ? elig_max + 1 : M_l;
    } else {
        const int32_t* kp = a.kept_in + i * K;
        if (K == KMAX && (KMAX & 3) == 0) {  // 16-byte loads (the list starts 16-byte aligned)
#pragma unroll
            for (int v = 0; v < KMAX / 4; ++v) {
                const int4 x = reinterpret_cast<const int4*>(kp)[v];
                kin[4 * v] = x.x; kin[4 * v + 1] = x.y; kin[4 * v + 2] = x.z; kin[4 * v + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int s = 0; s < KMAX; ++s)
                if (s < K) kin[s] = kp[s];
        }
#pragma unroll
        for (int s = 0; s < KMAX; ++s)
            if (kin[s] >= 0) nA += n_children(kin[s], g, M_l, elig_max);
    }

    int ids[KMAX];
    float val[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) { ids[j] = 0x7fffffff; val[j] = -INFINITY; }
    auto put = [&](int x, float v) {  // insert into the ascending id list
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (x < ids[j]) {
                const int ti = ids[j]; ids[j] = x; x = ti;
                const float tv = val[j]; val[j] = v; v = tv;
            }
    };
    int F[3];
    const int nF = forced_nodes(c, shl, causal, F);
    // insertion-list length: the largest R = K - nF over the wave's ranked items, a wave-uniform
    // (scalar) bound, so slots past it are skipped by scalar branches; each item then keeps the
    // first K - nF entries of its list, which are its best K - nF candidates
    const bool ranked = nA > K;
    const int Rw = ballot(ranked && nF == 0) ? K : (ballot(ranked && nF == 1) ? K - 1 : (ballot(ranked && nF == 2) ? K - 2 : K - 3));
    int nkept;
    if (nA <= K) {
        // at most K_top candidates: all are kept without scoring (section 3.2)
        nkept = (int)nA;
        if (a.init) {
            for (int x = 0; x < nA; ++x) put(x, INFINITY);
        } else {
#pragma unroll
            for (int s = 0; s < KMAX; ++s) {
                if (kin[s] < 0) continue;
                const int nc = n_children(kin[s], g, M_l, elig_max);
                for (int j = 0; j < nc; ++j) put(kin[s] * g + j, INFINITY);
            }
        }
    } else {
        const int R = K - nF;
        float bu[KMAX];
        int bi[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) { bu[j] = -INFINITY; bi[j] = 0x7fffffff; }
        const float* urow = a.u + i * (int64_t)(K * g);
        auto offer = [&](float xu, int xi) {
#pragma unroll
            for (int q = 0; q < KMAX; ++q) {
                if (q < Rw && before(xu, xi, bu[q], bi[q])) {
                    const float tu = bu[q]; bu[q] = xu; xu = tu;
                    const int ti = bi[q]; bi[q] = xi; xi = ti;
                }
            }
        };
        if constexpr (GB > 0) {
            // the whole score row in registers: K * g floats, 16-byte loads when aligned
            float ur[KMAX * GB];
            if (a.u_cols) {  // scores by node id (second level of a dense pair): the children of kin[s]
                const float* un = a.u + i * a.u_cols;
#pragma unroll
                for (int s = 0; s < KMAX; ++s) {
                    const int x = kin[s] < 0 ? 0 : kin[s];  // unused when kin[s] < 0
                    if constexpr (GB == 4) {
                        const f32x4 x4 = *reinterpret_cast<const f32x4*>(un + 4 * x);
                        ur[4 * s] = x4[0]; ur[4 * s + 1] = x4[1]; ur[4 * s + 2] = x4[2]; ur[4 * s + 3] = x4[3];
                    } else {
#pragma unroll
                        for (int j = 0; j < GB; ++j) ur[s * GB + j] = un[GB * x + j];
                    }
                }
            } else if (((K * GB) & 3) == 0) {
#pragma unroll
                for (int v = 0; v < KMAX * GB / 4; ++v) {
                    if (4 * v < K * GB) {
                        const f32x4 x4 = reinterpret_cast<const f32x4*>(urow)[v];
                        ur[4 * v] = x4[0]; ur[4 * v + 1] = x4[1]; ur[4 * v + 2] = x4[2]; ur[4 * v + 3] = x4[3];
                    }
                }
            } else {
#pragma unroll
                for (int v = 0; v < KMAX * GB; ++v)
                    if (v < K * GB) ur[v] = urow[v];
            }
#pragma unroll
            for (int s = 0; s < KMAX; ++s) {
                if (kin[s] < 0) continue;
                const int nc = n_children(kin[s], g, M_l, elig_max);
#pragma unroll
                for (int j = 0; j < GB; ++j) {
                    const int x = kin[s] * GB + j;
                    if (j < nc && !in3(x, F, nF)) offer(ur[s * GB + j], x);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < KMAX; ++s) {
                if (kin[s] < 0) continue;
                const int nc = n_children(kin[s], g, M_l, elig_max);
                // the children's scores: by slot, or by node id on a dense pair's second level
                const float* us = a.u_cols ? a.u + i * a.u_cols + (int64_t)kin[s] * g : urow + s * g;
                for (int j = 0; j < nc; ++j) {
                    const int x = kin[s] * g + j;
                    if (!in3(x, F, nF)) offer(us[j], x);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 3; ++k)
            if (k < nF) put((int)F[k], INFINITY);
        // a candidate whose score is NaN (non-finite inputs) never enters the list, so fewer
        // than R picks are possible only then: keep the real ones and pad with -1
        int npick = 0;
#pragma unroll
        for (int q = 0; q < KMAX; ++q)
            if (q < R && bi[q] != 0x7fffffff) {
                put(bi[q], bu[q]);
                ++npick;
            }
        nkept = nF + npick;
    }

    if (l == 1) {
        int32_t* out = a.idx + i * K;
        float* sc = a.score ? a.score + i * K : nullptr;
        const bool al16 = (((uintptr_t)a.idx | (uintptr_t)a.score) & 15) == 0;  // the caller's buffers
        if (K == KMAX && (KMAX & 3) == 0 && al16) {
#pragma unroll
            for (int v = 0; v < KMAX / 4; ++v) {
                int4 x;
                x.x = 4 * v < nkept ? ids[4 * v] : -1;
                x.y = 4 * v + 1 < nkept ? ids[4 * v + 1] : -1;
                x.z = 4 * v + 2 < nkept ? ids[4 * v + 2] : -1;
                x.w = 4 * v + 3 < nkept ? ids[4 * v + 3] : -1;
                reinterpret_cast<int4*>(out)[v] = x;
                if (sc) {
                    float4 y;
                    y.x = 4 * v < nkept ? val[4 * v] : -INFINITY;
                    y.y = 4 * v + 1 < nkept ? val[4 * v + 1] : -INFINITY;
                    y.z = 4 * v + 2 < nkept ? val[4 * v + 2] : -INFINITY;
                    y.w = 4 * v + 3 < nkept ? val[4 * v + 3] : -INFINITY;
                    reinterpret_cast<float4*>(sc)[v] = y;
                }
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < K) {
                const bool ok = j < nkept;
                out[j] = ok ? ids[j] : -1;
                if (sc) sc[j] = ok ? val[j] : -INFINITY;
            }
        }
        return;
    }

    int32_t* kout = a.kept_out + i * K;
    if (K == KMAX && (KMAX & 3) == 0) {
#pragma unroll
        for (int v = 0; v < KMAX / 4; ++v) {
            int4 x;
            x.x = 4 * v < nkept ? ids[4 * v] : -1;
            x.y = 4 * v + 1 < nkept ? ids[4 * v + 1] : -1;
            x.z = 4 * v + 2 < nkept ? ids[4 * v + 2] : -1;
            x.w = 4 * v + 3 < nkept ? ids[4 * v + 3] : -1;
            reinterpret_cast<int4*>(kout)[v] = x;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < K) kout[j] = j < nkept ? ids[j] : -1;
    }
    if (!a.counts) return;  // the next level is scored densely: no clusters to count

    // next level: is it ranked for this item, and which kept nodes own ranked candidates?
    const int shl2 = shl - a.g_log2;
    const int span2 = a.c_log2 + shl2;
    const int M_c = (int)((a.N + ((int64_t)1 << span2) - 1) >> span2);
    const int em_c = causal ? (int)(t >> span2) : M_c - 1;
    int nA2 = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (j < nkept) nA2 += n_children(ids[j], g, M_c, em_c);
    uint64_t mask = 0;
    if (nA2 > K) {
        int F2[3];
        const int nF2 = forced_nodes(c, shl2, causal, F2);
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < nkept) {
                const int P = ids[j];
                const int nc = n_children(P, g, M_c, em_c);
                int nforced = 0;
#pragma unroll
                for (int k = 0; k < 3; ++k) nforced += (k < nF2 && F2[k] >= P * g && F2[k] < P * g + nc) ? 1 : 0;
                if (nc > nforced) {
                    mask |= (uint64_t)1 << j;
                    if (use_lds) {
                        // forced and current-path nodes are shared by neighbouring queries:
                        // one LDS atomic per wave when every active lane adds to the same bin
                        const uint64_t act = ballot(true);
                        const int P0 = __builtin_amdgcn_readfirstlane(P);
                        if (ballot(P == P0) == act) {
                            if (lane_id() == __builtin_ctzll(act)) atomicAdd(&s_hist[P0], __popcll(act));
                        } else {
                            atomicAdd(&s_hist[P], 1);
                        }
                    } else {
                        const int64_t BH = (int64_t)a.B * a.H;
                        atomicAdd(&a.counts[((t >> a.win_log2) * BH + bh) * a.M_bins + P], 1);
                    }
                }
            }
        }
    }
    a.flags_out[i] = (int64_t)mask;
}

template <int KMAX, int GB>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a)
{
    extern __shared__ int s_hist[];
    const int64_t bh = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * kSelItemsPerBlock;
    const bool count = a.level > 1 && a.counts;
    const bool use_lds = count && a.M_bins <= kLdsBins;
    if (use_lds) {
        for (int64_t k = threadIdx.x; k < a.M_bins; k += kSelThreads) s_hist[k] = 0;
        __syncthreads();
    }
    for (int k = 0; k < kSelItemsPerThread; ++k) {
        const int64_t t = t0 + (int64_t)k * kSelThreads + threadIdx.x;
        if (t < a.N) select_item<KMAX, GB>(a, bh, t, s_hist, use_lds);
    }
    if (use_lds) {
        __syncthreads();
        const int64_t BH = (int64_t)a.B * a.H;
        int32_t* cnt = a.counts + ((t0 >> a.win_log2) * BH + bh) * a.M_bins;  // the block lies in one window
        for (int64_t k = threadIdx.x; k < a.M_bins; k += kSelThreads) {
            const int v = s_hist[k];
            if (v) atomicAdd(&cnt[k], v);
        }
    }
}

// Cluster entries: (t << 6) | slot for every flagged slot of every item, grouped
// by kept node. Positions inside a cluster are reserved per workgroup.
struct ScatterLvArgs {
    int H, K_top, win_log2;
    int64_t N, M_bins, BH;
    const int32_t* kept;
    const int64_t* flags;
    const int32_t* offsets;
    int32_t* cursor;
    int32_t* entries;
};


__global__ __launch_bounds__(kSelThreads) void scatter_lv_kernel(ScatterLvArgs a)
{
    extern __shared__ int s_mem[];
    int* s_cnt = s_mem;
    int* s_pos = s_mem + a.M_bins;
    const int64_t bh = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * (kSelThreads * kScatterItemsPerThread);
    const bool use_lds = a.M_bins <= kLdsBins;
    if (use_lds) {
        const int64_t cbase = ((t0 >> a.win_log2) * a.BH + bh) * a.M_bins;  // the block lies in one window
        const int32_t* base_off = a.offsets + cbase;
        int32_t* cur = a.cursor + cbase;
        for (int64_t k = threadIdx.x; k < a.M_bins; k += kSelThreads) s_cnt[k] = 0;
        __syncthreads();
        for (int k = 0; k < kScatterItemsPerThread; ++k) {
            const int64_t t = t0 + (int64_t)k * kSelThreads + threadIdx.x;
            if (t >= a.N) continue;
            const int64_t i = bh * a.N + t;
            const uint64_t m = (uint64_t)a.flags[i];
            for (int s = 0; s < a.K_top; ++s) {
                if (!((m >> s) & 1)) continue;
                const int P = a.kept[i * a.K_top + s];
                lds_add(&s_cnt[P], P, s_cnt);
            }
        }
        __syncthreads();
        for (int64_t k = threadIdx.x; k < a.M_bins; k += kSelThreads) {
            const int v = s_cnt[k];
            s_pos[k] = v ? base_off[k] + atomicAdd(&cur[k], v) : 0;
        }
        __syncthreads();
        for (int k = 0; k < kScatterItemsPerThread; ++k) {
            const int64_t t = t0 + (int64_t)k * kSelThreads + threadIdx.x;
            if (t >= a.N) continue;
            const int64_t i = bh * a.N + t;
            const uint64_t m = (uint64_t)a.flags[i];
            for (int s = 0; s < a.K_top; ++s) {
                if (!((m >> s) & 1)) continue;
                const int P = a.kept[i * a.K_top + s];
                const int pos = lds_add(&s_pos[P], P, s_pos);
                a.entries[pos] = (int32_t)((t << 6) | s);
            }
        }
    } else {
        for (int k = 0; k < kScatterItemsPerThread; ++k) {
            const int64_t t = t0 + (int64_t)k * kSelThreads + threadIdx.x;
            if (t >= a.N) continue;
            const int64_t i = bh * a.N + t;
            const int64_t cbase = ((t >> a.win_log2) * a.BH + bh) * a.M_bins;
            uint64_t m = (uint64_t)a.flags[i];
            while (m) {
                const int s = __builtin_ctzll(m);
                m &= m - 1;
                const int P = a.kept[i * a.K_top + s];
                const int pos = a.offsets[cbase + P] + atomicAdd(&a.cursor[cbase + P], 1);
                a.entries[pos] = (int32_t)((t << 6) | s);
            }
        }
    }
}

// Exclusive scans of cluster sizes and of their chunk counts, in two passes:
// per-block totals, then each block scans its 1024 clusters after adding the
// totals of the blocks before it.
__device__ __forceinline__ void block_scan2(int& x0, int& x1, int* s_w0, int* s_w1)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int v0 = x0, v1 = x1;
    for (int o = 1; o < 64; o <<= 1) {
        const int y0 = __shfl_up(x0, o, 64), y1 = __shfl_up(x1, o, 64);
        if (lane >= o) { x0 += y0; x1 += y1; }
    }
    if (lane == 63) { s_w0[wave] = x0; s_w1[wave] = x1; }
    __syncthreads();
    int p0 = 0, p1 = 0;
    for (int w = 0; w < wave; ++w) { p0 += s_w0[w]; p1 += s_w1[w]; }
    x0 = p0 + x0 - v0;  // exclusive
    x1 = p1 + x1 - v1;
}

__global__ __launch_bounds__(1024) void scan_totals_kernel(const int32_t* __restrict__ counts, int64_t n, int qc,
                                                           int32_t* __restrict__ sums)
{
    __shared__ int s0[16], s1[16];
    const int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x;
    const int cnt = i < n ? counts[i] : 0;
    int x0 = cnt, x1 = (cnt + qc - 1) / qc;
    for (int o = 32; o > 0; o >>= 1) { x0 += __shfl_xor(x0, o, 64); x1 += __shfl_xor(x1, o, 64); }
    if ((threadIdx.x & 63) == 0) { s0[threadIdx.x >> 6] = x0; s1[threadIdx.x >> 6] = x1; }
    __syncthreads();
    if (threadIdx.x == 0) {
        int a0 = 0, a1 = 0;
        for (int w = 0; w < 16; ++w) { a0 += s0[w]; a1 += s1[w]; }
        sums[2 * blockIdx.x] = a0;
        sums[2 * blockIdx.x + 1] = a1;
    }
}

__global__ __launch_bounds__(1024) void scan_final_kernel(const int32_t* __restrict__ counts, int64_t n, int qc,
                                                          const int32_t* __restrict__ sums,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ chunk_off)
{
    __shared__ int s_w0[16], s_w1[16], s_b[2];
    // prefix of the earlier blocks' totals
    if (threadIdx.x < 64) {
        int a0 = 0, a1 = 0;
        for (int k = threadIdx.x; k < (int)blockIdx.x; k += 64) { a0 += sums[2 * k]; a1 += sums[2 * k + 1]; }
        for (int o = 32; o > 0; o >>= 1) { a0 += __shfl_xor(a0, o, 64); a1 += __shfl_xor(a1, o, 64); }
        if (threadIdx.x == 0) { s_b[0] = a0; s_b[1] = a1; }
    }
    __syncthreads();
    const int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x;
    const int cnt = i < n ? counts[i] : 0;
    const int nch = (cnt + qc - 1) / qc;
    int x0 = cnt, x1 = nch;
    block_scan2(x0, x1, s_w0, s_w1);
    x0 += s_b[0];
    x1 += s_b[1];
    if (i < n) {
        offsets[i] = x0;
        chunk_off[i] = x1;
    }
    if (i == n - 1) {
        offsets[n] = x0 + cnt;
        chunk_off[n] = x1 + nch;
    }
}

// Chunk -> cluster map: chunk c belongs to the last cluster whose first chunk is <= c (an empty
// cluster shares its first-chunk offset with the next one). One thread per chunk: a cluster's
// chunks are written in parallel however many it has.
__global__ __launch_bounds__(256) void chunk_map_kernel(const int32_t* __restrict__ chunk_off, int64_t n,
                                                        int64_t max_chunks, int32_t* __restrict__ chunk_cl)
{
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= max_chunks || c >= chunk_off[n]) return;
    int64_t lo = 0, hi = n;  // chunk_off[lo] <= c < chunk_off[hi]
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (chunk_off[mid] <= c) lo = mid;
        else hi = mid;
    }
    chunk_cl[c] = (int32_t)lo;
}

// Output when no level is ranked (at most K_top leaf blocks): all eligible leaves.
__global__ __launch_bounds__(256) void keep_all_kernel(SelectArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.B * a.H * a.N) return;
    const int64_t t = i % a.N;
    const int64_t M1 = (a.N + ((int64_t)1 << a.c_log2) - 1) >> a.c_log2;
    const int64_t last = a.causal ? (t >> a.c_log2) : M1 - 1;
    const int64_t n = last + 1 < M1 ? last + 1 : M1;
    for (int j = 0; j < a.K_top; ++j) {
        a.idx[i * a.K_top + j] = j < n ? j : -1;
        if (a.score) a.score[i * a.K_top + j] = j < n ? INFINITY : -INFINITY;
    }
}

__global__ void fill_zero_lv_kernel(int32_t* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(fill_zero_lv_kernel, dim3(256), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_scan_chunks(const int32_t* counts, int64_t n, int qc, int32_t* block_sums, int32_t* offsets,
                              int32_t* chunk_off, int32_t* chunk_cl, int64_t max_chunks, hipStream_t s)
{
    const unsigned nsb = (unsigned)((n + 1023) / 1024);
    hipLaunchKernelGGL(scan_totals_kernel, dim3(nsb), dim3(1024), 0, s, counts, n, qc, block_sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_final_kernel, dim3(nsb), dim3(1024), 0, s, counts, n, qc, block_sums, offsets, chunk_off);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_map_kernel, dim3((unsigned)((max_chunks + 255) / 256)), dim3(256), 0, s, chunk_off, n,
                       max_chunks, chunk_cl);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
static int64_t nodes_n(int64_t n, int c_log2, int g_log2, int l)
{
    const int sh = c_log2 + (l - 1) * g_log2;
    return (n + ((int64_t)1 << sh) - 1) >> sh;
}

static hipError_t launch_select(const SelectArgs& sa, int K_top, hipStream_t s)
{
    const dim3 grid((unsigned)((sa.N + kSelItemsPerBlock - 1) / kSelItemsPerBlock), (unsigned)(sa.B * sa.H));
    const size_t lds = (sa.level > 1 && sa.counts && sa.M_bins <= kLdsBins) ? (size_t)sa.M_bins * 4 : 0;
    const int g = 1 << sa.g_log2;
#define PISA_SEL(KM, GBV) hipLaunchKernelGGL((select_kernel<KM, GBV>), grid, dim3(kSelThreads), lds, s, sa)
    if (K_top <= 8) {
        if (g == 4) PISA_SEL(8, 4);
        else if (g == 2) PISA_SEL(8, 2);
        else PISA_SEL(8, 0);
    } else if (K_top <= 16) {
        if (g == 4) PISA_SEL(16, 4);
        else if (g == 2) PISA_SEL(16, 2);
        else PISA_SEL(16, 0);
    } else {
        // K_top <= 32 (g * K_top <= 64, so g = 2): scores read as needed, which keeps the
        // 32-entry lists in registers
        PISA_SEL(32, 0);
    }
#undef PISA_SEL
    return hipGetLastError();
}

// Split of the summaries of levels l_lo .. l_hi into the two bf16 terms the MFMA operands take
// (split_layout): one thread per 8 values, in level order. The dense and sparse upper-level
// kernels then read both terms with plain loads instead of splitting the same rows in every
// workgroup.
struct SplitArgs {
    PyrArgs p;
    int l_lo, l_hi;
    int64_t nodes[PISA_MAX_LEVELS + 2];   // nodes of level l over the routed tokens
    int64_t first[PISA_MAX_LEVELS + 2];   // first 8-value piece of level l; first[l_hi + 1] = total
    int64_t off[PISA_MAX_LEVELS + 2];     // bf16 element offset of level l in out
    void* out;
};

__global__ __launch_bounds__(256) void split_kernel(SplitArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.first[a.l_hi + 1]) return;
    int l = a.l_lo;
    while (l < a.l_hi && i >= a.first[l + 1]) ++l;
    const int d8 = a.p.d >> 3;
    const int64_t k = i - a.first[l];
    const int64_t row = k / d8;  // over [B * H][nodes]
    const int c8 = (int)(k - row * d8);
    const int64_t bh = row / a.nodes[l], r = row - bh * a.nodes[l];
    const float* src = a.p.buf + a.p.off[l] + (bh * a.p.M_cap[l] + r) * a.p.d + 8 * c8;
    bf16* dst = reinterpret_cast<bf16*>(a.out) + a.off[l] + row * 2 * a.p.d + 8 * c8;
    bf16x8 hi, lo;
    split8(load8f(src), hi, lo);
    *reinterpret_cast<bf16x8*>(dst) = hi;
    *reinterpret_cast<bf16x8*>(dst + a.p.d) = lo;
}

hipError_t launch_levels(const LevelsArgs& a, int dtype, int d, hipStream_t s)
{
    const RouteArgs& r = a.r;
    const PyrArgs& p = r.p;
    const int64_t N = r.N;
    const int BH = p.B * p.H;
    hipError_t err;

    SelectArgs sa;
    memset(&sa, 0, sizeof(sa));
    sa.B = p.B; sa.H = p.H; sa.c_log2 = p.c_log2; sa.g_log2 = p.g_log2; sa.K_top = r.K_top;
    sa.causal = r.causal; sa.N = N; sa.idx = r.idx; sa.score = r.score;

    if (a.l_top == 0) {
        // at most K_top leaf blocks: every eligible leaf is kept, unscored (section 3.2)
        const int64_t items = (int64_t)BH * N;
        hipLaunchKernelGGL(keep_all_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, sa);
        return hipGetLastError();
    }

    stage_mark(PISA_STAGE_CLUSTER, false, s);
    hipLaunchKernelGGL(fill_zero_lv_kernel, dim3(256), dim3(256), 0, s, a.counts, 2 * a.cnt_total);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    stage_mark(PISA_STAGE_CLUSTER, true, s);

    // the summaries the upper levels score against, as two bf16 terms (split_layout)
    int64_t hl_off[PISA_MAX_LEVELS + 2] = {};
    split_layout(N, p.c_log2, p.g_log2, a.l_top, BH, d, hl_off);
    auto hl_rows = [&](int lv) { return reinterpret_cast<const uint16_t*>(a.rows_hl) + hl_off[lv]; };
    auto hl_h_stride = [&](int lv) { return nodes_n(N, p.c_log2, p.g_log2, lv) * 2 * d; };
    if (a.l_top >= 2) {
        SplitArgs sp;
        memset(&sp, 0, sizeof(sp));
        sp.p = p;
        sp.l_lo = 1;
        sp.l_hi = a.l_top - 1;
        int64_t pieces = 0;
        for (int lv = 1; lv <= sp.l_hi; ++lv) {
            sp.nodes[lv] = nodes_n(N, p.c_log2, p.g_log2, lv);
            sp.first[lv] = pieces;
            sp.off[lv] = hl_off[lv];
            pieces += BH * sp.nodes[lv] * (d / 8);
        }
        sp.first[sp.l_hi + 1] = pieces;
        sp.out = a.rows_hl;
        stage_mark(PISA_STAGE_UPPER, false, s);
        hipLaunchKernelGGL(split_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, sp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        stage_mark(PISA_STAGE_UPPER, true, s);
    }

    // the level above the first ranked one: every eligible node is kept
    int cur = 0;
    stage_mark(PISA_STAGE_FINAL, false, s);
    sa.level = a.l_top + 1;
    sa.init = 1;
    sa.kept_out = a.kept[cur];
    sa.flags_out = a.flags;
    sa.M_bins = nodes_n(N, p.c_log2, p.g_log2, a.l_top + 1);
    sa.counts = a.counts + a.cnt_off[a.l_top];
    sa.win_log2 = cluster_win_log2(a.l_top);
    {
        const bool dl = a.l_top >= 2 && (p.g == 2 || p.g == 4) &&
                        nodes_n(N, p.c_log2, p.g_log2, a.l_top + 1) <= kDenseParents &&
                        nodes_n(N, p.c_log2, p.g_log2, a.l_top - 1) <= kDenseRows;
        if (dl) sa.counts = nullptr;
    }
    if ((err = launch_select(sa, r.K_top, s)) != hipSuccess) return err;
    stage_mark(PISA_STAGE_FINAL, true, s);

    const int64_t per_blk = (int64_t)kSelThreads * kSelItemsPerThread;
    // levels scored densely (see kDenseParents / kDenseRows)
    auto dense_level = [&](int l) { return pisa::dense_level(N, p.c_log2, p.g_log2, l); };
    bool paired = false;  // this level's scores were written by the level above's dense pass
    for (int l = a.l_top; l >= 1; --l) {
        if (paired) {
            // second level of a dense pair: its scores are in u_pair by node id
            paired = false;
            stage_mark(PISA_STAGE_FINAL, false, s);
            sa.level = l;
            sa.init = 0;
            sa.kept_in = a.kept[cur];
            sa.u = a.u_pair;
            sa.u_cols = dense_pair_cols(N, p.c_log2, p.g_log2, l + 1);
            sa.kept_out = a.kept[cur ^ 1];
            sa.flags_out = a.flags;
            sa.M_bins = nodes_n(N, p.c_log2, p.g_log2, l);
            sa.counts = (l > 1 && !dense_level(l - 1)) ? a.counts + a.cnt_off[l - 1] : nullptr;
            sa.win_log2 = l > 1 ? cluster_win_log2(l - 1) : 0;
            if ((err = launch_select(sa, r.K_top, s)) != hipSuccess) return err;
            sa.u_cols = 0;
            stage_mark(PISA_STAGE_FINAL, true, s);
            cur ^= 1;
            continue;
        }
        if (dense_level(l)) {
            DenseArgs da;
            memset(&da, 0, sizeof(da));
            da.Q = r.Q; da.N = N; da.B = p.B; da.H = p.H; da.H_q = r.H_q; da.G = r.G; da.K_top = r.K_top; da.g = p.g;
            da.causal = r.causal;
            da.rows_hl = hl_rows(l - 1);
            da.rows_hl_h_stride = hl_h_stride(l - 1);
            da.rows_hl_b_stride = (int64_t)p.H * da.rows_hl_h_stride;
            da.rows_limit = nodes_n(N, p.c_log2, p.g_log2, l - 1);
            da.par_span_log2 = p.c_log2 + l * p.g_log2;
            da.M_par = nodes_n(N, p.c_log2, p.g_log2, l + 1);
            da.kept = a.kept[cur];
            da.sk = r.score_kind;
            da.u = a.u;
            if (dense_pair(N, p.c_log2, p.g_log2, l)) {
                // level l - 1 rides along: rows of level l - 2, parents = level-l nodes
                da.rows2_hl = hl_rows(l - 2);
                da.rows2_hl_h_stride = hl_h_stride(l - 2);
                da.rows2_hl_b_stride = (int64_t)p.H * da.rows2_hl_h_stride;
                da.rows2_limit = nodes_n(N, p.c_log2, p.g_log2, l - 2);
                da.par2_span_log2 = p.c_log2 + (l - 1) * p.g_log2;
                da.M_par2 = nodes_n(N, p.c_log2, p.g_log2, l);
                da.u2 = a.u_pair;
                da.u2_cols = dense_pair_cols(N, p.c_log2, p.g_log2, l);
                paired = true;
            }
            stage_mark(PISA_STAGE_UPPER, false, s);
            if ((err = launch_dense(da, dtype, d, s)) != hipSuccess) return err;
            stage_mark(PISA_STAGE_UPPER, true, s);
            stage_mark(PISA_STAGE_FINAL, false, s);
            sa.level = l;
            sa.init = 0;
            sa.kept_in = a.kept[cur];
            sa.u = a.u;
            sa.kept_out = a.kept[cur ^ 1];
            sa.flags_out = a.flags;
            sa.M_bins = nodes_n(N, p.c_log2, p.g_log2, l);
            sa.counts = (l > 1 && !dense_level(l - 1)) ? a.counts + a.cnt_off[l - 1] : nullptr;
            sa.win_log2 = l > 1 ? cluster_win_log2(l - 1) : 0;
            if ((err = launch_select(sa, r.K_top, s)) != hipSuccess) return err;
            stage_mark(PISA_STAGE_FINAL, true, s);
            cur ^= 1;
            continue;
        }
        const int64_t M_bins = nodes_n(N, p.c_log2, p.g_log2, l + 1);
        const int wl = cluster_win_log2(l);
        const int64_t n_win = (N + ((int64_t)1 << wl) - 1) >> wl;
        const int64_t n_clusters = n_win * BH * M_bins;
        const bool leaf = l == 1;
        // otherwise: leaf, 256 entries per workgroup sharing one node's g * C staged keys; upper
        // levels with g * g <= 16 rows per node, 32 entries per wave, rows held in registers.
        // leaf keys held in registers: bf16, g in {2, 4}, 16 / G_Q query columns per tile; upper
        // levels of the same shapes: 256 entries per workgroup, queries through LDS, the node's
        // g * g grandchildren in registers
        const bool reg_keys = leaf && dtype == 1 && (p.g == 2 || p.g == 4) && r.G <= 8;
        const bool reg_upper = !leaf && dtype == 1 && (p.g == 2 || p.g == 4) && r.G <= 8;
        const bool reg_rows = !leaf && !reg_upper && p.g * p.g <= 16;
        // one wave per chunk when a sequence's query elements index in 31 bits (offsets are 32-bit)
        const bool wave_upper = reg_upper && N * r.H_q * d < ((int64_t)1 << 31);
        const int qc = reg_rows ? kRegChunk : (reg_keys ? kLeafQC : (wave_upper ? kWaveQC : (reg_upper ? kLeafQC : 256)));
        int32_t* counts = a.counts + a.cnt_off[l];
        int32_t* cursor = a.cursor + a.cnt_off[l];

        stage_mark(PISA_STAGE_CLUSTER, false, s);
        // bound on the chunks: every entry in chunks of qc, plus one partial chunk per cluster
        const int64_t max_chunks = ((int64_t)BH * N * r.K_top + qc - 1) / qc + n_clusters;
        if ((err = launch_scan_chunks(counts, n_clusters, qc, a.block_sums, a.offsets, a.chunk_off, a.chunk_cl,
                                      max_chunks, s)) != hipSuccess)
            return err;
        ScatterLvArgs sc;
        sc.H = p.H; sc.K_top = r.K_top; sc.win_log2 = wl; sc.N = N; sc.M_bins = M_bins; sc.BH = BH;
        sc.kept = a.kept[cur]; sc.flags = a.flags; sc.offsets = a.offsets; sc.cursor = cursor;
        sc.entries = a.entries;
        {
            const int64_t per_sc = (int64_t)kSelThreads * kScatterItemsPerThread;
            static_assert(kSelThreads * kScatterItemsPerThread <= 4096, "a scatter block lies in one 2^12 window");
            const dim3 grid((unsigned)((N + per_sc - 1) / per_sc), (unsigned)BH);
            const size_t lds = M_bins <= kLdsBins ? (size_t)2 * M_bins * 4 : 0;
            hipLaunchKernelGGL(scatter_lv_kernel, grid, dim3(kSelThreads), lds, s, sc);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        stage_mark(PISA_STAGE_CLUSTER, true, s);

        ScoreArgs sc2;
        memset(&sc2, 0, sizeof(sc2));
        sc2.Q = r.Q; sc2.N = N; sc2.H = p.H; sc2.H_q = r.H_q; sc2.G = r.G; sc2.K_top = r.K_top; sc2.g = p.g;
        if (leaf) {
            sc2.rows = r.K;
            sc2.rows_b_stride = p.N_cap * p.H * d;
            sc2.rows_h_stride = d;
            sc2.row_stride = (int64_t)p.H * d;
            sc2.rows_limit = N;
            sc2.rc = p.C;
        } else {
            sc2.rows = p.buf + p.off[l - 1];
            sc2.rows_b_stride = (int64_t)p.H * p.M_cap[l - 1] * d;
            sc2.rows_h_stride = p.M_cap[l - 1] * d;
            sc2.row_stride = d;
            sc2.rows_limit = nodes_n(N, p.c_log2, p.g_log2, l - 1);
            sc2.rc = p.g;
            sc2.rows_hl = hl_rows(l - 1);
            sc2.rows_hl_h_stride = hl_h_stride(l - 1);
            sc2.rows_hl_b_stride = (int64_t)p.H * sc2.rows_hl_h_stride;
        }
        sc2.qc = qc;
        sc2.n_clusters = n_clusters;
        sc2.M_bins = M_bins;
        sc2.BH = BH;
        // leaf windows are large and shared by all XCDs (one window's queries and keys at a
        // time in the last-level cache); small upper-level windows go to one XCD each (L2)
        sc2.xcd = leaf ? 0 : 1;
        sc2.offsets = a.offsets; sc2.chunk_off = a.chunk_off; sc2.chunk_cl = a.chunk_cl; sc2.entries = a.entries;
        sc2.u = a.u;
        sc2.sk = r.score_kind;
        int64_t grid = ((int64_t)BH * N * r.K_top + qc - 1) / qc + n_clusters;  // bound on the chunks
        if (reg_rows) grid = (grid + kRegWaves - 1) / kRegWaves;
        stage_mark(leaf ? PISA_STAGE_LEAF : PISA_STAGE_UPPER, false, s);
        const int kind = reg_keys ? 3 : (wave_upper ? 6 : (reg_upper ? 4 : (leaf ? 1 : (reg_rows ? 2 : 0))));
        if ((err = launch_score(sc2, dtype, d, kind, grid, s)) != hipSuccess) return err;
        stage_mark(leaf ? PISA_STAGE_LEAF : PISA_STAGE_UPPER, true, s);

        stage_mark(PISA_STAGE_FINAL, false, s);
        sa.level = l;
        sa.init = 0;
        sa.kept_in = a.kept[cur];
        sa.u = a.u;
        sa.kept_out = a.kept[cur ^ 1];
        sa.flags_out = a.flags;
        sa.M_bins = nodes_n(N, p.c_log2, p.g_log2, l);
        sa.counts = (l > 1 && !dense_level(l - 1)) ? a.counts + a.cnt_off[l - 1] : nullptr;
        sa.win_log2 = l > 1 ? cluster_win_log2(l - 1) : 0;
        if ((err = launch_select(sa, r.K_top, s)) != hipSuccess) return err;
        stage_mark(PISA_STAGE_FINAL, true, s);
        cur ^= 1;
    }
    return hipSuccess;
}

}  // namespace pisa

namespace pisa {

hipError_t dense_bf16(const DenseArgs& a, int d, hipStream_t s);
hipError_t dense_f32(const DenseArgs& a, int d, hipStream_t s);

hipError_t launch_dense(const DenseArgs& a, int dtype, int d, hipStream_t s)
{
    return dtype == 0 ? dense_f32(a, d, s) : dense_bf16(a, d, s);
}

hipError_t score_bf16(const ScoreArgs& a, int d, int kind, int64_t grid, hipStream_t s);
hipError_t score_f32(const ScoreArgs& a, int d, int kind, int64_t grid, hipStream_t s);

hipError_t launch_score(const ScoreArgs& a, int dtype, int d, int kind, int64_t grid, hipStream_t s)
{
    return dtype == 0 ? score_f32(a, d, kind, grid, s) : score_bf16(a, d, kind, grid, s);
}

}  // namespace pisa
