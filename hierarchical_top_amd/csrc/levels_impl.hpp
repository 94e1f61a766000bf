// levels_impl.hpp -- clustered scoring kernel of the level-synchronous router
// ("Block Sparse Attention with Log-Linear Complexity", section 3.2 eq 21-22;
// section 3.3, "Training/Prefill Stage 2" and eq 23-24, applied at every level).
//
// One level at a time, every (query, KV head) item has at most K_top kept
// nodes P at level l+1; the candidates of level l are their children. The
// (item, slot of P) pairs are clustered by P. A workgroup takes one chunk of
// one cluster: it stages P's grandchildren -- the level-(l-1) summaries of the
// g children (fp32, as two bf16 terms) or, for l = 1, the raw keys of the g
// leaf blocks -- in LDS once, then scores all g children of P for every
// query of the chunk:
//   S^T = rows x (query, head) columns on 16x16x32 bf16 MFMA (A = staged rows
//   from LDS, B = the gathered queries), so that each lane holds logits of
//   four rows of one column and a candidate's log-sum-exp is mostly an
//   in-lane reduction;
//   sum of 2^(z log2(e) / sqrt(d)) over the candidate's rows, log2, sum over
//   the G_Q heads (eq 22), scaled by ln 2 -> u[item][slot * g + child].
// Without max-subtraction when the sum is a normal float (the common case),
// with it otherwise (per column, so a column's result never depends on which
// other queries share its wave).
#pragma once

#include "pisa_device.hpp"
#include "pisa_internal.hpp"

namespace pisa {

// Rows staged per workgroup and row-class selectors.
enum { RC2 = 2, RC4 = 4, RC8 = 8, RC16 = 16 };  // rows per candidate: 2, 4, 8, or a multiple of 16

constexpr int kScoreThreads = 256;
constexpr int kScoreNQT = 2;  // query tiles (of 16 columns) per wave pass

__device__ __forceinline__ int64_t xcd_chunk(int64_t blk, int64_t total)
{
    // blocks are dealt round-robin over the 8 XCDs: give each XCD one
    // contiguous range of chunks so the chunks of a cluster share an L2
    const int64_t per = total >> 3;
    if (blk < (per << 3)) return (blk & 7) * per + (blk >> 3);
    return blk;
}

// ---------------------------------------------------------------------------
// Reductions of e = 2^(scaled logit) values held by a lane (4 rows of one
// column per row tile) into per-candidate sums.
// ---------------------------------------------------------------------------
template <int D, typename T, typename TS, int RC>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a)
{
    constexpr int TA = Src<T>::TERMS;   // query terms
    constexpr int TB = Src<TS>::TERMS;  // row terms
    constexpr int KS = D / 32;
    constexpr int LDW = D + 8;          // LDS row stride (bf16 elements)
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    bf16* s_rows = reinterpret_cast<bf16*>(s_raw);

    const int64_t total = a.chunk_off[a.n_clusters];
    if ((int64_t)blockIdx.x >= total) return;
    const int64_t chunk = xcd_chunk(blockIdx.x, total);
    // cluster: the last cl with chunk_off[cl] <= chunk
    int64_t lo = 0, hi = a.n_clusters;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (a.chunk_off[mid] <= chunk) lo = mid; else hi = mid;
    }
    const int64_t cl = lo;
    const int64_t e0 = a.offsets[cl] + (chunk - a.chunk_off[cl]) * a.qc;
    const int64_t e1 = min((int64_t)a.offsets[cl + 1], e0 + a.qc);
    const int64_t P = cl % a.M_bins;
    const int64_t bh = cl / a.M_bins;
    const int h = (int)(bh % a.H);
    const int b = (int)(bh / a.H);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lg = lane >> 4;
    const int G = a.G, GT = a.G * TA, QT = 16 / GT;
    const int g = a.g, RCr = a.rc;  // children per candidate (runtime)
    const int nrows = g * RCr;      // rows of P's grandchildren
    const int nrows_pad = (nrows + 15) & ~15;  // staged rows (whole MFMA row tiles; padding is zero)
    const int64_t row0 = P * (int64_t)nrows;

    // Stage P's grandchildren rows (bf16 hi plane, and a lo plane for fp32 rows).
    const TS* rb = reinterpret_cast<const TS*>(a.rows) + (int64_t)b * a.rows_b_stride + (int64_t)h * a.rows_h_stride;
    for (int i = threadIdx.x; i < nrows_pad * (D / 8); i += kScoreThreads) {
        const int r = i / (D / 8), c8 = i % (D / 8);
        const bool ok = r < nrows && row0 + r < a.rows_limit;
        bf16x8 vh, vl;
        Src<TS>::load(rb + (ok ? (row0 + r) : 0) * a.row_stride + 8 * c8, ok, vh, vl);
        *reinterpret_cast<bf16x8*>(s_rows + r * LDW + 8 * c8) = vh;
        if constexpr (TB == 2) *reinterpret_cast<bf16x8*>(s_rows + (nrows_pad + r) * LDW + 8 * c8) = vl;
    }
    __syncthreads();

    const float scale = kLog2e * rsqrtf((float)D);
    const int col = lane & 15;
    const int qi = col / GT, term = (col % GT) / G, head = col % G;
    const int ucols = a.K_top * g;
    const int64_t nent = e1 - e0;
    const int ntiles = (int)((nent + QT - 1) / QT);
    const int nrt = nrows_pad / 16;  // row tiles

    for (int tp = wave * kScoreNQT; tp < ntiles; tp += 4 * kScoreNQT) {
        // B operands: queries of kScoreNQT tiles
        bf16x8 qb[kScoreNQT][KS];
        int ent[kScoreNQT];
        bool has[kScoreNQT];
#pragma unroll
        for (int qt = 0; qt < kScoreNQT; ++qt) {
            const int64_t e = e0 + (int64_t)(tp + qt) * QT + qi;
            has[qt] = (tp + qt) < ntiles && qi < QT && e < e1;
            ent[qt] = has[qt] ? a.entries[e] : 0;
            const int64_t tq = ent[qt] >> 6;
            const T* qp = reinterpret_cast<const T*>(a.Q) +
                          (((int64_t)b * a.N + tq) * a.H_q + (int64_t)h * G + head) * D + 8 * lg;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 vh, vl;
                Src<T>::load(qp + 32 * s, has[qt], vh, vl);
                qb[qt][s] = term == 0 ? vh : vl;
            }
        }

        if constexpr (RC == RC16) {
            // one candidate (RCr / 16 row tiles) at a time
            const int tpc = RCr / 16;
            for (int j = 0; j < g; ++j) {
                if (row0 + (int64_t)j * RCr >= a.rows_limit) break;  // P's remaining children do not exist
                f32x4 acc[4][kScoreNQT];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int qt = 0; qt < kScoreNQT; ++qt) acc[rt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    if (rt < tpc) {
                        const int r = (j * tpc + rt) * 16 + (lane & 15);
#pragma unroll
                        for (int s = 0; s < KS; ++s) {
                            const bf16x8 ah = *reinterpret_cast<const bf16x8*>(s_rows + r * LDW + 32 * s + 8 * lg);
#pragma unroll
                            for (int qt = 0; qt < kScoreNQT; ++qt) acc[rt][qt] = mfma(ah, qb[qt][s], acc[rt][qt]);
                            if constexpr (TB == 2) {
                                const bf16x8 al =
                                    *reinterpret_cast<const bf16x8*>(s_rows + (nrows_pad + r) * LDW + 32 * s + 8 * lg);
#pragma unroll
                                for (int qt = 0; qt < kScoreNQT; ++qt) acc[rt][qt] = mfma(al, qb[qt][s], acc[rt][qt]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int qt = 0; qt < kScoreNQT; ++qt) {
                    // logits of this lane's rows; fp32 queries: add the low-term column
                    float z[4][4];
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float v = acc[rt][qt][i];
                            if constexpr (TA == 2) v += shfl_xor(v, G);
                            const int64_t row = row0 + (int64_t)(j * tpc + rt) * 16 + 4 * lg + i;
                            z[rt][i] = (rt < tpc && row < a.rows_limit) ? v * scale : -INFINITY;
                        }
                    float s = 0.f;
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) s += __builtin_amdgcn_exp2f(z[rt][i]);
                    s += shfl_xor(s, 16);
                    s += shfl_xor(s, 32);
                    float l2 = __builtin_amdgcn_logf(s);
                    const bool bad = !(s > 0.f && s < INFINITY);
                    if (__builtin_expect(ballot(bad) != 0, 0)) {
                        float m = -INFINITY;
#pragma unroll
                        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) m = fmaxf(m, z[rt][i]);
                        m = fmaxf(m, shfl_xor(m, 16));
                        m = fmaxf(m, shfl_xor(m, 32));
                        float s2 = 0.f;
                        if (m != -INFINITY) {
#pragma unroll
                            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                                for (int i = 0; i < 4; ++i) s2 += __builtin_amdgcn_exp2f(z[rt][i] - m);
                        }
                        s2 += shfl_xor(s2, 16);
                        s2 += shfl_xor(s2, 32);
                        const float l2m = m == -INFINITY ? -INFINITY : m + __builtin_amdgcn_logf(s2);
                        if (bad) l2 = l2m;
                    }
                    // sum over the heads of the entry (adjacent columns)
                    for (int o = 1; o < G; o <<= 1) l2 += shfl_xor(l2, o);
                    // writer: first lane group, head 0, term 0 of each entry
                    if (has[qt] && lg == 0 && head == 0 && term == 0) {
                        const int64_t tq = ent[qt] >> 6;
                        const int slot = ent[qt] & 63;
                        a.u[((int64_t)bh * a.N + tq) * ucols + slot * g + j] = l2 * kLn2;
                    }
                }
            }
        } else {
            // all nrows (<= 64) rows; candidate of row r is r / RC
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if (rt < nrt) {
                    f32x4 acc[kScoreNQT];
#pragma unroll
                    for (int qt = 0; qt < kScoreNQT; ++qt) acc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const int r = rt * 16 + (lane & 15);
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(s_rows + r * LDW + 32 * s + 8 * lg);
#pragma unroll
                        for (int qt = 0; qt < kScoreNQT; ++qt) acc[qt] = mfma(ah, qb[qt][s], acc[qt]);
                        if constexpr (TB == 2) {
                            const bf16x8 al =
                                *reinterpret_cast<const bf16x8*>(s_rows + (nrows_pad + r) * LDW + 32 * s + 8 * lg);
#pragma unroll
                            for (int qt = 0; qt < kScoreNQT; ++qt) acc[qt] = mfma(al, qb[qt][s], acc[qt]);
                        }
                    }
#pragma unroll
                    for (int qt = 0; qt < kScoreNQT; ++qt) {
                        float z[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float v = acc[qt][i];
                            if constexpr (TA == 2) v += shfl_xor(v, G);
                            const int rr = rt * 16 + 4 * lg + i;
                            z[i] = (rr < nrows && row0 + rr < a.rows_limit) ? v * scale : -INFINITY;
                        }
                        // candidate sums: RC rows each
                        constexpr int CPL = 4 / (RC < 4 ? RC : 4);  // candidates per lane (RC = 2 -> 2)
                        float s[CPL], m[CPL];
#pragma unroll
                        for (int k = 0; k < CPL; ++k) {
                            s[k] = 0.f;
                            m[k] = -INFINITY;
#pragma unroll
                            for (int i = 0; i < 4 / CPL; ++i) {
                                s[k] += __builtin_amdgcn_exp2f(z[k * (4 / CPL) + i]);
                                m[k] = fmaxf(m[k], z[k * (4 / CPL) + i]);
                            }
                            if constexpr (RC == RC8) {
                                s[k] += shfl_xor(s[k], 16);
                                m[k] = fmaxf(m[k], shfl_xor(m[k], 16));
                            }
                        }
                        float l2[CPL];
                        bool badk[CPL];
                        bool badl = false;
#pragma unroll
                        for (int k = 0; k < CPL; ++k) {
                            // a candidate part with no existing row is never written; it is not a bad sum
                            const int rfirst = rt * 16 + 4 * lg + k * (4 / CPL);
                            const bool exists = rfirst < nrows && row0 + rfirst < a.rows_limit;
                            l2[k] = __builtin_amdgcn_logf(s[k]);
                            badk[k] = exists && !(s[k] > 0.f && s[k] < INFINITY);
                            badl = badl || badk[k];
                        }
                        if (__builtin_expect(ballot(badl) != 0, 0)) {
#pragma unroll
                            for (int k = 0; k < CPL; ++k) {
                                float s2 = 0.f;
                                if (m[k] != -INFINITY)
#pragma unroll
                                    for (int i = 0; i < 4 / CPL; ++i)
                                        s2 += __builtin_amdgcn_exp2f(z[k * (4 / CPL) + i] - m[k]);
                                if constexpr (RC == RC8) s2 += shfl_xor(s2, 16);
                                const float l2m = m[k] == -INFINITY ? -INFINITY : m[k] + __builtin_amdgcn_logf(s2);
                                if (badk[k]) l2[k] = l2m;
                            }
                        }
#pragma unroll
                        for (int k = 0; k < CPL; ++k) {
                            for (int o = 1; o < G; o <<= 1) l2[k] += shfl_xor(l2[k], o);
                            const int rfirst = rt * 16 + 4 * lg + k * (4 / CPL);  // first row of this candidate part
                            const int j = rfirst / RC;                            // candidate (child of P)
                            const bool owner = RC == RC8 ? (lg & 1) == 0 : true;
                            if (has[qt] && owner && head == 0 && term == 0 && j < g && rfirst < nrows) {
                                const int64_t tq = ent[qt] >> 6;
                                const int slot = ent[qt] & 63;
                                a.u[((int64_t)bh * a.N + tq) * ucols + slot * g + j] = l2[k] * kLn2;
                            }
                        }
                    }
                }
            }
        }
    }
}

}  // namespace pisa
