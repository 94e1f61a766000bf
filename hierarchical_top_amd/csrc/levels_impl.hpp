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
// The sum is taken without max-subtraction when it is a normal float (the
// common case) and with it otherwise, per column, so a column's result never
// depends on which other queries share its wave.
#pragma once

#include "pisa_device.hpp"
#include "pisa_internal.hpp"
#include "stream.hpp"

namespace pisa {

constexpr int kScoreNQT = 2;  // query tiles (of 16 columns) per wave pass

__device__ __forceinline__ int64_t xcd_chunk(int64_t blk, int64_t total)
{
    // blocks are dealt round-robin over the 8 XCDs: give each XCD one
    // contiguous range of chunks so the chunks of a window share an L2
    const int64_t per = total >> 3;
    if (blk < (per << 3)) return (blk & 7) * per + (blk >> 3);
    return blk;
}

// log2 of sum_i 2^z_i over the N values of z (all finite or -inf), plus the
// cross-lane partners selected by XMASK (bit 0: lanes ^ 16, bit 1: lanes ^ 32).
// Fast path without max-subtraction; exact-max path when the plain sum is not
// a normal positive float. `exists` = the candidate has at least one row.
template <int N, int XMASK, typename F>
__device__ __forceinline__ float lse2f(F zf, bool exists)
{
    float e[N];
#pragma unroll
    for (int i = 0; i < N; ++i) e[i] = __builtin_amdgcn_exp2f(zf(i));
#pragma unroll
    for (int w = 1; w < N; w <<= 1)  // pairwise tree: independent adds
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w) e[i] += e[i + w];
    float s = e[0];
    if constexpr (XMASK & 1) s = add_xor16(s);
    if constexpr (XMASK & 2) s = add_xor32(s);
    float l2 = __builtin_amdgcn_logf(s);
    const bool bad = exists && !(s > 0.f && s < INFINITY);
    if (__builtin_expect(ballot(bad) != 0, 0)) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < N; ++i) m = fmaxf(m, zf(i));
        if constexpr (XMASK & 1) m = max_xor16(m);
        if constexpr (XMASK & 2) m = max_xor32(m);
        float s2 = 0.f;
        if (m != -INFINITY) {
#pragma unroll
            for (int i = 0; i < N; ++i) s2 += __builtin_amdgcn_exp2f(zf(i) - m);
        }
        if constexpr (XMASK & 1) s2 = add_xor16(s2);
        if constexpr (XMASK & 2) s2 = add_xor32(s2);
        const float l2m = m == -INFINITY ? -INFINITY : m + __builtin_amdgcn_logf(s2);
        if (bad) l2 = l2m;
    }
    return l2;
}

template <int N, int XMASK>
__device__ __forceinline__ float lse2(const float* z, bool exists)
{
    float e[N];
#pragma unroll
    for (int i = 0; i < N; ++i) e[i] = __builtin_amdgcn_exp2f(z[i]);
#pragma unroll
    for (int w = 1; w < N; w <<= 1)  // pairwise tree: independent adds
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w) e[i] += e[i + w];
    float s = e[0];
    if constexpr (XMASK & 1) s = add_xor16(s);
    if constexpr (XMASK & 2) s = add_xor32(s);
    float l2 = __builtin_amdgcn_logf(s);
    const bool bad = exists && !(s > 0.f && s < INFINITY);
    if (__builtin_expect(ballot(bad) != 0, 0)) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < N; ++i) m = fmaxf(m, z[i]);
        if constexpr (XMASK & 1) m = max_xor16(m);
        if constexpr (XMASK & 2) m = max_xor32(m);
        float s2 = 0.f;
        if (m != -INFINITY) {
#pragma unroll
            for (int i = 0; i < N; ++i) s2 += __builtin_amdgcn_exp2f(z[i] - m);
        }
        if constexpr (XMASK & 1) s2 = add_xor16(s2);
        if constexpr (XMASK & 2) s2 = add_xor32(s2);
        const float l2m = m == -INFINITY ? -INFINITY : m + __builtin_amdgcn_logf(s2);
        if (bad) l2 = l2m;
    }
    return l2;
}

// Block score of one candidate and query head from its logits in base-2
// units (z log2(e), rows that do not exist = -inf), returned in base-2 units
// (the caller multiplies by ln 2). SK selects the score (section 4.4, appendix
// A.2): 0 = log-sum-exp (PISA, eq 21); 1 = the mean of the valid logits
// (PISA-1, eq 33); 2 = that mean plus half their population variance
// (PISA-2, eq 34), the variance taken about the mean in a second pass. The
// variance of base-2 logits is ln 2^-2 times the natural one, hence the ln 2
// factor on it. XMASK as in lse2f: the candidate's rows span those lanes.
template <int SK, int N, int XMASK, typename F>
__device__ __forceinline__ float block_score2f(F zf, bool exists)
{
    if constexpr (SK == 0) {
        return lse2f<N, XMASK>(zf, exists);
    } else {
        float s = 0.f, c = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float z = zf(i);
            const bool v = z > -INFINITY;
            s += v ? z : 0.f;
            c += v ? 1.f : 0.f;
        }
        if constexpr (XMASK & 1) { s = add_xor16(s); c = add_xor16(c); }
        if constexpr (XMASK & 2) { s = add_xor32(s); c = add_xor32(c); }
        const float mu = c > 0.f ? s / c : 0.f;
        if constexpr (SK == 1) {
            return c > 0.f ? mu : -INFINITY;
        } else {
            float q = 0.f;
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const float z = zf(i);
                const float dz = z - mu;
                q += z > -INFINITY ? dz * dz : 0.f;
            }
            if constexpr (XMASK & 1) q = add_xor16(q);
            if constexpr (XMASK & 2) q = add_xor32(q);
            return c > 0.f ? mu + (0.5f * kLn2) * (q / c) : -INFINITY;
        }
    }
}

template <int SK, int N, int XMASK>
__device__ __forceinline__ float block_score2(const float* z, bool exists)
{
    if constexpr (SK == 0) return lse2<N, XMASK>(z, exists);
    else return block_score2f<SK, N, XMASK>([&](int i) { return z[i]; }, exists);
}

// RC: rows per candidate (g for summary rows, C for key rows), a compile-time
// constant in {2, 4, 8, 16, 32, 64}. WAVES: waves per workgroup.
template <int D, typename T, typename TS, int RC, int WAVES, int SK>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(4))) void score_kernel(ScoreArgs a)
{
    constexpr int TA = Src<T>::TERMS;   // query terms
    constexpr int TB = Src<TS>::TERMS;  // row terms
    constexpr int KS = D / 32;
    constexpr int LDW = D + 8;          // LDS row stride (bf16 elements)
    constexpr int TPC = RC >= 16 ? RC / 16 : 1;
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    bf16* s_rows = reinterpret_cast<bf16*>(s_raw);
    int* s_ent = reinterpret_cast<int*>(s_raw + (size_t)TB * ((a.g * RC + 15) & ~15) * LDW * 2);

    const int64_t total = a.chunk_off[a.n_clusters];
    if ((int64_t)blockIdx.x >= total) return;
    const int64_t chunk = a.xcd ? xcd_chunk(blockIdx.x, total) : (int64_t)blockIdx.x;
    const int64_t cl = a.chunk_cl[chunk];
    const int e0 = a.offsets[cl] + (int)(chunk - a.chunk_off[cl]) * a.qc;
    const int e1 = min(a.offsets[cl + 1], e0 + a.qc);
    const int64_t P = cl % a.M_bins;
    const int64_t bh = (cl / a.M_bins) % a.BH;
    const int h = (int)(bh % a.H);
    const int b = (int)(bh / a.H);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lg = lane >> 4;
    const int G = a.G, GT = a.G * TA, QT = 16 / GT;
    const int g = a.g;
    const int nrows = g * RC;                       // rows of P's grandchildren
    const int nrows_pad = (nrows + 15) & ~15;       // staged rows (whole MFMA row tiles; padding is zero)
    const int64_t row0 = P * (int64_t)nrows;
    const int64_t rem = a.rows_limit - row0;        // rows of P that exist
    const int lim_rows = rem < nrows ? (int)rem : nrows;

    const float scale = kLog2e * rsqrtf((float)D);
    const int col = lane & 15;
    const int qi = col / GT, term = (col % GT) / G, head = col % G;
    const bool writer_col = lg == 0 && head == 0 && term == 0;
    const int ucols = a.K_top * g;
    const int ntiles = (e1 - e0 + QT - 1) / QT;
    const T* Qb = reinterpret_cast<const T*>(a.Q) + (int64_t)b * a.N * a.H_q * D + (h * G + head) * D + 8 * lg;
    const uint32_t qrow = (uint32_t)(a.H_q * D);
    float* ub = a.u + bh * a.N * ucols;

    // one pass = kScoreNQT query tiles of this wave; loaded one pass ahead of its use
    struct QPass {
        bf16x8 qb[kScoreNQT][KS];
        bool has[kScoreNQT];
        float* up[kScoreNQT];
    };
    auto load_pass = [&](int tp, QPass& Pq) {
        auto& qb = Pq.qb;
        auto& has = Pq.has;
        auto& up = Pq.up;
        // B operands: queries of kScoreNQT tiles. Lanes past the chunk's end
        // load the last entry's query (valid memory) and never write.
#pragma unroll
        for (int qt = 0; qt < kScoreNQT; ++qt) {
            const int e = e0 + (tp + qt) * QT + qi;
            has[qt] = e < e1;
            const int ent = s_ent[(has[qt] ? e : e1 - 1) - e0];
            const uint32_t tq = (uint32_t)ent >> 6;
            const T* qp = Qb + (uint64_t)tq * qrow;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 vh, vl;
                Src<T>::load(qp + 32 * s, true, vh, vl);
                qb[qt][s] = term == 0 ? vh : vl;
            }
            up[qt] = ub + (uint64_t)tq * (uint32_t)ucols + (ent & 63) * g;
        }

    };
    auto compute = [&](QPass& Pq) {
        auto& qb = Pq.qb;
        auto& has = Pq.has;
        auto& up = Pq.up;
        if constexpr (RC >= 16) {
            // one candidate (TPC row tiles) at a time; lane holds 4 rows per tile of its column
            for (int j = 0; j < g; ++j) {
                const int lim = lim_rows - j * RC;  // rows of candidate j that exist
                if (lim <= 0) break;
                f32x4 acc[TPC][kScoreNQT];
#pragma unroll
                for (int rt = 0; rt < TPC; ++rt)
#pragma unroll
                    for (int qt = 0; qt < kScoreNQT; ++qt) acc[rt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int rt = 0; rt < TPC; ++rt) {
                    const int r = (j * TPC + rt) * 16 + (lane & 15);
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
#pragma unroll
                for (int qt = 0; qt < kScoreNQT; ++qt) {
                    if constexpr (TA == 2) {  // add the low query term of the same head
#pragma unroll
                        for (int rt = 0; rt < TPC; ++rt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[rt][qt][i] += shfl_xor(acc[rt][qt][i], G);
                    }
                    const bool tail = lim < RC;  // the tail block of the sequence: rows past its end drop out
                    auto zf = [&](int x) {
                        const int rt = x >> 2, i = x & 3;
                        const float zz = acc[rt][qt][i] * scale;
                        return (tail && rt * 16 + 4 * lg + i >= lim) ? -INFINITY : zz;
                    };
                    float l2 = block_score2f<SK, TPC * 4, 3>(zf, true);
                    l2 = sum_adjacent(l2, G);  // heads are adjacent columns
                    if (has[qt] && writer_col) up[qt][j] = l2 * kLn2;
                }
            }
        } else {
            // all rows of P (g * RC <= 64: at most 4 row tiles); candidate of row r is r / RC
            constexpr int CPL = RC < 4 ? 4 / RC : 1;  // candidates per lane and row tile
            constexpr int RPL = 4 / CPL;               // rows per candidate held by one lane
            const int nrt = nrows_pad / 16;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if (rt >= nrt) break;
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
                        z[i] = v * scale;
                    }
                    if (lim_rows < nrows_pad) {  // padding rows, or a tail node with missing children
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (rt * 16 + 4 * lg + i >= lim_rows) z[i] = -INFINITY;
                    }
#pragma unroll
                    for (int k = 0; k < CPL; ++k) {
                        const int rfirst = rt * 16 + 4 * lg + k * RPL;  // first row of this candidate part
                        const bool exists = rfirst < lim_rows;
                        float l2 = block_score2<SK, RPL, RC == 8 ? 1 : 0>(z + k * RPL, exists);
                        l2 = sum_adjacent(l2, G);
                        const int j = rfirst / RC;  // candidate (child of P)
                        const bool owner = RC == 8 ? (lg & 1) == 0 : true;
                        if (has[qt] && owner && head == 0 && term == 0 && exists) up[qt][j] = l2 * kLn2;
                    }
                }
            }
        }
    };
    QPass A, B;
    const int stride = WAVES * kScoreNQT;
    int tp = wave * kScoreNQT;

    // Stage P's grandchildren rows (bf16 hi plane, and a lo plane for fp32 rows).
    const TS* rb = reinterpret_cast<const TS*>(a.rows) + (int64_t)b * a.rows_b_stride + (int64_t)h * a.rows_h_stride +
                   row0 * a.row_stride;
    for (int i = threadIdx.x; i < nrows_pad * (D / 8); i += 64 * WAVES) {
        const int r = i / (D / 8), c8 = i % (D / 8);
        const bool ok = r < lim_rows;
        bf16x8 vh, vl;
        Src<TS>::load(rb + (ok ? r : 0) * a.row_stride + 8 * c8, ok, vh, vl);
        *reinterpret_cast<bf16x8*>(s_rows + r * LDW + 8 * c8) = vh;
        if constexpr (TB == 2) *reinterpret_cast<bf16x8*>(s_rows + (nrows_pad + r) * LDW + 8 * c8) = vl;
    }
    // the chunk's entries (<= qc) next to the rows
    for (int i = threadIdx.x; i < e1 - e0; i += 64 * WAVES) s_ent[i] = a.entries[e0 + i];
    __syncthreads();

    if (tp < ntiles) {
        load_pass(tp, A);
        while (true) {
            if (tp + stride < ntiles) load_pass(tp + stride, B);
            compute(A);
            tp += stride;
            if (tp >= ntiles) break;
            if (tp + stride < ntiles) load_pass(tp + stride, A);
            compute(B);
            tp += stride;
            if (tp >= ntiles) break;
        }
    }
}

// Upper levels with g * g <= 16 grandchildren per node (one MFMA row tile):
// one wave per chunk of kRegChunk entries, no LDS and no workgroup barrier.
// The wave loads P's rows (fp32 summaries, as two bf16 terms) straight into
// its A operand registers; RC = g rows per candidate.
template <int D, typename T, int RC, int SK>
__global__ __launch_bounds__(64 * kRegWaves) void score_reg_kernel(ScoreArgs a)
{
    constexpr int TA = Src<T>::TERMS;
    constexpr int KS = D / 32;
    constexpr int CPL = RC < 4 ? 4 / RC : 1;  // candidates per lane
    constexpr int RPL = 4 / CPL;               // rows per candidate held by one lane
    const int64_t total = a.chunk_off[a.n_clusters];
    const int64_t nblk = (total + kRegWaves - 1) / kRegWaves;
    if ((int64_t)blockIdx.x >= nblk) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lg = lane >> 4;
    const int64_t lblk = a.xcd ? xcd_chunk(blockIdx.x, nblk) : (int64_t)blockIdx.x;
    const int64_t chunk = lblk * kRegWaves + wave;
    if (chunk >= total) return;  // the whole wave leaves; no barrier follows
    const int64_t cl = a.chunk_cl[chunk];
    const int e0 = a.offsets[cl] + (int)(chunk - a.chunk_off[cl]) * a.qc;
    const int e1 = min(a.offsets[cl + 1], e0 + a.qc);
    const int64_t P = cl % a.M_bins;
    const int64_t bh = (cl / a.M_bins) % a.BH;
    const int h = (int)(bh % a.H);
    const int b = (int)(bh / a.H);
    const int G = a.G, GT = a.G * TA, QT = 16 / GT;
    const int g = a.g;
    const int nrows = g * RC;  // <= 16
    const int64_t row0 = P * (int64_t)nrows;
    const int64_t rem = a.rows_limit - row0;
    const int lim_rows = rem < nrows ? (int)rem : nrows;

    // A operand: row (lane & 15) of P's rows, k-chunk 8 * lg + 32 * s
    bf16x8 ah[KS], al[KS];
    {
        const int r = lane & 15;
        const bool ok = r < lim_rows;
        const float* rp = reinterpret_cast<const float*>(a.rows) + (int64_t)b * a.rows_b_stride +
                          (int64_t)h * a.rows_h_stride + (row0 + (ok ? r : 0)) * a.row_stride + 8 * lg;
#pragma unroll
        for (int s = 0; s < KS; ++s) Src<float>::load(rp + 32 * s, ok, ah[s], al[s]);
    }

    const float scale = kLog2e * rsqrtf((float)D);
    const int col = lane & 15;
    const int qi = col / GT, term = (col % GT) / G, head = col % G;
    const int ucols = a.K_top * g;
    const int ntiles = (e1 - e0 + QT - 1) / QT;
    const T* Qb = reinterpret_cast<const T*>(a.Q) + (int64_t)b * a.N * a.H_q * D + (h * G + head) * D + 8 * lg;
    const uint32_t qrow = (uint32_t)(a.H_q * D);
    float* ub = a.u + bh * a.N * ucols;
    // the chunk's entries (<= 64), one per lane, fetched once; passes take theirs by shuffle
    const int ent_lane = a.entries[e0 + (lane < e1 - e0 ? lane : e1 - e0 - 1)];

    struct QPass {
        bf16x8 qb[kScoreNQT][KS];
        bool has[kScoreNQT];
        float* up[kScoreNQT];
    };
    auto load_pass = [&](int tp, QPass& Pq) {
        auto& qb = Pq.qb;
        auto& has = Pq.has;
        auto& up = Pq.up;
#pragma unroll
        for (int qt = 0; qt < kScoreNQT; ++qt) {
            const int e = e0 + (tp + qt) * QT + qi;
            has[qt] = e < e1;
            const int ent = shfl(ent_lane, has[qt] ? e - e0 : e1 - 1 - e0);
            const uint32_t tq = (uint32_t)ent >> 6;
            const T* qp = Qb + (uint64_t)tq * qrow;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 vh, vl;
                Src<T>::load(qp + 32 * s, true, vh, vl);
                qb[qt][s] = term == 0 ? vh : vl;
            }
            up[qt] = ub + (uint64_t)tq * (uint32_t)ucols + (ent & 63) * g;
        }
    };
    auto compute = [&](QPass& Pq) {
        auto& qb = Pq.qb;
        auto& has = Pq.has;
        auto& up = Pq.up;
        f32x4 acc[kScoreNQT];
#pragma unroll
        for (int qt = 0; qt < kScoreNQT; ++qt) acc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int qt = 0; qt < kScoreNQT; ++qt) {
                acc[qt] = mfma(ah[s], qb[qt][s], acc[qt]);
                acc[qt] = mfma(al[s], qb[qt][s], acc[qt]);
            }
#pragma unroll
        for (int qt = 0; qt < kScoreNQT; ++qt) {
            float z[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = acc[qt][i];
                if constexpr (TA == 2) v += shfl_xor(v, G);
                z[i] = v * scale;
            }
            if (lim_rows < 16) {  // padding rows, or a tail node with missing children
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * lg + i >= lim_rows) z[i] = -INFINITY;
            }
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int rfirst = 4 * lg + k * RPL;
                const bool exists = rfirst < lim_rows;
                float l2 = block_score2<SK, RPL, 0>(z + k * RPL, exists);
                l2 = sum_adjacent(l2, G);
                if (has[qt] && head == 0 && term == 0 && exists) up[qt][rfirst / RC] = l2 * kLn2;
            }
        }
    };
    // passes of kScoreNQT tiles, each loaded one pass ahead of its use
    QPass A, B;
    int tp = 0;
    load_pass(tp, A);
    while (true) {
        if (tp + kScoreNQT < ntiles) load_pass(tp + kScoreNQT, B);
        compute(A);
        tp += kScoreNQT;
        if (tp >= ntiles) break;
        if (tp + kScoreNQT < ntiles) load_pass(tp + kScoreNQT, A);
        compute(B);
        tp += kScoreNQT;
        if (tp >= ntiles) break;
    }
}

// Dense scoring of one upper level (g = GB in {2, 4}). Workgroup = 4 waves x
// up to 4 column tiles of (query, head) columns = QW consecutive queries of one
// (sequence, KV head). Rows (level l-1 summaries of the eligible level-(l+1)
// nodes) stream through LDS in batches of 4 row tiles as two bf16 terms; a row
// tile holds 16 / g^2 parents whose g children are the candidates. A per-query
// table maps each parent to its slot in the query's kept list (0xFF = not
// kept); only kept parents' candidates are written to u. With rows2_hl set, the
// workgroup then scores level l - 1 from the query tiles it already holds: the
// children of every eligible level-l node, written to u2 by node id (the kept
// level-l nodes are chosen after this kernel).
constexpr int kDenseBatch = 4;
constexpr int kDenseQW = 64;  // queries per workgroup (at most)

template <int D, typename T, int GB, int SK>
__global__ __launch_bounds__(256) void dense_kernel(DenseArgs a)
{
    constexpr int TA = Src<T>::TERMS;
    constexpr int KS = D / 32;
    constexpr int LDW = D + 8;
    constexpr int RP = GB * GB;  // rows per parent: 4 or 16
    constexpr int CPL = 4 / GB;  // candidates per lane: 2 (g = 2) or 1 (g = 4)
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    bf16* s_rows = reinterpret_cast<bf16*>(s_raw);  // [2][kDenseBatch * 16][LDW]
    uint8_t* s_slot = s_raw + 2 * kDenseBatch * 16 * LDW * 2;

    const int G = a.G, GT = G * TA, QT = 16 / GT;
    const int nct = GT < 4 ? GT : 4;  // column tiles per wave
    const int QW = 4 * nct * QT;
    const int K = a.K_top;
    const int64_t bh = blockIdx.y;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const int64_t t0 = (int64_t)blockIdx.x * QW;
    if (t0 >= a.N) return;
    const int64_t tl = (t0 + QW < a.N ? t0 + QW : a.N) - 1;
    const int64_t pm = a.causal ? tl >> a.par_span_log2 : a.M_par - 1;  // last eligible parent
    const int npar = (int)((pm < a.M_par - 1 ? pm : a.M_par - 1) + 1);  // eligible parents of the tile

    for (int k = threadIdx.x; k < QW * npar; k += 256) s_slot[k] = 0xFF;
    __syncthreads();
    for (int k = threadIdx.x; k < QW * K; k += 256) {
        const int q = k / K, sl = k % K;
        const int64_t t = t0 + q;
        if (t < a.N) {
            const int P = a.kept[(bh * a.N + t) * K + sl];
            if (P >= 0 && P < npar) s_slot[q * npar + P] = (uint8_t)sl;
        }
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lg = lane >> 4;
    const int col = lane & 15;
    const int qi = col / GT, term = (col % GT) / G, head = col % G;
    const float scale = kLog2e * rsqrtf((float)D);
    const int ucols = K * GB;

    bf16x8 qb[4][KS];
    int qloc[4];
    bool qok[4];
    const T* Qb = reinterpret_cast<const T*>(a.Q) + (int64_t)b * a.N * a.H_q * D + (h * G + head) * D + 8 * lg;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        qloc[ct] = (wave * nct + ct) * QT + qi;
        const int64_t t = t0 + qloc[ct];
        qok[ct] = ct < nct && t < a.N;
        const T* qp = Qb + (uint64_t)(qok[ct] ? t : t0) * (uint32_t)(a.H_q * D);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 vh, vl;
            Src<T>::load(qp + 32 * s, true, vh, vl);
            qb[ct][s] = term == 0 ? vh : vl;
        }
    }

    // one level: rows (level l-1 summaries of the np eligible parents, rows_limit of them exist)
    // stream through LDS; write(ct, P, j, score, exists) stores candidate j of parent P for the
    // queries of column tile ct
    auto pass = [&](const bf16* rh, int64_t rows_limit, int np, auto write) {
        const int nrows = np * RP;
        const int nrt = (nrows + 15) / 16;
        for (int kb = 0; kb < nrt; kb += kDenseBatch) {
            __syncthreads();  // the previous batch is consumed (first pass: the slot table is written)
            for (int i = threadIdx.x; i < kDenseBatch * 16 * (D / 8); i += 256) {
                const int r = i / (D / 8), c8 = i % (D / 8);
                const int64_t row = (int64_t)kb * 16 + r;
                const bool ok = row < nrows && row < rows_limit;
                // the row's two terms, split once per call (split_kernel)
                const bf16* hp = rh + (ok ? row : 0) * (2 * D) + 8 * c8;
                const bf16x8 vh = ok ? load8h(hp) : zero8h(), vl = ok ? load8h(hp + D) : zero8h();
                *reinterpret_cast<bf16x8*>(s_rows + r * LDW + 8 * c8) = vh;
                *reinterpret_cast<bf16x8*>(s_rows + (kDenseBatch * 16 + r) * LDW + 8 * c8) = vl;
            }
            __syncthreads();
            const int kend = kb + kDenseBatch < nrt ? kb + kDenseBatch : nrt;
            for (int k = kb; k < kend; ++k) {
                const int rl = (k - kb) * 16 + (lane & 15);
                bf16x8 ah[KS], al[KS];
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    ah[s] = *reinterpret_cast<const bf16x8*>(s_rows + rl * LDW + 32 * s + 8 * lg);
                    al[s] = *reinterpret_cast<const bf16x8*>(s_rows + (kDenseBatch * 16 + rl) * LDW + 32 * s + 8 * lg);
                }
                const int rfirst = k * 16 + 4 * lg;  // this lane's first row
                const int P = rfirst / RP;           // its parent (all four rows share it)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    if (ct >= nct) break;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        acc = mfma(ah[s], qb[ct][s], acc);
                        acc = mfma(al[s], qb[ct][s], acc);
                    }
                    float z[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = acc[i];
                        if constexpr (TA == 2) v += shfl_xor(v, G);
                        z[i] = (rfirst + i < nrows && rfirst + i < rows_limit) ? v * scale : -INFINITY;
                    }
#pragma unroll
                    for (int kk = 0; kk < CPL; ++kk) {
                        const int r0 = rfirst + kk * GB;  // first row of the candidate
                        const bool exists = r0 < nrows && r0 < rows_limit;
                        float l2 = block_score2<SK, GB, 0>(z + kk * GB, exists);
                        l2 = sum_adjacent(l2, G);
                        write(ct, P, (r0 % RP) / GB, l2 * kLn2, exists);  // candidate = child j of P
                    }
                }
            }
        }
    };
    // level l: candidates of the kept parents, by slot
    pass(reinterpret_cast<const bf16*>(a.rows_hl) + (int64_t)b * a.rows_hl_b_stride + (int64_t)h * a.rows_hl_h_stride,
         a.rows_limit, npar,
         [&](int ct, int P, int j, float v, bool exists) {
             const int slot = P < npar ? s_slot[qloc[ct] * npar + P] : 0xFF;
             if (qok[ct] && head == 0 && term == 0 && exists && slot != 0xFF)
                 a.u[(bh * a.N + t0 + qloc[ct]) * ucols + slot * GB + j] = v;
         });
    if (a.rows2_hl) {
        // level l - 1 in the same pass: the children of every eligible level-l node, by node id
        const int64_t pm2 = a.causal ? tl >> a.par2_span_log2 : a.M_par2 - 1;
        const int npar2 = (int)((pm2 < a.M_par2 - 1 ? pm2 : a.M_par2 - 1) + 1);
        pass(reinterpret_cast<const bf16*>(a.rows2_hl) + (int64_t)b * a.rows2_hl_b_stride +
                 (int64_t)h * a.rows2_hl_h_stride,
             a.rows2_limit, npar2,
             [&](int ct, int P, int j, float v, bool exists) {
                 if (qok[ct] && head == 0 && term == 0 && exists)
                     a.u2[(bh * a.N + t0 + qloc[ct]) * a.u2_cols + P * GB + j] = v;
             });
    }
}

// LDS layout shared by both kernels: [NB][kSubRows][D] bf16 ring, then
// kLeafQC entries, then kLeafQC x 4 scores.
struct StreamLds {
    bf16* q;
    int* ent;
    float* u;
};
template <int D, int NB>
__device__ __forceinline__ StreamLds stream_lds(unsigned char* raw)
{
    StreamLds L;
    L.q = reinterpret_cast<bf16*>(raw);
    L.ent = reinterpret_cast<int*>(raw + (size_t)NB * kSubRows * D * 2);
    L.u = reinterpret_cast<float*>(L.ent + kLeafQC);
    return L;
}

// Scores gathered in LDS, written after the chunk: u[.][t][slot * g + c] for
// the ncand candidates that exist.
__device__ __forceinline__ void stream_write_scores(const StreamLds& L, float* ub, int n, int ucols, int g,
                                                    int ncand)
{
    for (int el = threadIdx.x; el < n; el += 256) {
        const int ent = L.ent[el];
        float* up = ub + (uint64_t)((uint32_t)ent >> 6) * (uint32_t)ucols + (ent & 63) * g;
        if (g == 4 && ncand == 4) *reinterpret_cast<f32x4*>(up) = *reinterpret_cast<const f32x4*>(L.u + el * 4);
        else
            for (int q = 0; q < ncand; ++q) up[q] = L.u[el * 4 + q];
    }
}

// Leaf level, bf16 keys, g in {2, 4}: a workgroup scores a chunk of up to
// kLeafQC entries of one cluster (window, sequence x KV head, level-2 node P)
// against P's g leaf candidates. The C keys of candidate j are held in the
// registers of the waves w with w % g == j (A operand, C / 16 row tiles);
// the queries stream through the LDS ring (B operand, 16 columns = 16 / G
// entries x G heads per tile). Per (query column, candidate) the C scores are
// reduced to log2-sum-exp in registers and across the 4 lane groups, the G
// heads summed with DPP, and the natural-log score kept in LDS.
template <int D, int C, int NB, int SK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NB >= 3 ? 3 : 4))) void leaf_kernel(ScoreArgs a)
{
    constexpr int KS = D / 32;
    constexpr int TPC = C / 16;
    constexpr int CH = D / 8;
    static_assert(16 % CH == 0, "a row tile spans whole swizzle periods");
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];

    const int64_t total = a.chunk_off[a.n_clusters];
    if ((int64_t)blockIdx.x >= total) return;
    const int64_t chunk = blockIdx.x;
    const int64_t cl = a.chunk_cl[chunk];
    const int e0 = a.offsets[cl] + (int)(chunk - a.chunk_off[cl]) * a.qc;
    const int e1 = min(a.offsets[cl + 1], e0 + a.qc);
    const int n = e1 - e0;
    const int64_t P = cl % a.M_bins;
    const int64_t bh = (cl / a.M_bins) % a.BH;
    const int h = (int)(bh % a.H);
    const int b = (int)(bh / a.H);
    const int lane = threadIdx.x & 63, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar branches below
    const int G = a.G, QT = 16 / G, SE = kSubRows / G;  // entries per tile / per sub-chunk
    const int glog = __builtin_ctz(G);                   // G is a power of two
    const int g = a.g;
    const int wpc = 4 / g;  // waves per candidate
    const int j = wave % g, part = wave / g;
    const int ucols = a.K_top * g;
    const StreamLds L = stream_lds<D, NB>(s_raw);

    const bf16* Qb = reinterpret_cast<const bf16*>(a.Q) + (int64_t)b * a.N * a.H_q * D + (int64_t)h * G * D;
    const uint32_t qrow = (uint32_t)(a.H_q * D);
    const int nsb = (n + SE - 1) / SE;  // sub-chunks
    StreamPrologue<D, NB> pr;
    const StreamLane sl = stream_lane<D>(wave, lane, glog);
    stream_prologue_load<D, NB>(pr, a.entries + e0, n, SE, sl, glog);
    stream_prologue_issue<D, NB>(pr, L.ent, Qb, qrow, sl, L.q, wave);

    // keys of candidate j (leaf P * g + j): rows (lane & 15) of each row tile, k-chunk 8 * lg + 32 * s
    const int64_t krow0 = (P * g + j) * (int64_t)C;
    const int64_t krem = a.rows_limit - krow0;
    const int lim = krem < C ? (int)krem : C;  // keys of the candidate that exist (<= 0: no candidate)
    bf16x8 A[TPC][KS];
    {
        const bf16* kb = reinterpret_cast<const bf16*>(a.rows) + (int64_t)b * a.rows_b_stride +
                         (int64_t)h * a.rows_h_stride;
#pragma unroll
        for (int rt = 0; rt < TPC; ++rt) {
            const int r = rt * 16 + (lane & 15);
            const bool ok = r < lim;
            const bf16* kp = kb + (ok ? krow0 + r : 0) * a.row_stride + 8 * lg;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 v = load8h(kp + 32 * s);
                A[rt][s] = ok ? v : zero8h();
            }
        }
    }

    const float scale = kLog2e * rsqrtf((float)D);
    const int col = lane & 15;
    const int qi = col / G, head = col % G;
    // column col of row tile tl is LDS row tl * 16 + col (entry tl * QT + qi, head `head`), so the
    // swizzled position of its k-chunk 4 * s + lg is fixed per lane: byte offsets hoisted here
    int boff[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) boff[s] = (col * D + 8 * ((4 * s + lg) ^ (col & (CH - 1)))) * 2;
    const int64_t nj = a.rows_limit - P * g * (int64_t)C;  // keys of P that exist
    const int ncand = (int)((nj + C - 1) / C < g ? (nj + C - 1) / C : g);

    for (int sb = 0; sb < nsb; ++sb) {
        const int base = sb * SE;
        const int nsub = min(SE, n - base);
        stream_wait<D, NB>(min(NB - 2, nsb - 1 - sb));
        lds_barrier();  // every wave's part has landed; the buffer of sub-chunk sb - 1 is free again
        if (sb + NB - 1 < nsb) {
            const int nb = sb + NB - 1;
            stream_fetch<D>(Qb, qrow, L.ent + nb * SE, min(SE, n - nb * SE), sl, glog, L.q + (nb % NB) * kSubRows * D,
                            wave);
        }
        if (lim > 0) {
            const unsigned char* cur = reinterpret_cast<const unsigned char*>(L.q + (sb % NB) * kSubRows * D);
            for (int tl = part; tl < kSubRows / 16 && tl * QT < nsub; tl += wpc) {
                const int el = tl * QT + qi;  // entry of this lane's column within the sub-chunk
                const unsigned char* tb = cur + tl * (16 * D * 2);
                bf16x8 B[KS];
#pragma unroll
                for (int s = 0; s < KS; ++s) B[s] = *reinterpret_cast<const bf16x8*>(tb + boff[s]);
                f32x4 acc[TPC];
#pragma unroll
                for (int rt = 0; rt < TPC; ++rt) {
                    acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s) acc[rt] = mfma(A[rt][s], B[s], acc[rt]);
                }
                float l2;
                if (lim == C) {
                    l2 = block_score2f<SK, TPC * 4, 3>([&](int x) { return acc[x >> 2][x & 3] * scale; }, true);
                } else {  // the tail block of the sequence: rows past its end drop out
                    l2 = block_score2f<SK, TPC * 4, 3>(
                        [&](int x) {
                            const int rt = x >> 2, i = x & 3;
                            return rt * 16 + 4 * lg + i < lim ? acc[rt][i] * scale : -INFINITY;
                        },
                        true);
                }
                l2 = sum_adjacent(l2, G);
                if (lg == 0 && head == 0 && el < nsub) L.u[(base + el) * 4 + j] = l2 * kLn2;
            }
        }
    }
    lds_barrier();
    stream_write_scores(L, a.u + bh * a.N * ucols, n, ucols, g, ncand);
}

// Upper levels with g in {2, 4} (g * g <= 16 grandchildren per node), bf16
// queries. A workgroup scores a chunk of up to kLeafQC entries of one cluster
// (window, sequence x KV head, node P). P's g * g grandchild summaries (fp32,
// split into two bf16 terms) form one 16-row A tile that every wave keeps in
// registers; the chunk's query rows stream through the LDS ring, each wave
// taking one 16-column tile per sub-chunk. Tile rows 4 * lg .. 4 * lg + 3 hold
// 4 / RC whole candidates, so a lane reduces its candidates without crossing
// lanes; the G heads of a query sit in adjacent lanes and are summed with DPP.
// RC = g rows per candidate.
template <int D, int RC, int NB, int SK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void upper_kernel(ScoreArgs a)
{
    static_assert(RC == 2 || RC == 4, "g in {2, 4}");
    constexpr int KS = D / 32;
    constexpr int CH = D / 8;
    constexpr int CPL = 4 / RC;  // candidates per lane
    static_assert(16 % CH == 0, "a row tile spans whole swizzle periods");
    static_assert(kSubRows == 64, "one tile per wave and sub-chunk");
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];

    const int64_t total = a.chunk_off[a.n_clusters];
    if ((int64_t)blockIdx.x >= total) return;
    const int64_t chunk = a.xcd ? xcd_chunk(blockIdx.x, total) : (int64_t)blockIdx.x;
    const int64_t cl = a.chunk_cl[chunk];
    const int e0 = a.offsets[cl] + (int)(chunk - a.chunk_off[cl]) * a.qc;
    const int e1 = min(a.offsets[cl + 1], e0 + a.qc);
    const int n = e1 - e0;
    const int64_t P = cl % a.M_bins;
    const int64_t bh = (cl / a.M_bins) % a.BH;
    const int h = (int)(bh % a.H);
    const int b = (int)(bh / a.H);
    const int lane = threadIdx.x & 63, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = a.G, QT = 16 / G, SE = kSubRows / G;
    const int glog = __builtin_ctz(G);  // G is a power of two
    const int ucols = a.K_top * RC;
    const StreamLds L = stream_lds<D, NB>(s_raw);

    const bf16* Qb = reinterpret_cast<const bf16*>(a.Q) + (int64_t)b * a.N * a.H_q * D + (int64_t)h * G * D;
    const uint32_t qrow = (uint32_t)(a.H_q * D);
    const int nsb = (n + SE - 1) / SE;
    StreamPrologue<D, NB> pr;
    const StreamLane sl = stream_lane<D>(wave, lane, glog);
    stream_prologue_load<D, NB>(pr, a.entries + e0, n, SE, sl, glog);
    stream_prologue_issue<D, NB>(pr, L.ent, Qb, qrow, sl, L.q, wave);

    // A operand: row (lane & 15) of P's grandchildren, k-chunk 8 * lg + 32 * s, as hi / lo bf16 terms
    constexpr int nrows = RC * RC;
    const int64_t row0 = P * nrows;
    const int64_t rem = a.rows_limit - row0;
    const int lim_rows = rem < nrows ? (int)rem : nrows;  // >= 1: P's first grandchild exists
    bf16x8 ah[KS], al[KS];
    {
        const int r = lane & 15;
        const bool ok = r < lim_rows;
        const float* rp = reinterpret_cast<const float*>(a.rows) + (int64_t)b * a.rows_b_stride +
                          (int64_t)h * a.rows_h_stride + (row0 + (ok ? r : 0)) * a.row_stride + 8 * lg;
#pragma unroll
        for (int s = 0; s < KS; ++s) Src<float>::load(rp + 32 * s, ok, ah[s], al[s]);
    }

    const float scale = kLog2e * rsqrtf((float)D);
    const int col = lane & 15;
    const int qi = col / G, head = col % G;
    int boff[KS];  // byte offset of this lane's B piece within a row tile (as in leaf_kernel)
#pragma unroll
    for (int s = 0; s < KS; ++s) boff[s] = (col * D + 8 * ((4 * s + lg) ^ (col & (CH - 1)))) * 2;
    const int ncand = (lim_rows + RC - 1) / RC;  // children of P that exist

    for (int sb = 0; sb < nsb; ++sb) {
        const int base = sb * SE;
        const int nsub = min(SE, n - base);
        stream_wait<D, NB>(min(NB - 2, nsb - 1 - sb));
        lds_barrier();
        if (sb + NB - 1 < nsb) {
            const int nb = sb + NB - 1;
            stream_fetch<D>(Qb, qrow, L.ent + nb * SE, min(SE, n - nb * SE), sl, glog, L.q + (nb % NB) * kSubRows * D,
                            wave);
        }
        const int el = wave * QT + qi;  // this wave's tile is row tile `wave` of the sub-chunk
        const unsigned char* tb =
            reinterpret_cast<const unsigned char*>(L.q + (sb % NB) * kSubRows * D) + wave * (16 * D * 2);
        bf16x8 B[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) B[s] = *reinterpret_cast<const bf16x8*>(tb + boff[s]);
        f32x4 acc_h = f32x4{0.f, 0.f, 0.f, 0.f}, acc_l = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            acc_h = mfma(ah[s], B[s], acc_h);
            acc_l = mfma(al[s], B[s], acc_l);
        }
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = (acc_h[i] + acc_l[i]) * scale;
        if (lim_rows < 16) {  // padding rows (g = 2), or a tail node with missing grandchildren
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * lg + i >= lim_rows) z[i] = -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int rfirst = 4 * lg + k * RC;
            const bool exists = rfirst < lim_rows;
            float l2 = block_score2<SK, RC, 0>(z + k * RC, exists);
            l2 = sum_adjacent(l2, G);
            if (head == 0 && exists && el < nsub) L.u[(base + el) * 4 + rfirst / RC] = l2 * kLn2;
        }
    }
    lds_barrier();
    stream_write_scores(L, a.u + bh * a.N * ucols, n, ucols, RC, ncand);
}

// Upper levels with g in {2, 4}, bf16 queries: one wave per chunk of at most kWaveQC
// entries, so a small cluster costs one wave's start-up, which the other waves of the CU
// overlap (clusters are small when the windows are L2-sized: a window's query rows then
// stay in the XCD's L2 across the clusters that re-read them). The per-tile arithmetic is
// upper_kernel's: P's g * g grandchild summaries as one 16-row A tile of two bf16 terms in
// registers; a tile of 16 query columns (16 / G entries x G heads) on the MFMA; each lane
// reduces whole candidates; heads summed with DPP. Query rows stream through a ring of NBW
// tiles in the wave's own LDS (global_load_lds, 16-byte pieces XOR-swizzled by row as in
// the shared ring), with exact vmcnt waits and no workgroup barrier. Lane j collects the
// scores of entry j with permutes and writes them after the chunk (no LDS beyond the ring, so
// five workgroups fit a CU).
template <int D>
struct WaveRing {
    static constexpr int CH = D / 8;       // 16-byte pieces per row
    static constexpr int RPI = 64 / CH;    // rows per fetch instruction
    static constexpr int NIT = 16 / RPI;   // fetch instructions per 16-row tile
};
template <int D, int NBW>
constexpr size_t wave_ring_bytes() { return (size_t)NBW * 16 * D * 2; }

template <int D, int NB, int K = NB - 2>
__device__ __forceinline__ void wave_ring_wait(int later)
{
    constexpr int NIT = WaveRing<D>::NIT;
    static_assert(NB >= 2 && (NB - 2) * NIT < 64, "ring depth within the vmcnt range");
    if constexpr (K <= 0) {
        wait_vm<0>();
    } else {
        if (later >= K) {
            wait_vm<K * NIT>();
            return;
        }
        wave_ring_wait<D, NB, K - 1>(later);
    }
}

template <int D, int RC, int NBW, int SK>
__global__ __launch_bounds__(256) void upper_ring_kernel(ScoreArgs a)
{
    static_assert(RC == 2 || RC == 4, "g in {2, 4}");
    static_assert(kWaveQC == 64, "one entry per lane");
    using W = WaveRing<D>;
    constexpr int KS = D / 32;
    constexpr int CPL = 4 / RC;  // candidates per lane
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];

    const int64_t total = a.chunk_off[a.n_clusters];
    const int64_t nblk = (total + 3) >> 2;
    if ((int64_t)blockIdx.x >= nblk) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t chunk = (a.xcd ? xcd_chunk(blockIdx.x, nblk) : (int64_t)blockIdx.x) * 4 + wave;
    if (chunk >= total) return;  // whole wave; nothing below synchronises across waves
    bf16* ring = reinterpret_cast<bf16*>(s_raw + (size_t)wave * wave_ring_bytes<D, NBW>());
    const int64_t cl = a.chunk_cl[chunk];
    const int e0 = a.offsets[cl] + (int)(chunk - a.chunk_off[cl]) * a.qc;
    const int n = min(a.offsets[cl + 1], e0 + a.qc) - e0;  // 1 <= n <= kWaveQC
    const int64_t P = cl % a.M_bins;
    const int64_t bh = (cl / a.M_bins) % a.BH;
    const int h = (int)(bh % a.H);
    const int b = (int)(bh / a.H);
    const int lane = threadIdx.x & 63, lg = lane >> 4;
    const int G = a.G, QT = 16 / G;
    const int glog = __builtin_ctz(G);  // G is a power of two
    const int ucols = a.K_top * RC;
    const int ent = a.entries[e0 + min(lane, n - 1)];  // lane j: entry j (the last one past n)

    // A operand: row (lane & 15) of P's grandchildren, k-chunk 8 * lg + 32 * s, as hi / lo bf16 terms
    constexpr int nrows = RC * RC;
    const int64_t row0 = P * nrows;
    const int64_t rem = a.rows_limit - row0;
    const int lim_rows = rem < nrows ? (int)rem : nrows;  // >= 1: P's first grandchild exists
    bf16x8 ah[KS], al[KS];
    {
        const int r = lane & 15;
        const bool ok = r < lim_rows;
        // P's grandchildren as two bf16 terms, split once per call (split_kernel)
        const bf16* rp = reinterpret_cast<const bf16*>(a.rows_hl) + (int64_t)b * a.rows_hl_b_stride +
                         (int64_t)h * a.rows_hl_h_stride + (row0 + (ok ? r : 0)) * (2 * D) + 8 * lg;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            ah[s] = ok ? load8h(rp + 32 * s) : zero8h();
            al[s] = ok ? load8h(rp + D + 32 * s) : zero8h();
        }
    }
    // the A rows are in flight ahead of the ring's first fetches: a wait for a tile (exact count
    // of the fetches issued after it) also covers every older load

    const bf16* Qb = reinterpret_cast<const bf16*>(a.Q) + (int64_t)b * a.N * a.H_q * D + (int64_t)h * G * D;
    // element offset of this lane's entry's query row (below 2^31: N * H_q * D < 2^31 on this path)
    const uint32_t qoff = ((uint32_t)ent >> 6) * (uint32_t)(a.H_q * D);
    // this lane's part of fetch instruction i of a tile: tile row r = i * RPI + lane / CH holds
    // entry r / G, head r % G; the lane stores piece (lane % CH) of that row's LDS copy, which
    // holds piece (lane % CH) ^ (r % CH) of the global row. Per lane and instruction, the entry's
    // place in the tile and the offset within its G rows are fixed: only the tile changes.
    int rel[W::NIT], within[W::NIT];
#pragma unroll
    for (int i = 0; i < W::NIT; ++i) {
        const int r = i * W::RPI + lane / W::CH;
        rel[i] = r >> glog;
        within[i] = (r & (G - 1)) * D + 8 * ((lane % W::CH) ^ (r & (W::CH - 1)));
    }
    auto fetch = [&](int t, int slot) {
#pragma unroll
        for (int i = 0; i < W::NIT; ++i) {
            const int idx = min(t * QT + rel[i], n - 1);
            const uint32_t off = (uint32_t)shfl((int)qoff, idx) + (uint32_t)within[i];
            __builtin_amdgcn_global_load_lds(
                Qb + off, (__attribute__((address_space(3))) void*)(ring + (slot * 16 + i * W::RPI) * D), 16, 0, 0);
        }
    };
    const int ntiles = (n + QT - 1) / QT;
#pragma unroll
    for (int k = 0; k < NBW - 1; ++k)
        if (k < ntiles) fetch(k, k);

    const float scale = kLog2e * rsqrtf((float)D);
    const int col = lane & 15;
    const int qi = col / G, head = col % G;
    int boff[KS];  // byte offset of this lane's B piece within a tile (swizzled as fetched)
#pragma unroll
    for (int s = 0; s < KS; ++s) boff[s] = (col * D + 8 * ((4 * s + lg) ^ (col & (W::CH - 1)))) * 2;
    const int ncand = (lim_rows + RC - 1) / RC;  // children of P that exist
    float us[4] = {0.f, 0.f, 0.f, 0.f};          // scores of this lane's entry (lane j: entry j)

    for (int t = 0; t < ntiles; ++t) {
        wave_ring_wait<D, NBW>(min(NBW - 2, ntiles - 1 - t));
        if (t + NBW - 1 < ntiles) {
            // the slot of tile t - 1, whose reads have completed (their values fed its products)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            fetch(t + NBW - 1, (t + NBW - 1) % NBW);
        }
        const unsigned char* tb = reinterpret_cast<const unsigned char*>(ring + (t % NBW) * 16 * D);
        bf16x8 B[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) B[s] = *reinterpret_cast<const bf16x8*>(tb + boff[s]);
        f32x4 acc_h = f32x4{0.f, 0.f, 0.f, 0.f}, acc_l = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            acc_h = mfma(ah[s], B[s], acc_h);
            acc_l = mfma(al[s], B[s], acc_l);
        }
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = (acc_h[r] + acc_l[r]) * scale;
        if (lim_rows < 16) {  // padding rows (g = 2), or a tail node with missing grandchildren
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * lg + r >= lim_rows) z[r] = -INFINITY;
        }
        float l2c[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int rfirst = 4 * lg + c * RC;
            float l2 = block_score2<SK, RC, 0>(z + c * RC, rfirst < lim_rows);
            l2c[c] = sum_adjacent(l2, G) * kLn2;
        }
        // candidate q of entry j = t * QT + i sits in lane (i * G, lane group 4 q / RC), slot q % CPL
        const int i = lane - t * QT;  // this lane's entry within the tile, when 0 <= i < QT
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float v = shfl(l2c[q % CPL], (i & (QT - 1)) * G + 16 * ((q * RC) >> 2));
            if (i >= 0 && i < QT) us[q] = v;
        }
    }
    if (lane < n) {
        float* up = a.u + bh * a.N * ucols + (uint64_t)((uint32_t)ent >> 6) * (uint32_t)ucols + (ent & 63) * RC;
        if (RC == 4 && ncand == 4) *reinterpret_cast<f32x4*>(up) = f32x4{us[0], us[1], us[2], us[3]};
        else
            for (int q = 0; q < ncand; ++q) up[q] = us[q];
    }
}

}  // namespace pisa
