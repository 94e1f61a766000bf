// route_impl.hpp -- PISA routing kernels ("Block Sparse Attention with
// Log-Linear Complexity", section 3.2 eq 16-22, section 3.3, appendix B).
//
// route_query_kernel: one (query position, KV head) per workgroup. The
//   candidate list lives in the lanes of each wave (one candidate per lane,
//   at most g * K_top <= 64), scores in LDS; no query-key score matrix is
//   stored. Levels run from the top down to `stop` (1 for the fused router
//   and the decode router, 2 for stage 1 of the two-stage router).
//   Scoring a level: the non-forced candidates are listed in rank order and
//   cut into groups of 64 (candidate, child) columns; each group is a
//   [16 x d] x [d x 64] bf16 MFMA product (rows = the G_Q query heads, and for
//   fp32 queries their low halves; columns = child summaries or raw keys,
//   fp32 sources split into two bf16 terms), then a per-head log-sum-exp over
//   each candidate's children and a sum over heads.
//   Selection: every candidate's rank on (score desc, id asc), forced
//   nodes keyed +inf, then one ds_permute; expansion and compaction with
//   ballot / ds_permute.
//
// stage2_kernel: leaf scoring of stage-1 survivors, clustered by retained
//   level-2 node p. A workgroup stages p's g leaf blocks (g * C keys) in LDS
//   once and scores them for every query of its chunk: rows = (query, head)
//   pairs, 16 per MFMA tile, so a key block is reused across queries and
//   across the heads of the group (section 3.3, Stage 2, eq 23-24).
#pragma once

#include "pisa_device.hpp"
#include "pisa_internal.hpp"

namespace pisa {

constexpr int kChunkQ = 128;  // queries per stage-2 workgroup

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Grid index -> logical item so that each XCD (blocks are dealt round-robin
// over 8 XCDs) receives one contiguous range of items.
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t total)
{
    const int64_t per = total >> 3;
    if (i < (per << 3)) return (i & 7) * per + (i >> 3);
    return i;
}

// Block score (base 2; the callers scale by ln 2) of one candidate and query head from the
// values its group of `width` adjacent lanes hold, n per lane with validity flags: SK 1 is
// the mean of the valid values (PISA-1, section 4.4 eq 33), SK 2 the mean plus half their
// population variance, the variance taken about the mean in a second pass and scaled by ln 2
// to natural units (PISA-2, eq 34). No valid value: -inf.
template <int SK, int N>
__device__ __forceinline__ float group_moment_score(const float* y, const bool* ok, int width)
{
    float s = 0.f, c = 0.f;
#pragma unroll
    for (int t = 0; t < N; ++t) {
        s += ok[t] ? y[t] : 0.f;
        c += ok[t] ? 1.f : 0.f;
    }
    s = group_sum(s, width);
    c = group_sum(c, width);
    const float mu = c > 0.f ? s / c : 0.f;
    if constexpr (SK == 1) {
        return c > 0.f ? mu : -INFINITY;
    } else {
        float q = 0.f;
#pragma unroll
        for (int t = 0; t < N; ++t) {
            const float dy = y[t] - mu;
            q += ok[t] ? dy * dy : 0.f;
        }
        q = group_sum(q, width);
        return c > 0.f ? mu + (0.5f * kLn2) * (q / c) : -INFINITY;
    }
}

template <int D, typename T, int G, int WAVES, int SK = 0>
struct RouteQuery {
    static constexpr int TA = Src<T>::TERMS;  // query terms per head
    static constexpr int R = G * TA;          // MFMA rows in use
    static constexpr int KS = D / 32;
    static_assert(R <= 16, "rows");

    // Grouped LSE scores (natural log) of the ns scored candidates of level l
    // whose ids are s_sid[0..ns); results to s_u[0..ns).
    template <typename TS>
    __device__ __forceinline__ static void score_level(const TS* base, int64_t row_stride, int64_t limit,
                                                       int nch_log2, int ns, const bf16x8* qa, float* s_z,
                                                       const int* s_sid, float* s_u)
    {
        constexpr int TB = Src<TS>::TERMS;
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int nch = 1 << nch_log2;
        const int cpg_log2 = 6 - nch_log2;
        const int ngroups = (ns + (1 << cpg_log2) - 1) >> cpg_log2;
        const float scale = kLog2e * rsqrtf((float)D);
        for (int grp = wave; grp < ngroups; grp += WAVES) {
            f32x4 acc[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int col = 16 * tt + (lane & 15);
                const int j = (grp << cpg_log2) + (col >> nch_log2);
                const int cand = j < ns ? s_sid[j] : -1;
                const int64_t row = (int64_t)cand * nch + (col & (nch - 1));
                const bool ok = cand >= 0 && row < limit;
                const TS* ptr = base + (ok ? row : 0) * row_stride + 8 * (lane >> 4);
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    bf16x8 hi, lo;
                    Src<TS>::load(ptr + 32 * s, ok, hi, lo);
                    c = mfma(qa[s], hi, c);
                    if constexpr (TB == 2) c = mfma(qa[s], lo, c);
                }
                acc[tt] = c;
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * (lane >> 4) + i;
                    if (r < R) s_z[r * 65 + 16 * tt + (lane & 15)] = acc[tt][i];
                }
            wave_lds_sync();
            const int j = (grp << cpg_log2) + (lane >> nch_log2);
            const int cand = j < ns ? s_sid[j] : -1;
            const bool ok = cand >= 0 && (int64_t)cand * nch + (lane & (nch - 1)) < limit;
            float u = 0.f;
#pragma unroll
            for (int hd = 0; hd < G; ++hd) {
                float y = s_z[hd * 65 + lane];
                if constexpr (TA == 2) y += s_z[(G + hd) * 65 + lane];
                y = ok ? y * scale : -INFINITY;
                if constexpr (SK != 0) {
                    u += group_moment_score<SK, 1>(&y, &ok, nch);
                } else {
                    const float m = group_max(y, nch);
                    const float e = ok ? __builtin_amdgcn_exp2f(y - m) : 0.f;
                    const float ssum = group_sum(e, nch);
                    u += m + __builtin_amdgcn_logf(ssum);
                }
            }
            if ((lane & (nch - 1)) == 0 && j < ns) s_u[j] = u * kLn2;
            wave_lds_sync();
        }
    }

    // Decode, bf16 queries (one query row per head): the same scores as
    // score_level, with every load of a task issued before its products and
    // the reductions kept in registers. A task is one 16-column tile of
    // (candidate, child) columns when a candidate has nch <= 16 children, else
    // one candidate's nch / 16 tiles; the waves share the tasks.
    template <typename TS>
    __device__ __forceinline__ static void score_level_regs(const TS* base, int64_t row_stride, int64_t limit,
                                                            int nch_log2, int ns, const bf16x8* qa, const int* s_sid,
                                                            float* s_u)
    {
        static_assert(TA == 1, "one query row per head");
        constexpr int TB = Src<TS>::TERMS;
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int col = lane & 15, lg = lane >> 4;
        const int nch = 1 << nch_log2;
        const float scale = kLog2e * rsqrtf((float)D);
        if (nch <= 16) {
            const int ntasks = (ns * nch + 15) >> 4;
            for (int task = wave; task < ntasks; task += WAVES) {
                const int cc = task * 16 + col;  // (candidate, child) column
                const int j = cc >> nch_log2;
                const int cand = j < ns ? s_sid[j] : -1;
                const int64_t row = (int64_t)cand * nch + (cc & (nch - 1));
                const bool ok = cand >= 0 && row < limit;
                const TS* ptr = base + (ok ? row : 0) * row_stride + 8 * lg;
                bf16x8 hi[KS], lo[KS];
#pragma unroll
                for (int s = 0; s < KS; ++s) Src<TS>::load(ptr + 32 * s, ok, hi[s], lo[s]);
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    c = mfma(qa[s], hi[s], c);
                    if constexpr (TB == 2) c = mfma(qa[s], lo[s], c);
                }
                // rows 4 lg + i are heads; a candidate's children are nch adjacent lanes
                float u = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float y = ok ? c[i] * scale : -INFINITY;
                    float sc;
                    if constexpr (SK != 0) {
                        sc = group_moment_score<SK, 1>(&y, &ok, nch);
                    } else {
                        const float m = group_max(y, nch);
                        const float e = ok ? __builtin_amdgcn_exp2f(y - m) : 0.f;
                        const float sum = group_sum(e, nch);
                        sc = m + __builtin_amdgcn_logf(sum);
                    }
                    if (4 * lg + i < G) u += sc;
                }
                u += shfl_xor(u, 16);
                u += shfl_xor(u, 32);
                if (lg == 0 && (cc & (nch - 1)) == 0 && j < ns) s_u[j] = u * kLn2;
            }
        } else {
            const int nt = nch >> 4;  // 2 or 4 tiles per candidate
            for (int task = wave; task < ns; task += WAVES) {
                const int cand = s_sid[task];
                bf16x8 hi[4][KS], lo[4][KS];
                bool ok[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int64_t row = (int64_t)cand * nch + 16 * tt + col;
                    ok[tt] = tt < nt && row < limit;
                    const TS* ptr = base + (ok[tt] ? row : 0) * row_stride + 8 * lg;
#pragma unroll
                    for (int s = 0; s < KS; ++s) Src<TS>::load(ptr + 32 * s, ok[tt], hi[tt][s], lo[tt][s]);
                }
                f32x4 c[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    c[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        c[tt] = mfma(qa[s], hi[tt][s], c[tt]);
                        if constexpr (TB == 2) c[tt] = mfma(qa[s], lo[tt][s], c[tt]);
                    }
                }
                float u = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float sc;
                    if constexpr (SK != 0) {
                        float y[4];
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) y[tt] = c[tt][i] * scale;
                        sc = group_moment_score<SK, 4>(y, ok, 16);
                    } else {
                        float m = -INFINITY;
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) m = fmaxf(m, ok[tt] ? c[tt][i] * scale : -INFINITY);
                        m = group_max(m, 16);
                        float sum = 0.f;
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) sum += ok[tt] ? __builtin_amdgcn_exp2f(c[tt][i] * scale - m) : 0.f;
                        sum = group_sum(sum, 16);
                        sc = m + __builtin_amdgcn_logf(sum);
                    }
                    if (4 * lg + i < G) u += sc;
                }
                u += shfl_xor(u, 16);
                u += shfl_xor(u, 32);
                if (lane == 0) s_u[task] = u * kLn2;
            }
        }
    }

    template <int MODE>
    __device__ static void run(const RouteArgs& a)
    {
        __shared__ int s_sid[64];
        __shared__ float s_u[64];
        __shared__ float s_zall[WAVES][R * 65];  // the R MFMA rows in use
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        float* s_z = s_zall[wave];
        const PyrArgs& p = a.p;
        const Geo geo{p.c_log2, p.g_log2};

        int b, h;
        int64_t t, n;
        if constexpr (MODE == MODE_DECODE) {
            b = blockIdx.x / p.H;
            h = blockIdx.x % p.H;
            n = a.seqlen[b];
            if (n < 1 || n > p.N_cap) {  // lengths live on the device; refuse out-of-range ones
                if (threadIdx.x < a.K_top) {
                    a.idx[((int64_t)b * p.H + h) * a.K_top + threadIdx.x] = -1;
                    if (a.score) a.score[((int64_t)b * p.H + h) * a.K_top + threadIdx.x] = -INFINITY;
                }
                return;
            }
            t = n - 1;
        } else {
            const int64_t total = (int64_t)gridDim.x;
            const int64_t item = xcd_remap(blockIdx.x, total);
            t = item % a.N;
            const int64_t bh = item / a.N;
            h = (int)(bh % p.H);
            b = (int)(bh / p.H);
            n = a.N;
        }

        // A operand: row r = lane % 16 -> (term, head); k chunk = lane / 16.
        bf16x8 qa[KS];
        {
            const int r = lane & 15;
            const int term = r / G, head = r % G;
            const bool ok = r < R;
            const int64_t qrow = (MODE == MODE_DECODE) ? ((int64_t)b * a.H_q + (int64_t)h * G + head)
                                                       : (((int64_t)b * a.N + t) * a.H_q + (int64_t)h * G + head);
            const T* qp = (const T*)a.Q + qrow * D + 8 * (lane >> 4);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 hi, lo;
                Src<T>::load(qp + 32 * s, ok, hi, lo);
                qa[s] = (term == 0) ? hi : lo;
            }
        }

        const int64_t c = t >> p.c_log2;
        const int L = geo.top(n);
        constexpr int stop = (MODE == MODE_STAGE1) ? 2 : 1;
        int cid = lane == 0 ? 0 : -1;
        int nA = 1, nkept = 1;
        float key = lane == 0 ? INFINITY : -INFINITY;

        for (int l = L; l >= stop; --l) {
            const int sh = (l - 1) * p.g_log2;
            const bool forced = a.causal && cid >= 0 &&
                                (cid == 0 || cid == (int)(c >> sh) || (c >= 1 && cid == (int)((c - 1) >> sh)));
            if (nA <= a.K_top) {
                key = cid >= 0 ? INFINITY : -INFINITY;
                nkept = nA;
            } else {
                const bool scored = cid >= 0 && !forced;
                const uint64_t sm = ballot(scored);
                const int ns = __popcll(sm);
                const int rk = rank_below(sm);
                if (wave == 0 && scored) s_sid[rk] = cid;
                __syncthreads();
                constexpr bool regs = MODE == MODE_DECODE && TA == 1;
                if (l == 1) {
                    const T* kb = (const T*)a.K + ((int64_t)b * p.N_cap * p.H + h) * D;
                    if constexpr (regs)
                        score_level_regs<T>(kb, (int64_t)p.H * D, n, p.c_log2, ns, qa, s_sid, s_u);
                    else
                        score_level<T>(kb, (int64_t)p.H * D, n, p.c_log2, ns, qa, s_z, s_sid, s_u);
                } else {
                    const float* lb = p.buf + p.off[l - 1] + ((int64_t)b * p.H + h) * p.M_cap[l - 1] * D;
                    if constexpr (regs)
                        score_level_regs<float>(lb, D, geo.nodes(n, l - 1), p.g_log2, ns, qa, s_sid, s_u);
                    else
                        score_level<float>(lb, D, geo.nodes(n, l - 1), p.g_log2, ns, qa, s_z, s_sid, s_u);
                }
                __syncthreads();
                const float u = scored ? s_u[rk] : 0.f;
                // a NaN score (non-finite inputs) drops its candidate, as in the other selects
                const bool live = cid >= 0 && !(scored && !(u == u));
                key = forced ? INFINITY : (scored && live ? u : -INFINITY);
                int sid = live ? cid : (0x7fffffff - lane);
                const uint64_t lv = ballot(live);
                rank_sort(key, sid, lv);
                nkept = __popcll(lv) < a.K_top ? __popcll(lv) : a.K_top;
                cid = lane < nkept ? sid : -1;
                if (lane >= nkept) key = -INFINITY;
                __syncthreads();  // s_sid / s_u are rewritten at the next level
            }
            if (l > stop) {
                const int k = lane >> p.g_log2;
                const int parent = shfl(cid, k < 64 ? k : 0);
                const int64_t child = (int64_t)parent * p.g + (lane & (p.g - 1));
                const bool ok = k < nkept && parent >= 0 && child < geo.nodes(n, l - 1) &&
                                (!a.causal || (child << geo.span_log2(l - 1)) <= t);
                int nid = ok ? (int)child : -1;
                float dummy = 0.f;
                nA = compact(ok, nid, dummy);
                cid = lane < nA ? nid : -1;
            }
        }

        if constexpr (MODE == MODE_STAGE1) {
            // kept level-2 nodes (or the single node {0} when the pyramid has one level)
            const int64_t item = ((int64_t)b * p.H + h) * a.N + t;
            if (lane < a.K_top) a.kept2[item * a.K_top + lane] = lane < nkept ? cid : -1;
            const int64_t M1 = geo.nodes(n, 1);
            int nvalid = 0, nscored = 0;
            if (lane < nkept && cid >= 0) {
                for (int cc = 0; cc < p.g; ++cc) {
                    const int64_t leaf = (int64_t)cid * p.g + cc;
                    if (leaf >= M1) break;
                    if (a.causal && (leaf << p.c_log2) > t) break;
                    ++nvalid;
                    const bool f = a.causal && (leaf == 0 || leaf == c || leaf == c - 1);
                    if (!f) ++nscored;
                }
            }
            int tot = nvalid;
            for (int o = 1; o < 64; o <<= 1) tot += shfl_xor(tot, o);
            const bool leaf_scored = tot > a.K_top;
            // meta: bit 0 = the leaf level ranks candidates; bit 1 + k = kept slot k
            // has at least one leaf to score (it joins the cluster of its node).
            const uint64_t mask = ballot(leaf_scored && nscored > 0);
            if (lane == 0) a.meta[item] = (int64_t)((mask << 1) | (leaf_scored ? 1u : 0u));
            if (leaf_scored && nscored > 0) atomicAdd(&a.counts[((int64_t)b * p.H + h) * a.M2 + cid], 1);
        } else {
            int id = lane < nkept ? cid : (0x7fffffff - lane);
            float val = lane < nkept ? key : -INFINITY;
            rank_sort_ids(id, val, ballot(lane < nkept));
            const int64_t base = (MODE == MODE_DECODE) ? ((int64_t)b * p.H + h) * a.K_top
                                                       : (((int64_t)b * p.H + h) * a.N + t) * a.K_top;
            if (lane < a.K_top) {
                a.idx[base + lane] = lane < nkept ? id : -1;
                if (a.score) a.score[base + lane] = lane < nkept ? val : -INFINITY;
            }
        }
    }
};

template <int D, typename T, int G, int MODE, int SK = 0>
__global__ __launch_bounds__(64) void route_query_kernel(RouteArgs a)
{
    RouteQuery<D, T, G, 1, SK>::template run<MODE>(a);
}

// Decode: one workgroup per (sequence, KV head); kDecodeWaves waves share the
// scoring of a level's candidate groups (at the leaf level, one group per
// candidate block), so their loads are in flight together.
constexpr int kDecodeWaves = 8;

template <int D, typename T, int G, int SK = 0>
__global__ __launch_bounds__(64 * kDecodeWaves) void route_decode_kernel(RouteArgs a)
{
    RouteQuery<D, T, G, kDecodeWaves, SK>::template run<MODE_DECODE>(a);
}

// ---------------------------------------------------------------------------
// Stage 2: leaf scoring per retained level-2 node.
// Rows of a tile: QT = 16 / (G * TA) queries x TA terms x G heads.
// ---------------------------------------------------------------------------
template <int D, typename T, int G>
__global__ __launch_bounds__(256) void stage2_kernel(Stage2Args a)
{
    constexpr int TA = Src<T>::TERMS;
    constexpr int TB = Src<T>::TERMS;
    constexpr int R = G * TA;
    constexpr int QT = 16 / R;
    constexpr int KS = D / 32;
    constexpr int LDW = D + 8;
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    bf16* s_keys = reinterpret_cast<bf16*>(s_raw);

    const PyrArgs& p = a.p;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t chunk = blockIdx.x;
    if (chunk >= a.chunk_off[a.n_clusters]) return;
    // cluster: the last cl with chunk_off[cl] <= chunk
    int64_t lo = 0, hi = a.n_clusters;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (a.chunk_off[mid] <= chunk) lo = mid; else hi = mid;
    }
    const int64_t cl = lo;
    const int64_t e0 = a.offsets[cl] + (chunk - a.chunk_off[cl]) * kChunkQ;
    const int64_t e1 = min((int64_t)a.offsets[cl + 1], e0 + kChunkQ);
    const int64_t pnode = cl % a.M2;
    const int h = (int)((cl / a.M2) % p.H);
    const int b = (int)(cl / (a.M2 * p.H));
    const int64_t n = a.N;
    const int C = p.C, g = p.g;
    const int64_t row0 = pnode * g * C;
    const int nrows = g * C;

    // Stage the g leaf blocks of pnode: bf16 (hi) plane, and a lo plane for fp32 keys.
    const T* kb = (const T*)a.K + ((int64_t)b * p.N_cap * p.H + h) * D;
    for (int i = threadIdx.x; i < nrows * (D / 8); i += 256) {
        const int r = i / (D / 8), c8 = i % (D / 8);
        const bool ok = row0 + r < n;
        bf16x8 vh, vl;
        Src<T>::load(kb + (ok ? (row0 + r) : 0) * ((int64_t)p.H * D) + 8 * c8, ok, vh, vl);
        *reinterpret_cast<bf16x8*>(s_keys + r * LDW + 8 * c8) = vh;
        if constexpr (TB == 2) *reinterpret_cast<bf16x8*>(s_keys + (nrows + r) * LDW + 8 * c8) = vl;
    }
    __syncthreads();

    const float scale = kLog2e * rsqrtf((float)D);
    const int64_t M1 = (n + C - 1) / C;
    const int ntiles = (int)((e1 - e0 + QT - 1) / QT);
    const int ucols = g * a.K_top;
    for (int tile = wave; tile < ntiles; tile += 4) {
        // A operand rows: r -> (query ql, term, head)
        const int r = lane & 15;
        const int ql = r / R, term = (r % R) / G, head = r % G;
        const int64_t e = e0 + (int64_t)tile * QT + ql;
        const bool has = e < e1;
        const int ent = has ? a.entries[e] : 0;
        const int64_t tq = ent >> 6;
        bf16x8 qa[KS];
        {
            const T* qp = (const T*)a.Q + (((int64_t)b * n + tq) * a.H_q + (int64_t)h * G + head) * D + 8 * (lane >> 4);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 vh, vl;
                Src<T>::load(qp + 32 * s, has, vh, vl);
                qa[s] = term == 0 ? vh : vl;
            }
        }
        for (int cc = 0; cc < g; ++cc) {
            const int64_t leaf = pnode * g + cc;
            if (leaf >= M1) break;
            float y[4][4];  // [column tile][row i]; at most C/16 = 4 tiles
            const int ntc = C / 16;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                if (ct < ntc) {
                    const int krow = cc * C + 16 * ct + (lane & 15);
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(s_keys + krow * LDW + 32 * s + 8 * (lane >> 4));
                        acc = mfma(qa[s], bh, acc);
                        if constexpr (TB == 2) {
                            const bf16x8 bl = *reinterpret_cast<const bf16x8*>(s_keys + (nrows + krow) * LDW + 32 * s + 8 * (lane >> 4));
                            acc = mfma(qa[s], bl, acc);
                        }
                    }
                    const bool kok = row0 + krow < n;
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[ct][i] = kok ? acc[i] : -INFINITY;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[ct][i] = -INFINITY;
                }
            }
            // Fold the low query terms into the high ones (their rows hold the same head).
            if constexpr (TA == 2) {
                if constexpr (R <= 4) {
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                        {
                            const int j = (i + G < 4) ? i + G : i;
                            if (((i % R) / G) == 0 && j != i) y[ct][i] += y[ct][j];
                        }
                } else {
                    // R = 8 or 16: the low rows of a query sit R/2 rows (R/8 lane groups) further on.
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                        for (int i = 0; i < 4; ++i) y[ct][i] += shfl_xor(y[ct][i], 16 * (R / 8));
                }
            }
            // Per-row log-sum-exp over the C keys (4 tiles x 16 lanes), in base 2.
            float lse[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m = -INFINITY;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) m = fmaxf(m, y[ct][i] * scale);
                m = group_max(m, 16);
                float s = 0.f;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    if (ct < ntc) s += __builtin_amdgcn_exp2f(y[ct][i] * scale - m);
                s = group_sum(s, 16);
                lse[i] = m + __builtin_amdgcn_logf(s);
            }
            // Sum over the heads of each query, then write u (natural log).
            float uq[4];
            int nq_lane;  // queries held by this lane group
            if constexpr (R <= 4) {
                nq_lane = 4 / R;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float acc = 0.f;
                    if (q < 4 / R)
#pragma unroll
                        for (int hd = 0; hd < G; ++hd) acc += lse[q * R + hd];
                    uq[q] = acc * kLn2;
                }
            } else {
                nq_lane = 1;
                constexpr int HG = (TA == 2) ? R / 2 : R;  // distinct head rows per query
                float part = 0.f;
                if constexpr (TA == 2) {
                    // rows hold heads in the first half of the query's lane groups
#pragma unroll
                    for (int i = 0; i < 4; ++i) part += lse[i];
                    // sum over the lane groups that hold distinct heads
                    if constexpr (HG == 8) part += shfl_xor(part, 16);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) part += lse[i];
                    if constexpr (R >= 8) part += shfl_xor(part, 16);
                    if constexpr (R >= 16) part += shfl_xor(part, 32);
                }
                uq[0] = part * kLn2;
                uq[1] = uq[2] = uq[3] = 0.f;
            }
            // lane (lane & 15) == 0 of the first lane group of each query writes
            const int lg = lane >> 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int qtile;  // query index within the tile
                bool writer;
                if constexpr (R <= 4) {
                    qtile = lg * (4 / R) + q;
                    writer = (lane & 15) == 0 && q < nq_lane;
                } else {
                    qtile = lg / (R / 4);
                    writer = (lane & 15) == 0 && q == 0 && (lg % (R / 4)) == 0;
                }
                const int src = (qtile * R) & 15;  // a lane that loaded this query (k chunk 0)
                const int ent_q = shfl(ent, src);
                const int64_t eq = e0 + (int64_t)tile * QT + qtile;
                if (writer && eq < e1) {
                    const int64_t t_q = ent_q >> 6;
                    const int slot = ent_q & 63;
                    a.u[(((int64_t)b * p.H + h) * n + t_q) * ucols + slot * g + cc] = uq[q];
                }
            }
        }
    }
}

}  // namespace pisa
