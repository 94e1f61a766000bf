// bsa.hip -- exhaustive single-level block selection in the style of BSA
// ("Block Sparse Attention with Log-Linear Complexity", section 3.1 eq 2-5,
// with the per-head normalisation its BSA baseline applies before summing the
// heads of a group), the same-GPU comparison point for the pyramid router.
//
// Workgroup = 8 waves x QT queries of one KV head (QT = 16 / (G_Q * terms)).
// Leaf means (pyramid level 1, fp32) are staged 64 at a time in LDS as two
// bf16 terms and multiplied with the queries on MFMA (rows = query heads,
// columns = leaves). Two sweeps over the eligible leaves:
//   1. per head, a running base-2 log-sum-exp over the scored leaves;
//   2. p = exp(z - lse) per head, u = sum over the group's heads, and a
//      streaming top-(K_top - |forced|) list per lane; the 16 lanes of a
//      query merge their lists with shuffles at the end.
#include "pisa_device.hpp"
#include "pisa_internal.hpp"

namespace pisa {

constexpr int kBsaWaves = 8;
constexpr int kBsaKMax = 8;      // K_top of the MFMA-stationary kernel below (bsa_tile_kernel)
constexpr int kBsaKMaxWide = 16;  // largest K_top of the exhaustive selector (this kernel, KM = 16)

template <int D, typename T, int G, int KM>
__global__ __launch_bounds__(512) void bsa_kernel(BsaArgs a)
{
    constexpr int TA = Src<T>::TERMS;
    constexpr int R = G * TA;           // rows per query
    constexpr int QT = 16 / R;          // queries per wave
    constexpr int NQ = R <= 4 ? 4 / R : 1;  // queries held by one lane group
    constexpr int HG = R / TA;           // distinct head rows per query
    constexpr int KS = D / 32;
    constexpr int LDW = D + 8;
    __shared__ __attribute__((aligned(16))) bf16 s_m[2][64 * LDW];

    const PyrArgs& p = a.p;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lg = lane >> 4;
    const int64_t N = a.N;
    const int64_t per_wg = (int64_t)kBsaWaves * QT;
    const int64_t ntile = (N + per_wg - 1) / per_wg;
    const int64_t bh = blockIdx.x / ntile;
    const int64_t t0 = (blockIdx.x % ntile) * per_wg;
    const int h = (int)(bh % p.H), b = (int)(bh / p.H);
    const int64_t M1 = (N + p.C - 1) >> p.c_log2;
    const float* lev1 = p.buf + p.off[1] + ((int64_t)b * p.H + h) * p.M_cap[1] * D;

    // A operand rows
    bf16x8 qa[KS];
    {
        const int r = lane & 15;
        const int ql = r / R, term = (r % R) / G, head = r % G;
        const int64_t tq = t0 + (int64_t)wave * QT + ql;
        const bool has = tq < N;
        const T* qp = (const T*)a.Q + (((int64_t)b * N + (has ? tq : 0)) * a.H_q + (int64_t)h * G + head) * D + 8 * (lane >> 4);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 vh, vl;
            Src<T>::load(qp + 32 * s, has, vh, vl);
            qa[s] = term == 0 ? vh : vl;
        }
    }
    // per row i of this lane: its query and whether it scores at all
    int64_t tq_i[4], c_i[4];
    bool live_i[4], prim_i[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        const int ql = r / R, rq = r % R;
        tq_i[i] = t0 + (int64_t)wave * QT + ql;
        c_i[i] = tq_i[i] >> p.c_log2;
        const int64_t E = a.causal ? c_i[i] + 1 : M1;
        live_i[i] = tq_i[i] < N && E > a.K_top;
        prim_i[i] = (rq / G) == 0;
    }
    const int64_t tlast = min(N - 1, t0 + per_wg - 1);
    const int64_t last_leaf = a.causal ? (tlast >> p.c_log2) : M1 - 1;
    const int nchunks = (int)(last_leaf / 64) + 1;
    const float scale = kLog2e * rsqrtf((float)D);

    float m2[4], s2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m2[i] = -INFINITY; s2[i] = 0.f; }
    // top lists: per lane, per held query q (NQ), KMAX entries in selection order
    float tu[NQ][KM];
    int ti[NQ][KM];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int j = 0; j < KM; ++j) { tu[q][j] = -INFINITY; ti[q][j] = 0x7fffffff; }
    // number of ranked picks of each held query
    int rk[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int r = R <= 4 ? 4 * lg + q * R : 4 * lg;
        const int64_t tq = t0 + (int64_t)wave * QT + r / R;
        const int64_t c = tq >> p.c_log2;
        const int nF = a.causal ? (c == 0 ? 1 : (c == 1 ? 2 : 3)) : 0;
        rk[q] = a.K_top - nF;
    }

    for (int pass = 0; pass < 2; ++pass) {
        for (int ch = 0; ch < nchunks; ++ch) {
            __syncthreads();
            for (int i = threadIdx.x; i < 64 * (D / 8); i += 64 * kBsaWaves) {
                const int rr = i / (D / 8), c8 = i % (D / 8);
                const int64_t leaf = (int64_t)ch * 64 + rr;
                bf16x8 vh, vl;
                Src<float>::load(lev1 + (leaf < M1 ? leaf : 0) * D + 8 * c8, leaf < M1, vh, vl);
                *reinterpret_cast<bf16x8*>(&s_m[0][rr * LDW + 8 * c8]) = vh;
                *reinterpret_cast<bf16x8*>(&s_m[1][rr * LDW + 8 * c8]) = vl;
            }
            __syncthreads();
            float y[4][4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int rr = 16 * ct + (lane & 15);
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&s_m[0][rr * LDW + 32 * s + 8 * lg]);
                    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&s_m[1][rr * LDW + 32 * s + 8 * lg]);
                    acc = mfma(qa[s], bh, acc);
                    acc = mfma(qa[s], bl, acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) y[ct][i] = acc[i];
            }
            if constexpr (TA == 2) {
                if constexpr (R <= 4) {
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int j = (i + G < 4) ? i + G : i;
                            if (prim_i[i] && j != i) y[ct][i] += y[ct][j];
                        }
                } else {
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                        for (int i = 0; i < 4; ++i) y[ct][i] += shfl_xor(y[ct][i], 16 * (R / 8));
                }
            }
            // mask: eligible, not forced, query live
            bool ok[4][4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int64_t leaf = (int64_t)ch * 64 + 16 * ct + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t c = c_i[i];
                    bool v = live_i[i] && leaf < M1;
                    if (a.causal) v = v && leaf <= c && leaf != 0 && leaf != c && leaf != c - 1;
                    ok[ct][i] = v;
                    y[ct][i] *= scale;
                }
            }
            if (pass == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float cm = -INFINITY;
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) if (ok[ct][i]) cm = fmaxf(cm, y[ct][i]);
                    if (cm > m2[i]) {
                        s2[i] = (m2[i] == -INFINITY) ? 0.f : s2[i] * __builtin_amdgcn_exp2f(m2[i] - cm);
                        m2[i] = cm;
                    }
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        if (ok[ct][i]) s2[i] += __builtin_amdgcn_exp2f(y[ct][i] - m2[i]);
                }
            } else {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    float pv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        pv[i] = (ok[ct][i] && prim_i[i]) ? __builtin_amdgcn_exp2f(y[ct][i] - m2[i]) : 0.f;
                    const int leaf = ch * 64 + 16 * ct + (lane & 15);
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        float u = 0.f;
                        bool any = false;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bool mine = R <= 4 ? (i / R == q) : true;
                            if (mine) { u += pv[i]; any = any || ok[ct][i]; }
                        }
                        if constexpr (HG > 4) u += shfl_xor(u, 16);
                        if constexpr (HG > 8) u += shfl_xor(u, 32);
                        if (any) {
                            float xu = u;
                            int xi = leaf;
#pragma unroll
                            for (int j = 0; j < KM; ++j) {
                                if (j < rk[q] && before(xu, xi, tu[q][j], ti[q][j])) {
                                    const float t_ = tu[q][j]; tu[q][j] = xu; xu = t_;
                                    const int i_ = ti[q][j]; ti[q][j] = xi; xi = i_;
                                }
                            }
                        }
                    }
                }
            }
        }
        if (pass == 0) {
            // combine the 16 lanes of each row: (m, s) -> base-2 log-sum-exp
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m = m2[i], s = s2[i];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    const float mo = shfl_xor(m, o), so = shfl_xor(s, o);
                    const float mn = fmaxf(m, mo);
                    if (mn != -INFINITY)
                        s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(m - mn)) +
                            (mo == -INFINITY ? 0.f : so * __builtin_amdgcn_exp2f(mo - mn));
                    m = mn;
                }
                m2[i] = (m == -INFINITY) ? INFINITY : m + __builtin_amdgcn_logf(s);  // lse of the row
            }
        }
    }

    // merge the per-lane lists of each query over its 16 lanes
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            float ou[KM];
            int oi[KM];
#pragma unroll
            for (int j = 0; j < KM; ++j) { ou[j] = shfl_xor(tu[q][j], o); oi[j] = shfl_xor(ti[q][j], o); }
#pragma unroll
            for (int k = 0; k < KM; ++k) {
                float xu = ou[k];
                int xi = oi[k];
                if (xi == 0x7fffffff) continue;
#pragma unroll
                for (int j = 0; j < KM; ++j) {
                    if (j < rk[q] && before(xu, xi, tu[q][j], ti[q][j])) {
                        const float t_ = tu[q][j]; tu[q][j] = xu; xu = t_;
                        const int i_ = ti[q][j]; ti[q][j] = xi; xi = i_;
                    }
                }
            }
        }
    }

    // writers: lane (lane & 15) == 0 of the first lane group of each query
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        int qtile;
        bool writer;
        if constexpr (R <= 4) {
            qtile = lg * NQ + q;
            writer = (lane & 15) == 0;
        } else {
            qtile = lg / (R / 4);
            writer = (lane & 15) == 0 && (lg % (R / 4)) == 0;
        }
        const int64_t tq = t0 + (int64_t)wave * QT + qtile;
        if (!writer || tq >= N) continue;
        const int64_t c = tq >> p.c_log2;
        const int64_t E = a.causal ? c + 1 : M1;
        int ids[KM + 4];
        float val[KM + 4];
#pragma unroll
        for (int j = 0; j < KM + 4; ++j) { ids[j] = 0x7fffffff; val[j] = -INFINITY; }
        auto put = [&](int x, float v) {
#pragma unroll
            for (int j = 0; j < KM + 4; ++j)
                if (x < ids[j]) {
                    const int i_ = ids[j]; ids[j] = x; x = i_;
                    const float v_ = val[j]; val[j] = v; v = v_;
                }
        };
        if (E <= a.K_top) {
            for (int64_t l = 0; l < E; ++l) put((int)l, INFINITY);
        } else {
            if (a.causal) {
                put(0, INFINITY);
                if (c != 0) put((int)c, INFINITY);
                if (c - 1 >= 1) put((int)(c - 1), INFINITY);
            }
#pragma unroll
            for (int j = 0; j < KM; ++j)
                if (j < rk[q] && ti[q][j] != 0x7fffffff) put(ti[q][j], tu[q][j]);
        }
        const int64_t base = (((int64_t)b * p.H + h) * N + tq) * a.K_top;
#pragma unroll
        for (int j = 0; j < KM + 4; ++j) {
            if (j < a.K_top) {
                const bool okj = ids[j] != 0x7fffffff;
                a.idx[base + j] = okj ? ids[j] : -1;
                if (a.score) a.score[base + j] = okj ? val[j] : -INFINITY;
            }
        }
    }
}

// Output of one query: the forced blocks plus its ranked picks (or every eligible block when
// at most K_top are eligible), ascending, -1 padded; scores +inf for the unranked ones.
template <int KL>
__device__ __forceinline__ void bsa_write(const BsaArgs& a, int64_t b, int64_t h, int64_t tq, int64_t M1,
                                          const float* tu, const int* ti, int rk)
{
    const PyrArgs& p = a.p;
    const int64_t c = tq >> p.c_log2;
    const int64_t E = a.causal ? c + 1 : M1;
    int ids[KL + 3];
    float val[KL + 3];
#pragma unroll
    for (int j = 0; j < KL + 3; ++j) { ids[j] = 0x7fffffff; val[j] = -INFINITY; }
    auto put = [&](int x, float v) {
#pragma unroll
        for (int j = 0; j < KL + 3; ++j)
            if (x < ids[j]) {
                const int i_ = ids[j]; ids[j] = x; x = i_;
                const float v_ = val[j]; val[j] = v; v = v_;
            }
    };
    if (E <= a.K_top) {
        for (int64_t l = 0; l < E; ++l) put((int)l, INFINITY);
    } else {
        if (a.causal) {
            put(0, INFINITY);
            if (c != 0) put((int)c, INFINITY);
            if (c - 1 >= 1) put((int)(c - 1), INFINITY);
        }
#pragma unroll
        for (int j = 0; j < KL; ++j)
            if (j < rk && ti[j] != 0x7fffffff) put(ti[j], tu[j]);
    }
    const int64_t base = (((int64_t)b * p.H + h) * a.N + tq) * a.K_top;
#pragma unroll
    for (int j = 0; j < KL + 3; ++j) {
        if (j < a.K_top) {
            const bool okj = ids[j] != 0x7fffffff;
            a.idx[base + j] = okj ? ids[j] : -1;
            if (a.score) a.score[base + j] = okj ? val[j] : -INFINITY;
        }
    }
}

// bf16 queries, G_Q in {4, 8, 16}: the queries are the stationary MFMA A operand (a 16-row
// tile = 16 / G queries x G heads; NA tiles per wave, 8 waves per workgroup) and the leaf
// means stream through LDS as the B operand, 64 leaves per double-buffered batch (fp32
// means as two bf16 terms), so one staged batch feeds 8 * NA * 16 / G queries. A lane of
// an output tile holds four heads of one query for one leaf column:
//   pass 1: per head, a base-2 log-sum-exp over the scored leaves, one max rescale per
//           batch (the lane's leaves are those of its column; 16 lanes combine at the end);
//   pass 2: u = sum over the group's heads of 2^(z - lse), heads beyond the lane's four
//           added across lane groups, and a per-lane top list (KL = the ranked picks)
//           merged over the 16 columns at the end.
template <int D, int G, int NA, int KL>
__global__ __launch_bounds__(512) void bsa_tile_kernel(BsaArgs a)
{
    static_assert(G == 4 || G == 8 || G == 16, "four or more heads per KV head");
    constexpr int KS = D / 32, QA = 16 / G, QW = NA * QA, QG = 8 * QW;
    constexpr int LB = 64, LDW = D + 8;
    constexpr int CPT = LB * (D / 8) / 512;  // 8-float pieces of a batch per thread
    static_assert(CPT >= 1, "a batch covers the workgroup");
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    bf16* sb = reinterpret_cast<bf16*>(s_raw);  // [2 buffers][2 terms][LB][LDW]

    const PyrArgs& p = a.p;
    const int lane = threadIdx.x & 63, lg = lane >> 4, col = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t N = a.N;
    const int64_t ntile = (N + QG - 1) / QG;
    const int64_t bh = blockIdx.x / ntile;
    const int64_t t0 = (blockIdx.x % ntile) * QG;
    const int h = (int)(bh % p.H), b = (int)(bh / p.H);
    const int64_t M1 = (N + p.C - 1) >> p.c_log2;
    const float* lev1 = p.buf + p.off[1] + ((int64_t)b * p.H + h) * p.M_cap[1] * D;

    bf16x8 A[NA][KS];
#pragma unroll
    for (int x = 0; x < NA; ++x) {
        const int r = lane & 15;
        const int64_t tq = t0 + (int64_t)wave * QW + x * QA + r / G;
        const bool has = tq < N;
        const bf16* qp = (const bf16*)a.Q + (((int64_t)b * N + (has ? tq : 0)) * a.H_q + (int64_t)h * G + r % G) * D +
                         8 * lg;
#pragma unroll
        for (int s = 0; s < KS; ++s) A[x][s] = has ? load8h(qp + 32 * s) : zero8h();
    }
    // this lane's output rows 4 lg .. 4 lg + 3 of tile x: four heads of query (4 lg) / G
    int64_t cq[NA], tqx[NA];
    bool live[NA];
    int rk[NA];
#pragma unroll
    for (int x = 0; x < NA; ++x) {
        tqx[x] = t0 + (int64_t)wave * QW + x * QA + (4 * lg) / G;
        cq[x] = tqx[x] >> p.c_log2;
        const int64_t E = a.causal ? cq[x] + 1 : M1;
        live[x] = tqx[x] < N && E > a.K_top;
        const int nF = a.causal ? (cq[x] == 0 ? 1 : (cq[x] == 1 ? 2 : 3)) : 0;
        rk[x] = a.K_top - nF;
    }
    const int64_t tl = min(N - 1, t0 + QG - 1);
    const int64_t last_leaf = a.causal ? (tl >> p.c_log2) : M1 - 1;
    const int nb = (int)(last_leaf / LB) + 1;
    const float scale = kLog2e * rsqrtf((float)D);

    f32x8 pre[CPT];
    auto load_batch = [&](int bt) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int item = threadIdx.x + 512 * j, rr = item / (D / 8), c8 = item % (D / 8);
            const int64_t leaf = (int64_t)bt * LB + rr;
            const bool ok = leaf < M1;
            const f32x8 v = load8f(lev1 + (ok ? leaf : 0) * D + 8 * c8);
#pragma unroll
            for (int k = 0; k < 8; ++k) pre[j][k] = ok ? v[k] : 0.f;
        }
    };
    auto store_batch = [&](int buf) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int item = threadIdx.x + 512 * j, rr = item / (D / 8), c8 = item % (D / 8);
            bf16x8 hi, lo;
            split8(pre[j], hi, lo);
            *reinterpret_cast<bf16x8*>(sb + ((buf * 2 + 0) * LB + rr) * LDW + 8 * c8) = hi;
            *reinterpret_cast<bf16x8*>(sb + ((buf * 2 + 1) * LB + rr) * LDW + 8 * c8) = lo;
        }
    };

    float m2[NA][4], s2[NA][4];
#pragma unroll
    for (int x = 0; x < NA; ++x)
#pragma unroll
        for (int i = 0; i < 4; ++i) { m2[x][i] = -INFINITY; s2[x][i] = 0.f; }
    float tu[NA][KL];
    int ti[NA][KL];
#pragma unroll
    for (int x = 0; x < NA; ++x)
#pragma unroll
        for (int j = 0; j < KL; ++j) { tu[x][j] = -INFINITY; ti[x][j] = 0x7fffffff; }

    for (int pass = 0; pass < 2; ++pass) {
        load_batch(0);
        __syncthreads();  // the previous pass's last batch is consumed
        store_batch(0);
        __syncthreads();
        for (int bt = 0; bt < nb; ++bt) {
            const int cur = bt & 1;
            if (bt + 1 < nb) load_batch(bt + 1);
            const bf16* sh = sb + (cur * 2 + 0) * LB * LDW;
            const bf16* sl = sb + (cur * 2 + 1) * LB * LDW;
            f32x4 acc[4][NA];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
                for (int x = 0; x < NA; ++x) acc[ct][x] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int row = ct * 16 + col;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 bh_ = *reinterpret_cast<const bf16x8*>(sh + row * LDW + 32 * s + 8 * lg);
                    const bf16x8 bl_ = *reinterpret_cast<const bf16x8*>(sl + row * LDW + 32 * s + 8 * lg);
#pragma unroll
                    for (int x = 0; x < NA; ++x) {
                        acc[ct][x] = mfma(A[x][s], bh_, acc[ct][x]);
                        acc[ct][x] = mfma(A[x][s], bl_, acc[ct][x]);
                    }
                }
            }
            bool ok[4][NA];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int64_t leaf = (int64_t)bt * LB + ct * 16 + col;
#pragma unroll
                for (int x = 0; x < NA; ++x) {
                    bool v = live[x] && leaf < M1;
                    if (a.causal) v = v && leaf <= cq[x] && leaf != 0 && leaf != cq[x] && leaf != cq[x] - 1;
                    ok[ct][x] = v;
                }
            }
            if (pass == 0) {
#pragma unroll
                for (int x = 0; x < NA; ++x)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float bm = -INFINITY;
#pragma unroll
                        for (int ct = 0; ct < 4; ++ct)
                            if (ok[ct][x]) bm = fmaxf(bm, acc[ct][x][i] * scale);
                        if (bm > m2[x][i]) {
                            s2[x][i] = m2[x][i] == -INFINITY ? 0.f : s2[x][i] * __builtin_amdgcn_exp2f(m2[x][i] - bm);
                            m2[x][i] = bm;
                        }
#pragma unroll
                        for (int ct = 0; ct < 4; ++ct)
                            if (ok[ct][x]) s2[x][i] += __builtin_amdgcn_exp2f(fmaf(acc[ct][x][i], scale, -m2[x][i]));
                    }
            } else {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int leaf = bt * LB + ct * 16 + col;
#pragma unroll
                    for (int x = 0; x < NA; ++x) {
                        float u = 0.f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) u += __builtin_amdgcn_exp2f(fmaf(acc[ct][x][i], scale, -m2[x][i]));
                        if constexpr (G >= 8) u += shfl_xor(u, 16);
                        if constexpr (G >= 16) u += shfl_xor(u, 32);
                        if (ok[ct][x]) {
                            // a lane meets its leaves in increasing order, so an equal score never
                            // displaces an earlier (lower) leaf: a strict comparison keeps the tie rule
                            float xu = u;
                            int xi = leaf;
#pragma unroll
                            for (int j = 0; j < KL; ++j) {
                                if (j < rk[x] && xu > tu[x][j]) {
                                    const float t_ = tu[x][j]; tu[x][j] = xu; xu = t_;
                                    const int i_ = ti[x][j]; ti[x][j] = xi; xi = i_;
                                }
                            }
                        }
                    }
                }
            }
            if (bt + 1 < nb) {
                store_batch(cur ^ 1);  // its previous batch was read before the last barrier
                __syncthreads();
            }
        }
        if (pass == 0) {
            // the 16 columns of a lane group hold the same rows: combine (m, s) -> base-2 lse
#pragma unroll
            for (int x = 0; x < NA; ++x)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float m = m2[x][i], s = s2[x][i];
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) {
                        const float mo = shfl_xor(m, o), so = shfl_xor(s, o);
                        const float mn = fmaxf(m, mo);
                        if (mn != -INFINITY)
                            s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(m - mn)) +
                                (mo == -INFINITY ? 0.f : so * __builtin_amdgcn_exp2f(mo - mn));
                        m = mn;
                    }
                    // no scored leaf: +inf makes every 2^(z - lse) zero (the row is not ranked)
                    m2[x][i] = m == -INFINITY ? INFINITY : m + __builtin_amdgcn_logf(s);
                }
        }
    }

    // merge the per-column lists of each query over its 16 lanes, then one lane writes it
#pragma unroll
    for (int x = 0; x < NA; ++x) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            float ou[KL];
            int oi[KL];
#pragma unroll
            for (int j = 0; j < KL; ++j) { ou[j] = shfl_xor(tu[x][j], o); oi[j] = shfl_xor(ti[x][j], o); }
#pragma unroll
            for (int k = 0; k < KL; ++k) {
                float xu = ou[k];
                int xi = oi[k];
                if (xi == 0x7fffffff) continue;
#pragma unroll
                for (int j = 0; j < KL; ++j) {
                    if (j < rk[x] && before(xu, xi, tu[x][j], ti[x][j])) {
                        const float t_ = tu[x][j]; tu[x][j] = xu; xu = t_;
                        const int i_ = ti[x][j]; ti[x][j] = xi; xi = i_;
                    }
                }
            }
        }
        const bool writer = col == 0 && (4 * lg) % G == 0;  // first lane group of each query
        if (writer && tqx[x] < N) bsa_write<KL>(a, b, h, tqx[x], M1, tu[x], ti[x], rk[x]);
    }
}

template <int D, int G>
static hipError_t bsa_tile_launch(const BsaArgs& a, hipStream_t s)
{
    // A tiles per wave (more spill registers): 8 / 4 / 2 queries per wave for G = 4 / 8 / 16
    constexpr int NA = 2;
    constexpr int QG = 8 * NA * (16 / G);
    const size_t lds = (size_t)2 * 2 * 64 * (D + 8) * 2;
    // ranked picks per query: K_top - 3 for causal rows that rank (the first, previous and
    // current blocks are forced whenever more than K_top blocks are eligible), else K_top
    const bool five = a.causal && a.K_top == 8;
    const void* k = five ? (const void*)bsa_tile_kernel<D, G, NA, 5> : (const void*)bsa_tile_kernel<D, G, NA, kBsaKMax>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t grid = (int64_t)a.p.B * a.p.H * ((a.N + QG - 1) / QG);
    BsaArgs arg = a;
    void* args[] = {&arg};
    hipError_t e = hipLaunchKernel(k, dim3((unsigned)grid), dim3(512), args, lds, s);
    return e != hipSuccess ? e : hipGetLastError();
}

template <int D, typename T, int KM>
static hipError_t bsa_dk(const BsaArgs& a, hipStream_t s)
{
    const int R = a.G * Src<T>::TERMS;
    const int64_t per_wg = (int64_t)kBsaWaves * (16 / R);
    const int64_t grid = (int64_t)a.p.B * a.p.H * ((a.N + per_wg - 1) / per_wg);
    switch (a.G) {
    case 1: hipLaunchKernelGGL((bsa_kernel<D, T, 1, KM>), dim3((unsigned)grid), dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL((bsa_kernel<D, T, 2, KM>), dim3((unsigned)grid), dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL((bsa_kernel<D, T, 4, KM>), dim3((unsigned)grid), dim3(512), 0, s, a); break;
    case 8: hipLaunchKernelGGL((bsa_kernel<D, T, 8, KM>), dim3((unsigned)grid), dim3(512), 0, s, a); break;
    case 16:
        if constexpr (Src<T>::TERMS == 1) {
            hipLaunchKernelGGL((bsa_kernel<D, T, 16, KM>), dim3((unsigned)grid), dim3(512), 0, s, a);
            break;
        }
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, typename T>
static hipError_t bsa_d(const BsaArgs& a, hipStream_t s)
{
    return a.K_top <= kBsaKMax ? bsa_dk<D, T, kBsaKMax>(a, s) : bsa_dk<D, T, kBsaKMaxWide>(a, s);
}

hipError_t launch_bsa(const BsaArgs& a, int dtype, int d, hipStream_t s)
{
    if (dtype == 0) return d == 64 ? bsa_d<64, float>(a, s) : bsa_d<128, float>(a, s);
    if (a.K_top <= kBsaKMax && (a.G == 4 || a.G == 8 || a.G == 16)) {  // queries stationary in MFMA registers
        if (d == 64)
            return a.G == 4 ? bsa_tile_launch<64, 4>(a, s) : (a.G == 8 ? bsa_tile_launch<64, 8>(a, s) : bsa_tile_launch<64, 16>(a, s));
        return a.G == 4 ? bsa_tile_launch<128, 4>(a, s) : (a.G == 8 ? bsa_tile_launch<128, 8>(a, s) : bsa_tile_launch<128, 16>(a, s));
    }
    return d == 64 ? bsa_d<64, bf16>(a, s) : bsa_d<128, bf16>(a, s);
}

}  // namespace pisa
