// quality.hip -- block-selection quality against full attention
// ("Block Sparse Attention with Log-Linear Complexity", section 4.4 eq 35-36;
// appendix D.2 eq 55-57), causal.
//
//   1. block_lse_kernel: the log mass a_{h'}(B) of every (query head, row,
//      eligible leaf block) -- the log-sum-exp of the row's scaled scores over
//      the block's keys up to the row -- on 16x16x32 bf16 MFMA: a workgroup
//      holds 64 columns per wave (16 / G_Q rows x G_Q heads per 16-column tile,
//      four tiles) of queries in registers and streams the blocks' keys
//      through LDS, one block at a time, up to its last row's block;
//   2. quality_kernel: one thread per (sequence, KV head, row): normalises each
//      query head's log masses over the eligible blocks, averages the heads
//      (P(B), eq 56), builds the reference set (forced blocks plus the highest
//      P, ties to the lower index) and the selector's Recall@K, captured mass
//      and mass ratio.
#include "pisa_device.hpp"
#include "quality.hpp"

namespace pisa {

namespace {

constexpr int kQualNQT = 4;  // column tiles per wave

template <int D, int C>
__global__ __launch_bounds__(256) void block_lse_kernel(QualArgs a)
{
    constexpr int KS = D / 32, TPC = C / 16, LDW = D + 8, CH = D / 8;
    __shared__ __attribute__((aligned(16))) bf16 s_k[C * LDW];
    const int G = a.G, QT = 16 / G;
    const int rows_wg = 4 * kQualNQT * QT;
    const int64_t bh = blockIdx.y;
    const int b = (int)(bh / a.H_kv), h = (int)(bh % a.H_kv);
    const int64_t r0 = (int64_t)blockIdx.x * rows_wg;
    if (r0 >= a.N) return;
    const int lane = threadIdx.x & 63, lg = lane >> 4;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15, qi = col / G, head = col % G;
    const bf16* Qb = reinterpret_cast<const bf16*>(a.Q);
    const bf16* Kb = reinterpret_cast<const bf16*>(a.K) + (int64_t)b * a.N * a.H_kv * D + (int64_t)h * D;
    const int64_t kstride = (int64_t)a.H_kv * D;

    bf16x8 qb[kQualNQT][KS];
    int64_t row[kQualNQT];
#pragma unroll
    for (int qt = 0; qt < kQualNQT; ++qt) {
        row[qt] = r0 + (int64_t)(wave * kQualNQT + qt) * QT + qi;
        const int64_t r = row[qt] < a.N ? row[qt] : a.N - 1;
        const bf16* qp = Qb + (((int64_t)b * a.N + r) * a.H_q + (int64_t)h * G + head) * D + 8 * lg;
#pragma unroll
        for (int s = 0; s < KS; ++s) qb[qt][s] = load8h(qp + 32 * s);
    }
    const int64_t rlast = (r0 + rows_wg < a.N ? r0 + rows_wg : a.N) - 1;
    const int64_t cmax = rlast / C;
    const float sc2 = kLog2e * rsqrtf((float)D);
    for (int64_t B = 0; B <= cmax; ++B) {
        __syncthreads();  // the previous block's keys are consumed
        for (int p = threadIdx.x; p < C * CH; p += 256) {
            const int key = p / CH, dc = p % CH;
            const int64_t t = B * C + key;
            const bf16x8 v = load8h(Kb + (t < a.N ? t : 0) * kstride + 8 * dc);
            *reinterpret_cast<bf16x8*>(s_k + key * LDW + 8 * dc) = t < a.N ? v : zero8h();
        }
        __syncthreads();
#pragma unroll
        for (int qt = 0; qt < kQualNQT; ++qt) {
            const int64_t r = row[qt];
            // keys of block B visible to row r: [B C, min(B C + C, r + 1))
            const int64_t vis64 = r - B * C + 1;
            const int vis = vis64 < 0 ? 0 : (vis64 > C ? C : (int)vis64);
            if (ballot(vis > 0) == 0) continue;  // no column of this tile sees block B
            f32x4 acc[TPC];
#pragma unroll
            for (int rt = 0; rt < TPC; ++rt) {
                acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 ak = *reinterpret_cast<const bf16x8*>(s_k + (rt * 16 + (lane & 15)) * LDW + 32 * s + 8 * lg);
                    acc[rt] = mfma(ak, qb[qt][s], acc[rt]);
                }
            }
            float m = -INFINITY;
#pragma unroll
            for (int rt = 0; rt < TPC; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float z = rt * 16 + 4 * lg + i < vis ? acc[rt][i] * sc2 : -INFINITY;
                    acc[rt][i] = z;
                    m = fmaxf(m, z);
                }
            m = max_xor16(m);
            m = max_xor32(m);
            float sum = 0.f;
#pragma unroll
            for (int rt = 0; rt < TPC; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sum += vis > 0 ? __builtin_amdgcn_exp2f(acc[rt][i] - m) : 0.f;
            sum = add_xor16(sum);
            sum = add_xor32(sum);
            if (lg == 0 && r < a.N && vis > 0)
                a.lmass[(((int64_t)b * a.H_q + (int64_t)h * G + head) * a.N + r) * a.M1 + B] =
                    (m + __builtin_amdgcn_logf(sum)) * kLn2;
        }
    }
}

__global__ __launch_bounds__(256) void quality_kernel(QualArgs a)
{
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.B * a.H_kv * a.N;
    if (item >= total) return;
    const int64_t r = item % a.N;
    const int64_t bh = item / a.N;
    const int h = (int)(bh % a.H_kv), b = (int)(bh / a.H_kv);
    const int G = a.G, Kt = a.K_top;
    const int64_t c = r / a.C, nE = c + 1;
    const float* lm = a.lmass + (((int64_t)b * a.H_q + (int64_t)h * G) * a.N + r) * a.M1;
    const int64_t hstride = a.N * a.M1;
    float la[16];
    for (int g = 0; g < G; ++g) {  // each head's log normaliser over the eligible blocks
        float m = -INFINITY;
        for (int64_t B = 0; B < nE; ++B) m = fmaxf(m, lm[g * hstride + B]);
        float s = 0.f;
        for (int64_t B = 0; B < nE; ++B) s += __expf(lm[g * hstride + B] - m);
        la[g] = m + __logf(s);
    }
    auto mass = [&](int64_t B) {
        float p = 0.f;
        for (int g = 0; g < G; ++g) p += __expf(lm[g * hstride + B] - la[g]);
        return p / (float)G;
    };
    // top K_top - 3 of the non-forced blocks by (mass desc, index asc), kept sorted
    float tv[16];
    int ti[16];
    const int nfree = nE > Kt ? Kt - 3 : 0;
    int nt = 0;
    float* mo = a.mass ? a.mass + item * a.M1 : nullptr;
    for (int64_t B = 0; B < nE; ++B) {
        const float p = mass(B);
        if (mo) mo[B] = p;
        if (nfree == 0 || B == 0 || B == c || B == c - 1) continue;
        if (nt == nfree && !(p > tv[nt - 1])) continue;  // equal mass: the earlier (lower) index stays
        int k = nt < nfree ? nt++ : nfree - 1;
        while (k > 0 && p > tv[k - 1]) {
            tv[k] = tv[k - 1];
            ti[k] = ti[k - 1];
            --k;
        }
        tv[k] = p;
        ti[k] = (int)B;
    }
    if (mo)
        for (int64_t B = nE; B < a.M1; ++B) mo[B] = 0.f;
    // reference set, ascending
    int ref[16];
    int nr = 0;
    if (nE <= Kt) {
        for (int64_t B = 0; B < nE; ++B) ref[nr++] = (int)B;
    } else {
        ref[nr++] = 0;
        for (int k = 0; k < nt; ++k) ref[nr++] = ti[k];
        ref[nr++] = (int)(c - 1);
        ref[nr++] = (int)c;
        for (int x = 1; x < nr; ++x) {  // insertion sort of the middle
            const int v = ref[x];
            int y = x;
            while (y > 0 && ref[y - 1] > v) {
                ref[y] = ref[y - 1];
                --y;
            }
            ref[y] = v;
        }
    }
    if (a.ref)
        for (int k = 0; k < Kt; ++k) a.ref[item * Kt + k] = k < nr ? ref[k] : -1;
    const int32_t* sel = a.sel + item * Kt;
    float cap = 0.f, cap_ref = 0.f;
    int hit = 0;
    for (int k = 0; k < Kt; ++k) {
        const int s = sel[k];
        if (s >= 0 && s < nE) {
            cap += mass(s);
            for (int x = 0; x < nr; ++x) hit += ref[x] == s;
        }
    }
    for (int x = 0; x < nr; ++x) cap_ref += mass(ref[x]);
    a.recall[item] = (float)hit / (float)Kt;
    a.captured[item] = cap;
    a.ratio[item] = cap / cap_ref;
}

template <int D>
static hipError_t lse_d(const QualArgs& a, hipStream_t s)
{
    const int rows_wg = 4 * kQualNQT * (16 / a.G);
    const dim3 grid((unsigned)((a.N + rows_wg - 1) / rows_wg), (unsigned)(a.B * a.H_kv));
    if (a.C == 16) hipLaunchKernelGGL((block_lse_kernel<D, 16>), grid, dim3(256), 0, s, a);
    else if (a.C == 32) hipLaunchKernelGGL((block_lse_kernel<D, 32>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((block_lse_kernel<D, 64>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

size_t quality_workspace_bytes(int64_t B, int64_t N, int H_q, int C)
{
    return (size_t)B * H_q * N * ((N + C - 1) / C) * 4;
}

hipError_t launch_quality(QualArgs a, int d, hipStream_t s)
{
    hipError_t e = d == 64 ? lse_d<64>(a, s) : lse_d<128>(a, s);
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)a.B * a.H_kv * a.N;
    hipLaunchKernelGGL(quality_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace pisa
