// attn.hip -- block-sparse attention forward ("Block Sparse Attention with
// Log-Linear Complexity", section 3.1 eq 6; appendix B: future tokens inside
// a selected block are masked).
//
// One wave per (sequence, query row, KV head), four waves per workgroup; or,
// when there are few rows (decode), one workgroup per (sequence, row, KV head)
// whose four waves take every fourth selected block each and merge their
// partial softmax states (max, sum, output) through LDS at the end (NS = 4).
// Per selected block of C keys (C < 32 is padded to 32 with masked keys):
//   S^T = K_blk Q^T on MFMA: A = 16 keys x d, B = d x 16 columns holding the
//     G_Q query heads (and, for fp32 queries, their low halves). Tile rt's
//     row r holds key 32*(rt/2) + 8*(r/4) + 4*(rt%2) + r%4, so that after the
//     product every lane holds, for its head, the 8 consecutive keys that the
//     P V product needs from it: P is used straight from registers.
//   online softmax in base 2 per head (fp32);
//   O += P V on MFMA with V staged transposed in LDS (V^T[d][key]).
#include "pisa_device.hpp"
#include "pisa_internal.hpp"

namespace pisa {

template <int D, typename T, int G, int NS>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a, int Cp)
{
    static_assert(NS == 1 || NS == 4, "waves per row: one, or the whole workgroup");
    constexpr int TA = Src<T>::TERMS;  // query terms (columns per head)
    constexpr int TB = Src<T>::TERMS;  // key / value / probability terms
    constexpr int KS = D / 32;
    constexpr int CT = D / 16;          // output column tiles
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ldv = Cp + 8;  // V^T row stride (bf16)
    bf16* s_vt = reinterpret_cast<bf16*>(s_raw) + (size_t)wave * TB * D * ldv;

    const int64_t total = (int64_t)a.B * a.H_kv * a.N_q;
    const int64_t item = (int64_t)blockIdx.x * (4 / NS) + wave / NS;
    const int part = wave % NS;  // this wave's share of the row's blocks: k = part, part + NS, ...
    if (item >= total) return;   // NS = 4: the whole workgroup (no barrier is skipped)
    const int64_t r = item % a.N_q;
    const int h = (int)((item / a.N_q) % a.H_kv);
    const int b = (int)(item / ((int64_t)a.N_q * a.H_kv));
    int64_t nb = a.kv_len ? a.kv_len[b] : a.N_kv;  // lengths may live on the device: keep them in range
    nb = nb < 0 ? 0 : (nb > a.N_alloc ? a.N_alloc : nb);
    const int64_t pos = nb - a.N_q + r;
    const int C = a.C;

    // B operand: column j = lane % 16 -> (term, head); k chunk = lane / 16
    bf16x8 qb[KS];
    {
        const int j = lane & 15;
        const int term = j / G, head = j % G;
        const bool ok = j < G * TA && pos >= 0;
        const T* qp = (const T*)a.Q + (((int64_t)b * a.N_q + r) * a.H_q + (int64_t)h * G + head) * D + 8 * (lane >> 4);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 vh, vl;
            Src<T>::load(qp + 32 * s, ok, vh, vl);
            qb[s] = term == 0 ? vh : vl;
        }
    }
    const float scale = kLog2e * rsqrtf((float)D);
    const int col = lane & 15;          // this lane's head column in S^T
    const bool head_col = col < G;       // a combined (high + low) head lives here

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int32_t* sel = a.idx + (((int64_t)b * a.H_kv + h) * a.N_q + r) * a.K_top;
    const T* kbase = (const T*)a.K + ((int64_t)b * a.N_alloc * a.H_kv + h) * D;
    const T* vbase = (const T*)a.V + ((int64_t)b * a.N_alloc * a.H_kv + h) * D;
    const int64_t kstride = (int64_t)a.H_kv * D;
    const int nrt = Cp / 16;

    for (int k = part; k < a.K_top; k += NS) {
        const int blk = sel[k];
        if (blk < 0) continue;
        const int64_t k0 = (int64_t)blk * C;
        int64_t kend = k0 + C < nb ? k0 + C : nb;
        if (a.causal && kend > pos + 1) kend = pos + 1;
        if (kend <= k0) continue;  // no visible key in this block (uniform across the wave)

        // The block's loads are issued together, each at an address in the sequence (a masked
        // key reads row 0): the K rows of the four 16-key tiles first, so that the S products
        // wait for them only, then (bf16) the V rows, which go to LDS after the softmax; fp32
        // values, two terms each, are loaded after the softmax to stay within the registers.
        // A masked key's S entry is replaced by -inf (a select: whatever row 0 holds cannot leak)
        // and its V row is written as zeros.
        bf16x8 kh[4][KS], kl[4][KS];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int rr = lane & 15;
            const int key = 32 * (rt >> 1) + 8 * (rr >> 2) + 4 * (rt & 1) + (rr & 3);
            const bool kok = rt < nrt && k0 + key < kend && key < C;
            const T* kp = kbase + (kok ? (k0 + key) : 0) * kstride + 8 * (lane >> 4);
#pragma unroll
            for (int s = 0; s < KS; ++s) Src<T>::load(kp + 32 * s, true, kh[rt][s], kl[rt][s]);
        }
        // V: lane = key (lanes >= Cp load row 0 and write nothing)
        bf16x8 vh[D / 8], vl[D / 8];
        const T* vp = vbase + ((lane < Cp && k0 + lane < kend) ? (k0 + lane) : 0) * kstride;
        if constexpr (TB == 1) {
#pragma unroll
            for (int j = 0; j < D / 8; ++j) Src<T>::load(vp + 8 * j, true, vh[j], vl[j]);
        }

        // S^T tiles
        float y[4][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (rt < nrt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    acc = mfma(kh[rt][s], qb[s], acc);
                    if constexpr (TB == 2) acc = mfma(kl[rt][s], qb[s], acc);
                }
                // output rows 4*(lane/16)+i are keys of this tile
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int orow = 4 * (lane >> 4) + i;
                    const int okey = 32 * (rt >> 1) + 8 * (orow >> 2) + 4 * (rt & 1) + (orow & 3);
                    float v = acc[i];
                    if constexpr (TA == 2) v += __shfl_xor(v, G, 64);
                    y[rt][i] = (okey < C && k0 + okey < kend) ? v * scale : -INFINITY;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) y[rt][i] = -INFINITY;
            }
        }
        // online softmax per head column
        float mb = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mb = fmaxf(mb, y[rt][i]);
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const float m_new = fmaxf(m_run, mb);
        const float fac = __builtin_amdgcn_exp2f(m_run - m_new);
        float ps = 0.f;
        float pr[4][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = (rt < nrt && y[rt][i] != -INFINITY) ? __builtin_amdgcn_exp2f(y[rt][i] - m_new) : 0.f;
                pr[rt][i] = head_col ? pv : 0.f;
                ps += pv;
            }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l_run = l_run * fac + ps;
        m_run = m_new;
        // rescale O rows (heads 4*(lane/16)+i) by their heads' factors
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float f = __shfl(fac, 4 * (lane >> 4) + i, 64);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) o[ct][i] *= f;
        }
        if constexpr (TB == 2) {
#pragma unroll
            for (int j = 0; j < D / 8; ++j) Src<T>::load(vp + 8 * j, true, vh[j], vl[j]);
        }
        // Stage V^T (V^T[d][key]): pairs of lanes write packed dwords; a masked key's half is 0.
        {
            const bool even = (lane & 1) == 0;
            const int c0 = even ? lane : lane - 1;
            const uint32_t mine_ok = k0 + lane < kend ? 0xffffu : 0u;
            const uint32_t other_ok = k0 + (lane ^ 1) < kend ? 0xffffu : 0u;
#pragma unroll
            for (int j = 0; j < D / 8; ++j) {
#pragma unroll
                for (int tp = 0; tp < TB; ++tp) {
                    const bf16x8 v = tp == 0 ? vh[j] : vl[j];
                    const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
                    uint32_t pw[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) pw[q] = (uint32_t)__shfl_xor((int)w[q], 1, 64);
                    bf16* plane = s_vt + (size_t)tp * D * ldv;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // even lane: element 2q of itself (low) and of key+1 (high), row 8j+2q
                        // odd lane : element 2q+1 of key-1 (low) and of itself (high), row 8j+2q+1
                        const uint32_t mine = (even ? (w[q] & 0xffffu) : (w[q] >> 16)) & mine_ok;
                        const uint32_t other = (even ? (pw[q] & 0xffffu) : (pw[q] >> 16)) & other_ok;
                        const uint32_t dw = even ? (mine | (other << 16)) : (other | (mine << 16));
                        const int row = 8 * j + 2 * q + (even ? 0 : 1);
                        if (lane < Cp) *reinterpret_cast<uint32_t*>(plane + row * ldv + c0) = dw;
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // O += P V
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (2 * s < nrt) {
                f32x8 pv8;
#pragma unroll
                for (int i = 0; i < 4; ++i) { pv8[i] = pr[2 * s][i]; pv8[4 + i] = pr[2 * s + 1][i]; }
                // probabilities in bf16 (fp32 inputs: two bf16 terms)
                bf16x8 ph, pl;
                split8(pv8, ph, pl);
                (void)pl;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const int vrow = 16 * ct + (lane & 15);
                    const bf16* vp = s_vt + vrow * ldv + 32 * s + 8 * (lane >> 4);
                    const bf16x8 vh = *reinterpret_cast<const bf16x8*>(vp);
                    o[ct] = mfma(ph, vh, o[ct]);
                    if constexpr (TB == 2) {
                        const bf16x8 vl = *reinterpret_cast<const bf16x8*>(vp + (size_t)D * ldv);
                        o[ct] = mfma(ph, vl, o[ct]);
                        o[ct] = mfma(pl, vh, o[ct]);
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    if constexpr (NS > 1) {
        // merge the NS waves' states: with M = the largest running max of a head, the row's
        // sum is sum_w l_w 2^(m_w - M) and its output sum_w o_w 2^(m_w - M) (a wave that saw no
        // visible key has m_w = -inf and weighs 0). The V^T staging area is free again.
        __syncthreads();
        float* s_m = reinterpret_cast<float*>(s_raw);  // [NS][16] running max per head column
        float* s_l = s_m + NS * 16;                     // [NS][16] running sum
        float* s_o = s_l + NS * 16;                     // [NS][16 heads][D] unnormalised output
        if (lane < 16) {
            s_m[part * 16 + lane] = m_run;
            s_l[part * 16 + lane] = l_run;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int head = 4 * (lane >> 4) + i;
            if (head < G) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) s_o[(part * 16 + head) * D + 16 * ct + (lane & 15)] = o[ct][i];
            }
        }
        __syncthreads();
        if (part != 0) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int head = (4 * (lane >> 4) + i) & 15;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NS; ++w) M = fmaxf(M, s_m[w * 16 + head]);
            float L = 0.f;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) o[ct][i] = 0.f;
#pragma unroll
            for (int w = 0; w < NS; ++w) {
                const float mw = s_m[w * 16 + head];
                const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
                L += f * s_l[w * 16 + head];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) o[ct][i] += f * s_o[(w * 16 + head) * D + 16 * ct + (lane & 15)];
            }
        }
        // every lane: the merged (m, l) of head column lane % 16, as the single-wave path holds them
        {
            const int head = lane & 15;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NS; ++w) M = fmaxf(M, s_m[w * 16 + head]);
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < NS; ++w) {
                const float mw = s_m[w * 16 + head];
                L += (mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M)) * s_l[w * 16 + head];
            }
            m_run = M;
            l_run = L;
        }
    }

    // normalise and store rows (heads) 4*(lane/16)+i < G
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int head = 4 * (lane >> 4) + i;
        const float lh = __shfl(l_run, head & 15, 64);
        const float inv = lh > 0.f ? 1.f / lh : 0.f;
        if (head < G) {
            T* op = (T*)a.O + (((int64_t)b * a.N_q + r) * a.H_q + (int64_t)h * G + head) * D + (lane & 15);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) op[16 * ct] = static_cast<T>(o[ct][i] * inv);
        }
    }
    if (a.lse && lane < G) {
        a.lse[((int64_t)b * a.H_q + (int64_t)h * G + lane) * a.N_q + r] =
            l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
    }
}

// Rows (sequence x row x KV head) below which a row gets a whole workgroup (NS = 4): with
// one wave per row, 2,048 rows fill only two waves per CU.
constexpr int64_t kAttnSplitRows = 2048;

template <int D, typename T, int NS>
static hipError_t attn_ns(const AttnArgs& a, hipStream_t s)
{
    const int Cp = a.C < 32 ? 32 : a.C;
    // four waves' V^T staging; the NS = 4 merge reuses it for NS x 16 x (D + 2) floats
    const size_t stage = (size_t)4 * Src<T>::TERMS * D * (Cp + 8) * 2;
    const size_t merge = (size_t)NS * 16 * (D + 2) * 4;
    const size_t lds = NS > 1 && merge > stage ? merge : stage;
    const int64_t total = (int64_t)a.B * a.H_kv * a.N_q;
    const dim3 grid((unsigned)((total + 4 / NS - 1) / (4 / NS)));
#define PISA_ATTN_G(GG)                                                                                        \
    case GG: {                                                                                                 \
        auto k = attn_kernel<D, T, GG, NS>;                                                                    \
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
        if (e != hipSuccess) return e;                                                                         \
        hipLaunchKernelGGL(k, grid, dim3(256), lds, s, a, Cp);                                                 \
        return hipGetLastError();                                                                              \
    }
    switch (a.G) {
        PISA_ATTN_G(1)
        PISA_ATTN_G(2)
        PISA_ATTN_G(4)
        PISA_ATTN_G(8)
    case 16:
        if constexpr (Src<T>::TERMS == 1) {
            auto k = attn_kernel<D, T, 16, NS>;
            hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(k, grid, dim3(256), lds, s, a, Cp);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    default:
        return hipErrorInvalidValue;
    }
#undef PISA_ATTN_G
}

template <int D, typename T>
static hipError_t attn_d(const AttnArgs& a, hipStream_t s)
{
    const int64_t total = (int64_t)a.B * a.H_kv * a.N_q;
    return total < kAttnSplitRows ? attn_ns<D, T, 4>(a, s) : attn_ns<D, T, 1>(a, s);
}

hipError_t launch_attn(const AttnArgs& a, int dtype, int d, hipStream_t s)
{
    if (dtype == 0) return d == 64 ? attn_d<64, float>(a, s) : attn_d<128, float>(a, s);
    return d == 64 ? attn_d<64, bf16>(a, s) : attn_d<128, bf16>(a, s);
}

}  // namespace pisa
