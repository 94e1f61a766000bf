// attn_cl.hip -- clustered block-sparse attention forward for many query rows
// ("Block Sparse Attention with Log-Linear Complexity", section 3.1 eq 6;
// appendix B: future tokens inside a selected block are masked).
//
// The softmax over a row's selected blocks factors over the blocks: with
// m_j = max of the row's scaled scores in block j, l_j = sum of 2^(z - m_j)
// and O_j = sum of 2^(z - m_j) v / l_j, the row's output is
//   O = sum_j w_j O_j / sum_j w_j,  w_j = 2^(m_j + log2 l_j - M),  M = max_j (m_j + log2 l_j),
// and its log-normaliser is (M + log2 sum_j w_j) ln 2. So the (row, selected
// block) pairs can be computed in any grouping:
//   1. count / scatter: the pairs with at least one visible key become entries
//      (row << 6) | slot, clustered by (sequence, KV head, block);
//   2. attn_cl_kernel: a workgroup takes a chunk of one cluster, holds the
//      block's C keys in MFMA A registers and its values transposed in LDS,
//      streams the entries' G query heads through the LDS ring, and writes
//      for each (entry, head) m_j + log2 l_j, an exponent e_j and
//      O_j 2^-e_j in fp16 (e_j puts the row's largest |element| below 1, so
//      the stored row keeps 11 significant bits), P entering the P V product
//      as two bf16 terms;
//   3. attn_combine_kernel: one wave per (sequence, row, KV head) merges its
//      K_top partials.
// A block's keys and values are read once per chunk of up to 256 rows instead
// of once per row.
#include <algorithm>

#include "attn_bwd.hpp"
#include "pisa_device.hpp"
#include "pisa_internal.hpp"
#include "stream.hpp"

namespace pisa {

namespace {

constexpr int kClRowsPerThread = 4;
constexpr int kClThreads = 256;
constexpr int kClRowsPerBlock = kClThreads * kClRowsPerThread;
constexpr int kClLdsBins = 8192;  // blocks per sequence aggregated in LDS (more: global atomics)
constexpr int kAttnNB = 3;        // LDS ring depth with the fetch wave
constexpr bool kAttnFW = false;   // a dedicated fetch wave (costs a workgroup per CU in occupancy)

struct RowGeom {
    int64_t nb;   // keys of the sequence
    int64_t pos;  // position of the row
};

__device__ __forceinline__ RowGeom row_geom(const AttnClArgs& a, int b, int64_t r)
{
    int64_t nb = a.kv_len ? a.kv_len[b] : a.N_kv;
    nb = nb < 0 ? 0 : (nb > a.N_alloc ? a.N_alloc : nb);
    return RowGeom{nb, nb - a.N_q + r};
}

// Visible keys of block blk for a row: [k0, kend) with kend - k0 <= C.
__device__ __forceinline__ int64_t block_end(const AttnClArgs& a, const RowGeom& g, int64_t k0)
{
    int64_t kend = k0 + a.C < g.nb ? k0 + a.C : g.nb;
    if (a.causal && kend > g.pos + 1) kend = g.pos + 1;
    return kend;
}

__device__ __forceinline__ int lds_add_cl(int* base_arr, int P)
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
    return atomicAdd(&base_arr[P], 1);
}

// phase 0: cluster sizes; phase 1: entries. grid (row blocks, B * H_kv).
__global__ __launch_bounds__(kClThreads) void attn_cluster_kernel(AttnClArgs a, int phase)
{
    extern __shared__ int s_mem[];
    const int64_t bh = blockIdx.y;
    const int b = (int)(bh / a.H_kv);
    const int64_t r0 = (int64_t)blockIdx.x * kClRowsPerBlock;
    const int64_t cbase = bh * a.M_blk;
    const bool use_lds = a.M_blk <= kClLdsBins;
    int* s_cnt = s_mem;
    int* s_pos = s_mem + a.M_blk;
    if (use_lds) {
        for (int64_t k = threadIdx.x; k < a.M_blk; k += kClThreads) s_cnt[k] = 0;
        __syncthreads();
    }
    // pass over the rows: count (LDS or global), or place when counting globally
    for (int it = 0; it < kClRowsPerThread; ++it) {
        const int64_t r = r0 + (int64_t)it * kClThreads + threadIdx.x;
        if (r >= a.N_q) continue;
        const RowGeom g = row_geom(a, b, r);
        const int32_t* sel = a.idx + (bh * a.N_q + r) * a.K_top;
        for (int k = 0; k < a.K_top; ++k) {
            const int blk = sel[k];
            if (blk < 0) continue;
            const int64_t k0 = (int64_t)blk * a.C;
            if (k0 >= g.nb || block_end(a, g, k0) <= k0) continue;
            if (use_lds) {
                lds_add_cl(s_cnt, blk);
            } else if (phase == 0) {
                atomicAdd(&a.counts[cbase + blk], 1);
            } else {
                const int p = a.offsets[cbase + blk] + atomicAdd(&a.cursor[cbase + blk], 1);
                a.entries[p] = (int32_t)((r << 6) | k);
            }
        }
    }
    if (!use_lds) return;
    __syncthreads();
    if (phase == 0) {
        for (int64_t k = threadIdx.x; k < a.M_blk; k += kClThreads)
            if (s_cnt[k]) atomicAdd(&a.counts[cbase + k], s_cnt[k]);
        return;
    }
    for (int64_t k = threadIdx.x; k < a.M_blk; k += kClThreads) {
        const int v = s_cnt[k];
        s_pos[k] = v ? a.offsets[cbase + k] + atomicAdd(&a.cursor[cbase + k], v) : 0;
    }
    __syncthreads();
    for (int it = 0; it < kClRowsPerThread; ++it) {
        const int64_t r = r0 + (int64_t)it * kClThreads + threadIdx.x;
        if (r >= a.N_q) continue;
        const RowGeom g = row_geom(a, b, r);
        const int32_t* sel = a.idx + (bh * a.N_q + r) * a.K_top;
        for (int k = 0; k < a.K_top; ++k) {
            const int blk = sel[k];
            if (blk < 0) continue;
            const int64_t k0 = (int64_t)blk * a.C;
            if (k0 >= g.nb || block_end(a, g, k0) <= k0) continue;
            const int p = lds_add_cl(s_pos, blk);
            a.entries[p] = (int32_t)((r << 6) | k);
        }
    }
}

// Position of key kk (< 32) of a 32-key step in the transposed value rows:
// the P V product's B operand holds, in lane group lg, the probabilities of
// keys 4 lg .. 4 lg + 3 of the step's two S row tiles, so those eight keys sit
// side by side.
__device__ __forceinline__ int vt_pos(int key)
{
    const int kk = key & 31;
    return (key & ~31) + 8 * ((kk >> 2) & 3) + 4 * (kk >> 4) + (kk & 3);
}

// Row d of the transposed values holds its NK key positions with groups of eight XOR-swizzled by
// d / 8, so that the 16-bit stores of the eight d of one 16-byte value piece fall in different
// banks, while the eight positions an MFMA operand reads stay one 16-byte load.
template <int NK>
__device__ __forceinline__ int vt_swz(int d, int pos)
{
    return pos ^ ((((d >> 3) & (NK / 8 - 1))) << 3);
}

template <int D, int C, int NB, bool FW>
__global__ __launch_bounds__(FW ? 320 : 256) __attribute__((amdgpu_waves_per_eu(3))) void attn_cl_kernel(AttnClArgs a)
{
    constexpr int KS = D / 32;         // k-steps of S = K Q^T
    constexpr int TPC = C / 16;        // key row tiles
    constexpr int PS = (C + 31) / 32;  // 32-key steps of O = P V (C = 16: padded)
    constexpr int DT = D / 16;         // d tiles of O
    constexpr int CH = D / 8;
    constexpr int VLD = PS * 32 + 8;   // transposed value row stride (bf16)
    constexpr int NI = StreamGeom<D>::NI;
    static_assert(16 % CH == 0, "a row tile spans whole swizzle periods");
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    bf16* s_ring = reinterpret_cast<bf16*>(s_raw);                                  // [NB][kSubRows][D]
    bf16* s_vt = s_ring + (size_t)NB * kSubRows * D;                                // [D][VLD]
    int* s_ent = reinterpret_cast<int*>(s_vt + (size_t)D * VLD);                    // [kLeafQC]

    const int64_t total = a.chunk_off[a.n_clusters];
    if ((int64_t)blockIdx.x >= total) return;
    const int64_t chunk = blockIdx.x;
    const int64_t cl = a.chunk_cl[chunk];
    const int e0 = a.offsets[cl] + (int)(chunk - a.chunk_off[cl]) * a.qc;
    const int e1 = min(a.offsets[cl + 1], e0 + a.qc);
    const int n = e1 - e0;
    const int64_t blk = cl % a.M_blk;
    const int64_t bh = cl / a.M_blk;
    const int h = (int)(bh % a.H_kv);
    const int b = (int)(bh / a.H_kv);
    const int lane = threadIdx.x & 63, lg = lane >> 4;
    // FW: waves 0-3 compute and wave 4 fetches the query rows: it alone issues and waits for
    // the global-to-LDS loads, so its vmcnt counts nothing else and the compute waves' stores
    // never stall on them. Otherwise every compute wave fetches its own share of each sub-chunk
    // and waits for everything it issued (NB = 2).
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool fetcher = FW && wave == 4;
    static_assert(FW || NB == 2, "without the fetch wave the stores count in vmcnt: wait for all");
    const int G = a.G, QT = 16 / G, SE = kSubRows / G;
    const int glog = __builtin_ctz(G);
    const RowGeom g0 = row_geom(a, b, 0);
    const int64_t nb = g0.nb;
    const int64_t k0 = blk * C;
    const int kexist = (int)((k0 + C < nb ? k0 + C : nb) - k0);  // keys of the block that exist (>= 1)

    const bf16* Qb = reinterpret_cast<const bf16*>(a.Q) + (int64_t)b * a.N_q * a.H_q * D + (int64_t)h * G * D;
    const uint32_t qrow = (uint32_t)(a.H_q * D);
    const int nsb = (n + SE - 1) / SE;

    StreamLane sl[4];  // fetch wave: the rows of the four compute waves' shares
    bf16x8 A[TPC][KS];
    StreamPrologue<D, NB> pr;  // without the fetch wave: this wave's share
    if (!FW) {
        sl[0] = stream_lane<D>(wave, lane, glog);
        stream_prologue_load<D, NB>(pr, a.entries + e0, n, SE, sl[0], glog);
        stream_prologue_issue<D, NB>(pr, s_ent, Qb, qrow, sl[0], s_ring, wave);
    }
    if (fetcher) {
#pragma unroll
        for (int w = 0; w < 4; ++w) sl[w] = stream_lane<D>(w, lane, glog);
        int pe[NB - 1][4][NI];
#pragma unroll
        for (int k = 0; k < NB - 1; ++k)
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int el = k * SE + sl[w].el0 + ((i * StreamGeom<D>::STEP) >> glog);
                    const int lim = min(n, (k + 1) * SE) - 1;
                    pe[k][w][i] = a.entries[e0 + max(0, min(el, lim))];
                }
        wait_vm<0>();
        // branch-free: sub-chunks past the end refetch the last entry into buffers no tile reads
#pragma unroll
        for (int k = 0; k < NB - 1; ++k)
#pragma unroll
            for (int w = 0; w < 4; ++w) stream_issue<D>(Qb, qrow, pe[k][w], sl[w], s_ring + k * kSubRows * D, w);
    } else {
        if (FW) s_ent[threadIdx.x] = a.entries[e0 + min((int)threadIdx.x, n - 1)];  // slots past n: copies
        const int64_t kvstride = (int64_t)a.H_kv * D;
        const bf16* kb = reinterpret_cast<const bf16*>(a.K) + ((int64_t)b * a.N_alloc + k0) * kvstride + (int64_t)h * D;
        const bf16* vb = reinterpret_cast<const bf16*>(a.V) + ((int64_t)b * a.N_alloc + k0) * kvstride + (int64_t)h * D;
        // values: thread t loads 16-byte pieces (key, 8 d) of the padded block, then writes them transposed
        constexpr int VPIECES = PS * 32 * CH;
        constexpr int VPT = (VPIECES + 255) / 256;
        bf16x8 vreg[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int p = threadIdx.x + 256 * i;
            const int key = p / CH, dc = p % CH;
            const bool ok = p < VPIECES && key < kexist;
            const bf16x8 v = load8h(vb + (ok ? (int64_t)key * kvstride : 0) + 8 * dc);
            vreg[i] = ok ? v : zero8h();
        }
        // keys: A operand rows (lane & 15) of each row tile, k-chunk 8 * lg + 32 * s
#pragma unroll
        for (int rt = 0; rt < TPC; ++rt) {
            const int key = rt * 16 + (lane & 15);
            const bool ok = key < kexist;
            const bf16* kp = kb + (ok ? (int64_t)key * kvstride : 0) + 8 * lg;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 v = load8h(kp + 32 * s);
                A[rt][s] = ok ? v : zero8h();
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int p = threadIdx.x + 256 * i;
            if (p < VPIECES) {
                const int key = p / CH, dc = p % CH;
                const int vp = vt_pos(key);
#pragma unroll
                for (int j = 0; j < 8; ++j) s_vt[(8 * dc + j) * VLD + vt_swz<PS * 32>(8 * dc, vp)] = vreg[i][j];
            }
        }
    }

    const float scale = kLog2e * rsqrtf((float)D);
    const int col = lane & 15;
    const int qi = col / G, head = col % G;
    int boff[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) boff[s] = (col * D + 8 * ((4 * s + lg) ^ (col & (CH - 1)))) * 2;

    for (int sb = 0; sb < nsb; ++sb) {
        const int base = sb * SE;
        const int nsub = min(SE, n - base);
        if (!FW) stream_wait<D, NB>(0);
        if (fetcher) {
            // sub-chunk sb has landed once at most the later sub-chunks' fetches are outstanding
            const int later = min(NB - 2, nsb - 1 - sb);
            if (NB >= 4 && later >= 2) wait_vm<(NB >= 4 ? 8 * NI : 0)>();
            else if (NB >= 3 && later >= 1) wait_vm<(NB >= 3 ? 4 * NI : 0)>();
            else wait_vm<0>();
        }
        lds_barrier();  // sub-chunk sb is in LDS, and the buffer of sub-chunk sb - 1 is free again
        if (fetcher) {
            if (sb + NB - 1 < nsb) {
                const int nx = sb + NB - 1;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    stream_fetch<D>(Qb, qrow, s_ent + nx * SE, min(SE, n - nx * SE), sl[w], glog,
                                    s_ring + (nx % NB) * kSubRows * D, w);
            }
            continue;
        }
        if (!FW && sb + 1 < nsb)
            stream_fetch<D>(Qb, qrow, s_ent + (sb + 1) * SE, min(SE, n - (sb + 1) * SE), sl[0], glog,
                            s_ring + ((sb + 1) % NB) * kSubRows * D, wave);
            const unsigned char* cur = reinterpret_cast<const unsigned char*>(s_ring + (sb % NB) * kSubRows * D);
            // one 16-column tile per wave: entries wave * QT .. of the sub-chunk
            const int el = wave * QT + qi;
            const int ent = s_ent[base + (el < nsub ? el : nsub - 1)];
            const int64_t r = (uint32_t)ent >> 6;
            const int slot = ent & 63;
            const RowGeom gr{nb, nb - a.N_q + r};  // no reload of kv_len: a load here would wait on the stores
            const int vis = (int)(block_end(a, gr, k0) - k0);  // visible keys of this column (>= 1)

            const unsigned char* tb = cur + wave * (16 * D * 2);
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
            // scaled scores (base 2) in place, keys past the column's visible end dropped
            const bool any_masked = ballot(vis < C) != 0;
    #pragma unroll
            for (int rt = 0; rt < TPC; ++rt)
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = acc[rt][i] * scale;
                    acc[rt][i] = (!any_masked || rt * 16 + 4 * lg + i < vis) ? v : -INFINITY;
                }
            float m = -INFINITY;
    #pragma unroll
            for (int rt = 0; rt < TPC; ++rt)
    #pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, acc[rt][i]);
            m = max_xor16(m);
            m = max_xor32(m);
            // probabilities, packed straight into the P V operand as two bf16 terms, and their sum
            float l = 0.f;
            bf16x8 pbh[PS], pbl[PS];
    #pragma unroll
            for (int ps = 0; ps < PS; ++ps)
    #pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int rt = 2 * ps + hf;
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float pv = 0.f;
                        if (rt < TPC) {
                            pv = __builtin_amdgcn_exp2f(acc[rt < TPC ? rt : 0][i] - m);
                            l += pv;
                        }
                        const bf16 ph = to_bf16(pv);
                        pbh[ps][4 * hf + i] = ph;
                        pbl[ps][4 * hf + i] = to_bf16(pv - from_bf16(ph));
                    }
                }
            l = add_xor16(l);
            l = add_xor32(l);
            // O^T tile (d x column) = V^T P^T: A = transposed values (LDS), B = this lane's probabilities
            f32x4 o[DT];
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
            for (int ps = 0; ps < PS; ++ps)
    #pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int vd = dt * 16 + (lane & 15);
                    const bf16x8 va = *reinterpret_cast<const bf16x8*>(s_vt + vd * VLD + vt_swz<PS * 32>(vd, 32 * ps + 8 * lg));
                    o[dt] = mfma(va, pbh[ps], o[dt]);
                    o[dt] = mfma(va, pbl[ps], o[dt]);
                }
            // normalised row, scaled by 2^-e so that its largest |element| is below 1
            const float inv = 1.f / l;
            float amax = 0.f;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
                for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[dt][i]));
            amax = max_xor16(amax);
            amax = max_xor32(amax);
            const int e = amax * inv > 0.f ? __builtin_amdgcn_frexp_expf(amax * inv) : 0;
            const float sc = __builtin_ldexpf(inv, -e);
            if (el < nsub) {
                const int64_t row = ((bh * a.N_q + r) * a.K_top + slot) * G + head;
                f16* op = reinterpret_cast<f16*>(a.part_o) + row * D + 4 * lg;
    #pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    f16x4 w;
    #pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = (f16)(o[dt][i] * sc);
                    *reinterpret_cast<f16x4*>(op + 16 * dt) = w;
                }
                if (lg == 0) {
                    a.part_lse[2 * row] = m + __builtin_amdgcn_logf(l);
                    a.part_lse[2 * row + 1] = (float)e;
                }
            }

    }
}

// Waves loop over (sequence, row, KV head) items with a stride of the grid; a
// wave reads the next item's slot ids while it merges the current one. Each
// lane merges pairs (head, 8 d) of the G x D outputs, eight slots at a time
// with their loads in flight together and an online maximum across the groups.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnClArgs a)
{
    constexpr int CH = D / 8;
    const int lane = threadIdx.x & 63;
    const int64_t total = (int64_t)a.B * a.H_kv * a.N_q;
    const int64_t stride = (int64_t)gridDim.x * 4;
    const int G = a.G, K_top = a.K_top;
    const f16* po = reinterpret_cast<const f16*>(a.part_o);
    bf16* O = reinterpret_cast<bf16*>(a.O);
    int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    int blk_next = (item < total && lane < K_top) ? a.idx[item * K_top + lane] : -1;
    while (item < total) {
        const int blk = blk_next;
        const int64_t next = item + stride;
        blk_next = (next < total && lane < K_top) ? a.idx[next * K_top + lane] : -1;
        const int64_t r = item % a.N_q;
        const int64_t bh = item / a.N_q;
        const int h = (int)(bh % a.H_kv);
        const int b = (int)(bh / a.H_kv);
        const RowGeom g = row_geom(a, b, r);
        const int64_t prow = item * K_top;  // partial row of slot 0: items are ordered as the index rows
        bool vis = false;
        if (lane < K_top) {
            const int64_t k0 = (int64_t)blk * a.C;
            vis = blk >= 0 && k0 < g.nb && block_end(a, g, k0) > k0;
        }
        const uint64_t valid = ballot(vis);  // slots with visible keys (K_top <= 64)
        for (int pair = lane; pair - lane < G * CH; pair += 64) {
            const bool active = pair < G * CH;
            const int head = active ? pair / CH : 0, dc = active ? pair % CH : 0;
            float M = -INFINITY, L = 0.f;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < K_top; k0 += 8) {
                const uint64_t grp = (valid >> k0) & 0xffull;
                if (!grp) continue;
                float lse[8], ex[8];
                f16x8 x[8];
                const int kfirst = k0 + __builtin_ctzll(grp);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bool ok = (grp >> j) & 1;
                    const int64_t row = (prow + (ok ? k0 + j : kfirst)) * G + head;
                    lse[j] = ok ? a.part_lse[2 * row] : -INFINITY;
                    ex[j] = a.part_lse[2 * row + 1];
                    x[j] = *reinterpret_cast<const f16x8*>(po + row * D + 8 * dc);
                }
                float Mn = M;
#pragma unroll
                for (int j = 0; j < 8; ++j) Mn = fmaxf(Mn, lse[j]);
                const float f = __builtin_amdgcn_exp2f(M - Mn);  // M = -inf on the first group: f = 0
                L *= f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] *= f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float w = __builtin_amdgcn_exp2f(lse[j] - Mn);  // 0 for slots not in the group
                    const float ws = __builtin_ldexpf(w, (int)ex[j]);
                    L += w;
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] += ws * (float)x[j][i];
                }
                M = Mn;
            }
            if (!active) continue;
            const float inv = L > 0.f ? 1.f / L : 0.f;
            bf16x8 out;
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] = to_bf16(acc[i] * inv);
            *reinterpret_cast<bf16x8*>(O + (((int64_t)b * a.N_q + r) * a.H_q + (int64_t)h * G + head) * D + 8 * dc) = out;
            if (a.lse && dc == 0)
                a.lse[((int64_t)b * a.H_q + (int64_t)h * G + head) * a.N_q + r] =
                    L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
        }
        item = next;
    }
}

template <int D, int C>
static hipError_t launch_cl(const AttnClArgs& a, int64_t grid, hipStream_t s)
{
    constexpr int PS = (C + 31) / 32;
    constexpr int NB = kAttnFW ? kAttnNB : 2;
    const size_t lds = (size_t)NB * kSubRows * D * 2 + (size_t)D * (PS * 32 + 8) * 2 + (size_t)kLeafQC * 4;
    auto k = attn_cl_kernel<D, C, NB, kAttnFW>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kAttnFW ? 320 : 256), lds, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_cl_d(const AttnClArgs& a, int64_t grid, hipStream_t s)
{
    return a.C == 16 ? launch_cl<D, 16>(a, grid, s) : (a.C == 32 ? launch_cl<D, 32>(a, grid, s) : launch_cl<D, 64>(a, grid, s));
}

}  // namespace

AttnClLayout attn_cl_layout(int64_t B, int64_t N_q, int64_t N_alloc, int H_kv, int G, int d, int C, int K_top)
{
    AttnClLayout L;
    L.M_blk = (N_alloc + C - 1) / C;
    L.n_clusters = B * H_kv * L.M_blk;
    L.n_items = B * H_kv * N_q * K_top;
    L.max_chunks = L.n_items / kLeafQC + L.n_clusters + 1;
    L.n_sums = 2 * ((L.n_clusters + 1023) / 1024);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += (bytes + 255) & ~(size_t)255;
        return at;
    };
    L.counts = take((size_t)2 * L.n_clusters * 4);  // counts, then cursors
    L.offsets = take((size_t)(L.n_clusters + 1) * 4);
    L.chunk_off = take((size_t)(L.n_clusters + 1) * 4);
    L.chunk_cl = take((size_t)L.max_chunks * 4);
    L.block_sums = take((size_t)L.n_sums * 4);
    L.entries = take((size_t)L.n_items * 4);
    L.part_lse = take((size_t)L.n_items * G * 8);  // log-sum-exp and exponent per (row, slot, head)
    L.part_o = take((size_t)L.n_items * G * d * 2);
    L.bytes = o;
    return L;
}

hipError_t launch_attn_cluster(AttnClArgs& a, const AttnClLayout& L, char* ws, hipStream_t s)
{
    a.M_blk = L.M_blk;
    a.n_clusters = L.n_clusters;
    a.qc = kLeafQC;
    a.counts = reinterpret_cast<int32_t*>(ws + L.counts);
    a.cursor = a.counts + L.n_clusters;
    a.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    a.chunk_off = reinterpret_cast<int32_t*>(ws + L.chunk_off);
    a.chunk_cl = reinterpret_cast<int32_t*>(ws + L.chunk_cl);
    a.block_sums = reinterpret_cast<int32_t*>(ws + L.block_sums);
    a.entries = reinterpret_cast<int32_t*>(ws + L.entries);
    hipError_t e;
    if ((e = launch_fill_zero(a.counts, 2 * L.n_clusters, s)) != hipSuccess) return e;
    const dim3 cgrid((unsigned)((a.N_q + kClRowsPerBlock - 1) / kClRowsPerBlock), (unsigned)(a.B * a.H_kv));
    const size_t clds = L.M_blk <= kClLdsBins ? (size_t)2 * L.M_blk * 4 : 0;
    hipLaunchKernelGGL(attn_cluster_kernel, cgrid, dim3(kClThreads), clds, s, a, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_scan_chunks(a.counts, L.n_clusters, a.qc, a.block_sums, a.offsets, a.chunk_off, a.chunk_cl,
                                L.max_chunks, s)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(attn_cluster_kernel, cgrid, dim3(kClThreads), clds, s, a, 1);
    return hipGetLastError();
}

hipError_t launch_attn_clustered(AttnClArgs a, int d, char* ws, hipStream_t s)
{
    const AttnClLayout L = attn_cl_layout(a.B, a.N_q, a.N_alloc, a.H_kv, a.G, d, a.C, a.K_top);
    a.part_lse = reinterpret_cast<float*>(ws + L.part_lse);
    a.part_o = ws + L.part_o;
    hipError_t e;
    if ((e = launch_attn_cluster(a, L, ws, s)) != hipSuccess) return e;
    const int64_t grid = L.n_items / kLeafQC + L.n_clusters;  // bound on the chunks
    if ((e = (d == 64 ? launch_cl_d<64>(a, grid, s) : launch_cl_d<128>(a, grid, s))) != hipSuccess) return e;
    const int64_t items = (int64_t)a.B * a.H_kv * a.N_q;
    const int64_t cblocks = std::min<int64_t>((items + 3) / 4, 256 * 8);  // 8 workgroups per CU, grid-stride
    if (d == 64)
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((unsigned)cblocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(attn_combine_kernel<128>, dim3((unsigned)cblocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace pisa
