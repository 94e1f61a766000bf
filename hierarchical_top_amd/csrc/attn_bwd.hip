// attn_bwd.hip -- backward of block-sparse attention with fixed block indices
// ("Block Sparse Attention with Log-Linear Complexity", section 3.1 eq 6;
// section 3.3: in training the gradients flow through attention on the
// selected entries, the selection itself is not differentiated).
//
// For a query row and head with selected token set T, z_j = q.k_j / sqrt(d),
// p = softmax(z), o = sum_j p_j v_j, and an upstream gradient dO:
//   dv_j += p_j dO,  dp_j = dO.v_j,  dz_j = p_j (dp_j - D),  D = sum_j p_j dp_j = dO.o,
//   dq += sum_j dz_j k_j / sqrt(d),  dk_j += dz_j q / sqrt(d).
// Given the forward's log-normaliser (p_j = exp(z_j - lse)) and D, every term
// of a (row, selected block) pair is local to that pair, so the pairs are
// grouped by block exactly as in the clustered forward:
//   1. dsum_kernel: D = sum over d of dO * O per (row, head);
//   2. the forward's clustering: entries (row << 6) | slot per (sequence, KV
//      head, block);
//   3. attn_bwd_kernel: a workgroup takes a chunk of up to 256 entries of one
//      block. Wave w owns key tile w % (C/16) (16 keys, their K and V rows in
//      registers) and, per iteration, column tile w / (C/16) of 16 (entry,
//      head) columns. S = Q K^T and dP = dO V^T come out of the 16x16x32 MFMA
//      with one key per lane and four columns per lane, which is the A-operand
//      layout of the 16x16x16 MFMA over those columns: dV += P^T dO and
//      dK += dS^T Q accumulate in registers for the whole chunk (P and dS as two
//      bf16 terms, dO and Q transposed in LDS) and are added to global memory
//      once per chunk. dQ = dS K contracts over the keys of all waves: dS goes
//      to LDS and every wave computes some (column tile, d tile) products
//      against K^T in LDS, stored as the (row, slot, head)'s fp32 partial dQ;
//   4. dq_combine_kernel: one wave per (sequence, row, KV head) sums its
//      partials in slot order into dQ (rows with no visible key get 0).
// dK and dV are cleared first and take each chunk's part with fp32 atomics,
// so their last bits vary from run to run; dQ is deterministic. (Atomics for dQ
// too -- K_top per element, scattered over rows -- cost several times the
// whole kernel.)
#include <algorithm>

#include "attn_bwd.hpp"
#include "pisa_device.hpp"

namespace pisa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// D += A * B for one 16x16x16 bf16 tile: lane l holds A[l%16][4*(l/16) + j] and
// B[4*(l/16) + j][l%16], j = 0..3; D as for the 16x16x32 tile.
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}

__global__ __launch_bounds__(256) void fill_zero_f32_kernel(float* p, int64_t n)
{
    const int64_t n4 = n >> 2;
    f32x4* p4 = reinterpret_cast<f32x4*>(p);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
        p4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0.f;
}

// D[b][hq][r] = sum_e dO[b][r][hq][e] * O[b][r][hq][e] (fp32), D / 8 lanes per (row, head).
template <int D>
__global__ __launch_bounds__(256) void dsum_kernel(AttnBwdArgs a)
{
    constexpr int L = D / 8;
    const int64_t total = (int64_t)a.c.B * a.c.N_q * a.c.H_q;
    const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) / L;
    const int part = threadIdx.x % L;
    const bool ok = item < total;
    const int64_t it = ok ? item : 0;
    const bf16* o = reinterpret_cast<const bf16*>(a.O) + it * D + 8 * part;
    const bf16* g = reinterpret_cast<const bf16*>(a.dO) + it * D + 8 * part;
    const bf16x8 ov = load8h(o), gv = load8h(g);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += from_bf16(ov[j]) * from_bf16(gv[j]);
#pragma unroll
    for (int m = 1; m < L; m <<= 1) s += shfl_xor(s, m);
    if (ok && part == 0) {
        const int64_t hq = it % a.c.H_q, br = it / a.c.H_q;
        const int64_t r = br % a.c.N_q, b = br / a.c.N_q;
        a.dsum[(b * a.c.H_q + hq) * a.c.N_q + r] = s;
    }
}

// Column position of (d, column) in the transposed q / dO tiles: columns are XOR-swizzled in
// groups of four by d / 8, so that the 16-bit stores of the eight d of a 16-byte piece (one
// piece per thread, consecutive threads on consecutive d / 8) fall in different banks while a
// lane's four consecutive columns of one d stay one 8-byte read. Needs 32 | columns.
__device__ __forceinline__ int tcol(int d, int col) { return col ^ (((d >> 3) & 7) << 2); }

// Key position of a row of K^T or dS in LDS: groups of eight keys XOR-swizzled by a row tag f,
// so that 16-bit stores to rows that share banks spread out, while the eight keys an MFMA
// operand reads (positions 8 m .. 8 m + 7 of the natural order) stay one 16-byte load.
__device__ __forceinline__ int swz8(int pos, int f) { return pos ^ (f << 3); }

template <int D, int C>
struct BwdGeom {
    static constexpr int KS = D / 32;          // k-steps of S = Q K^T and dP = dO V^T
    static constexpr int DT = D / 16;          // d tiles
    static constexpr int TPC = C / 16;         // key tiles
    static constexpr int NCT = 4 / TPC;        // waves per key tile
    static constexpr int CPW = C == 64 ? 2 : 1;  // column tiles per wave and iteration
    static constexpr int PS = (C + 31) / 32;   // 32-key steps of dQ = dS K
    static constexpr int NCOL = 16 * NCT * CPW;  // columns per iteration
    static constexpr int LDW = D + 8;          // [column][d] row stride (bf16)
    static constexpr int TW = NCOL + 4;        // [d][column] row stride (bf16)
    static constexpr int KW = PS * 32 + 8;     // [d][key] and [column][key] row strides (bf16)
    static constexpr int CH = D / 8;           // 16-byte pieces of a row
    static constexpr int NPT = (NCOL * CH + 255) / 256;  // pieces per thread and tensor per iteration
    static constexpr int DQT = (NCOL / 16) * DT / 4;  // dQ tiles per wave per iteration
    // loads issued two iterations ahead (two register sets) for d = 64; at d = 128 the second
    // set does not fit in registers next to the accumulators
    static constexpr bool PD2 = D == 64;
    // LDS: q, dO [NCOL][LDW]; q^T, dO^T [D][TW]; K^T [D][KW]; dS hi, lo [NCOL][KW]; column metadata; entries
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_DO = OFF_Q + (size_t)NCOL * LDW * 2;
    static constexpr size_t OFF_QT = OFF_DO + (size_t)NCOL * LDW * 2;
    static constexpr size_t OFF_DOT = OFF_QT + (size_t)D * TW * 2;
    static constexpr size_t OFF_KT = OFF_DOT + (size_t)D * TW * 2;
    static constexpr size_t OFF_DSH = OFF_KT + (size_t)D * KW * 2;
    static constexpr size_t OFF_DSL = OFF_DSH + (size_t)NCOL * KW * 2;
    static constexpr size_t OFF_META = (OFF_DSL + (size_t)NCOL * KW * 2 + 15) & ~(size_t)15;
    static constexpr size_t OFF_ENT = OFF_META + (size_t)NCOL * 16;  // lse2, dsum (float), vis (int), dQ row (int)
    static constexpr size_t BYTES = OFF_ENT + (size_t)kLeafQC * 4;
    static_assert(TPC * NCT == 4, "four waves cover the key tiles times the column tiles");
    static_assert(NCOL % 32 == 0, "the transposed tiles' column swizzle spans 32 columns");
    static_assert(((NCOL / 16) * DT) % 4 == 0, "dQ tiles spread evenly over the waves");
};

template <int D, int C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_kernel(AttnBwdArgs A)
{
    using Gm = BwdGeom<D, C>;
    constexpr int KS = Gm::KS, DT = Gm::DT, TPC = Gm::TPC, NCT = Gm::NCT, CPW = Gm::CPW, PS = Gm::PS;
    constexpr int NCOL = Gm::NCOL;
    constexpr int LDW = Gm::LDW, TW = Gm::TW, KW = Gm::KW, CH = Gm::CH, NPT = Gm::NPT;
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    bf16* s_q = reinterpret_cast<bf16*>(s_raw + Gm::OFF_Q);
    bf16* s_do = reinterpret_cast<bf16*>(s_raw + Gm::OFF_DO);
    bf16* s_qt = reinterpret_cast<bf16*>(s_raw + Gm::OFF_QT);
    bf16* s_dot = reinterpret_cast<bf16*>(s_raw + Gm::OFF_DOT);
    bf16* s_kt = reinterpret_cast<bf16*>(s_raw + Gm::OFF_KT);
    bf16* s_dsh = reinterpret_cast<bf16*>(s_raw + Gm::OFF_DSH);
    bf16* s_dsl = reinterpret_cast<bf16*>(s_raw + Gm::OFF_DSL);
    float* s_lse2 = reinterpret_cast<float*>(s_raw + Gm::OFF_META);
    float* s_dsum = s_lse2 + NCOL;
    int* s_vis = reinterpret_cast<int*>(s_dsum + NCOL);
    int* s_dqrow = s_vis + NCOL;  // partial row ((bh * N_q + r) * K_top + slot) * G + head, or -1 (padding)
    int* s_ent = reinterpret_cast<int*>(s_raw + Gm::OFF_ENT);

    const AttnClArgs& a = A.c;
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
    const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kt = wave % TPC, ct = wave / TPC;
    const int G = a.G;
    const int epi = NCOL / G;  // entries per iteration
    const int n_it = (n + epi - 1) / epi;
    int64_t nb = a.kv_len ? a.kv_len[b] : a.N_kv;
    nb = nb < 0 ? 0 : (nb > a.N_alloc ? a.N_alloc : nb);
    const int64_t k0 = blk * C;
    const int kexist = (int)((k0 + C < nb ? k0 + C : nb) - k0);  // >= 1: the block holds a visible key
    const int64_t kvstride = (int64_t)a.H_kv * D;
    const bf16* Kb = reinterpret_cast<const bf16*>(a.K) + ((int64_t)b * a.N_alloc + k0) * kvstride + (int64_t)h * D;
    const bf16* Vb = reinterpret_cast<const bf16*>(a.V) + ((int64_t)b * a.N_alloc + k0) * kvstride + (int64_t)h * D;
    const bf16* Qg = reinterpret_cast<const bf16*>(a.Q);
    const bf16* dOg = reinterpret_cast<const bf16*>(A.dO);

    for (int i = tid; i < n; i += 256) s_ent[i] = a.entries[e0 + i];
    // dS padding keys (C = 16: keys 16..31 of the single 32-key step) stay zero
    for (int i = tid; i < 2 * NCOL * KW; i += 256) s_dsh[i] = to_bf16(0.f);  // s_dsl follows s_dsh
    // K^T in LDS for dQ = dS K: [d][key], keys past the block's end (and the padding) zero
    for (int p = tid; p < PS * 32 * CH; p += 256) {
        const int key = p / CH, dc = p % CH;
        const bool ok = key < kexist;
        const bf16x8 v = load8h(Kb + (ok ? (int64_t)key * kvstride : 0) + 8 * dc);
#pragma unroll
        for (int j = 0; j < 8; ++j) s_kt[(8 * dc + j) * KW + swz8(key, dc & (PS * 4 - 1))] = ok ? v[j] : to_bf16(0.f);
    }
    // this wave's keys as the B operand of S = Q K^T and dP = dO V^T: lane (key, 8 d)
    bf16x8 bK[KS], bV[KS];
    {
        const int key = kt * 16 + (lane & 15);
        const bool ok = key < kexist;
        const int64_t ro = (ok ? (int64_t)key * kvstride : 0) + 8 * lg;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 kv = load8h(Kb + ro + 32 * s), vv = load8h(Vb + ro + 32 * s);
            bK[s] = ok ? kv : zero8h();
            bV[s] = ok ? vv : zero8h();
        }
    }
    __syncthreads();  // entries in LDS

    // global -> registers for one iteration: q and dO pieces (column, 8 d), and per column its
    // metadata; at d = 64 two sets, so that an iteration's loads are issued two iterations
    // before use (one iteration before at d = 128)
    struct Regs {
        bf16x8 q[NPT], o[NPT];
        float lse2, dsum;
        int vis, row;
    };
    auto load_it = [&](int it, Regs& R) {
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int p = tid + 256 * j;
            const int col = (p < NCOL * CH ? p : 0) / CH, dc = p % CH;
            const int el = it * epi + col / G, head = col % G;
            const int ent = s_ent[el < n ? el : n - 1];
            const int64_t r = (uint32_t)ent >> 6;
            const int64_t off = (((int64_t)b * a.N_q + r) * a.H_q + (int64_t)h * G + head) * D + 8 * dc;
            R.q[j] = load8h(Qg + off);
            R.o[j] = load8h(dOg + off);
        }
        R.lse2 = INFINITY;  // padding column: p = 2^-inf = 0
        R.dsum = 0.f;
        R.vis = 0;
        R.row = -1;
        if (tid < NCOL) {
            const int col = tid;
            const int el = it * epi + col / G, head = col % G;
            if (el < n) {
                const int ent = s_ent[el];
                const int64_t r = (uint32_t)ent >> 6;
                const int64_t li = ((int64_t)b * a.H_q + (int64_t)h * G + head) * a.N_q + r;
                R.lse2 = A.lse[li] * kLog2e;
                R.dsum = A.dsum[li];
                int64_t kend = k0 + C < nb ? k0 + C : nb;
                const int64_t pos = nb - a.N_q + r;
                if (a.causal && kend > pos + 1) kend = pos + 1;
                R.vis = (int)(kend - k0);
                R.row = (int)(((bh * a.N_q + r) * a.K_top + (ent & 63)) * G + head);
            }
        }
    };
    auto store_it = [&](const Regs& R) {
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int p = tid + 256 * j;
            if (p < NCOL * CH) {
                const int col = p / CH, dc = p % CH;
                *reinterpret_cast<bf16x8*>(s_q + col * LDW + 8 * dc) = R.q[j];
                *reinterpret_cast<bf16x8*>(s_do + col * LDW + 8 * dc) = R.o[j];
                const int tc = tcol(8 * dc, col);  // the same for the eight d of the piece
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    s_qt[(8 * dc + k) * TW + tc] = R.q[j][k];
                    s_dot[(8 * dc + k) * TW + tc] = R.o[j][k];
                }
            }
        }
        if (tid < NCOL) {
            s_lse2[tid] = R.lse2;
            s_dsum[tid] = R.dsum;
            s_vis[tid] = R.vis;
            s_dqrow[tid] = R.row;
        }
    };

    const float sc2 = kLog2e * rsqrtf((float)D);  // logits in base 2
    const float inv_sqrt_d = rsqrtf((float)D);
    const int key = kt * 16 + (lane & 15);
    f32x4 accV[DT], accK[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        accV[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        accK[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // one iteration over the columns in LDS: this wave's CPW column tiles against its key tile
    auto compute = [&]() {
#pragma unroll 1
        for (int j = 0; j < CPW; ++j) {
            const int cb = 16 * (ct + NCT * j);
            // S and dP for 16 columns x this wave's 16 keys: lane = key, columns cb + 4 lg + i
            f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f}, pacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 aq = *reinterpret_cast<const bf16x8*>(s_q + (cb + (lane & 15)) * LDW + 32 * s + 8 * lg);
                const bf16x8 ad = *reinterpret_cast<const bf16x8*>(s_do + (cb + (lane & 15)) * LDW + 32 * s + 8 * lg);
                sacc = mfma(aq, bK[s], sacc);
                pacc = mfma(ad, bV[s], pacc);
            }
            bf16x4 ph, pl, dh, dl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = cb + 4 * lg + i;
                const float p = key < s_vis[c] ? __builtin_amdgcn_exp2f(sacc[i] * sc2 - s_lse2[c]) : 0.f;
                const float ds = p * (pacc[i] - s_dsum[c]);
                ph[i] = to_bf16(p);
                pl[i] = to_bf16(p - from_bf16(ph[i]));
                dh[i] = to_bf16(ds);
                dl[i] = to_bf16(ds - from_bf16(dh[i]));
            }
            // dV += P^T dO and dK += dS^T Q over these 16 columns (lane = d, keys 4 lg + i)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = dt * 16 + (lane & 15);
                const bf16x4 bdo = *reinterpret_cast<const bf16x4*>(s_dot + d * TW + tcol(d, cb + 4 * lg));
                const bf16x4 bq = *reinterpret_cast<const bf16x4*>(s_qt + d * TW + tcol(d, cb + 4 * lg));
                accV[dt] = mfma16(ph, bdo, accV[dt]);
                accV[dt] = mfma16(pl, bdo, accV[dt]);
                accK[dt] = mfma16(dh, bq, accK[dt]);
                accK[dt] = mfma16(dl, bq, accK[dt]);
            }
            // dS to LDS as [column][key] for dQ = dS K
#pragma unroll
            for (int i = 0; i < 4; ++i) {  // row cb + 4 lg + i: tag ((row / 4) & 3) = lg
                s_dsh[(cb + 4 * lg + i) * KW + swz8(key, lg)] = dh[i];
                s_dsl[(cb + 4 * lg + i) * KW + swz8(key, lg)] = dl[i];
            }
        }
        __syncthreads();
        // dQ^T tiles (16 d x 16 columns) = K^T dS^T over the block's keys; lane = column, d 4 lg + i
#pragma unroll 1
        for (int k = 0; k < Gm::DQT; ++k) {
            const int ti = wave + 4 * k;
            const int ctq = ti / DT, dt = ti % DT;
            f32x4 q = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ps = 0; ps < PS; ++ps) {
                const int dk = dt * 16 + (lane & 15), ka = swz8(32 * ps + 8 * lg, (dk >> 3) & (PS * 4 - 1));
                const int kb = swz8(32 * ps + 8 * lg, ((lane & 15) >> 2) & 3);
                const bf16x8 ak = *reinterpret_cast<const bf16x8*>(s_kt + dk * KW + ka);
                const bf16x8 bh_ = *reinterpret_cast<const bf16x8*>(s_dsh + (16 * ctq + (lane & 15)) * KW + kb);
                const bf16x8 bl_ = *reinterpret_cast<const bf16x8*>(s_dsl + (16 * ctq + (lane & 15)) * KW + kb);
                q = mfma(ak, bh_, q);
                q = mfma(ak, bl_, q);
            }
            const int row = s_dqrow[16 * ctq + (lane & 15)];
            if (row >= 0)
                *reinterpret_cast<f32x4*>(A.part_dq + (int64_t)row * D + dt * 16 + 4 * lg) = q * inv_sqrt_d;
        }
        __syncthreads();  // every wave is done with this iteration's LDS
    };

    Regs RA, RB;
    load_it(0, RA);
    store_it(RA);
    __syncthreads();
    if constexpr (!Gm::PD2) {  // one iteration ahead: the next iteration's loads fly during this one
        for (int it = 0; it < n_it; ++it) {
            if (it + 1 < n_it) load_it(it + 1, RA);
            compute();
            if (it + 1 < n_it) {
                store_it(RA);
                __syncthreads();
            }
        }
    } else {
    if (n_it > 1) load_it(1, RB);
    for (int it = 0; it < n_it; it += 2) {
        if (it + 2 < n_it) load_it(it + 2, RA);  // RA's data is in LDS already
        compute();
        if (it + 1 >= n_it) break;
        store_it(RB);
        __syncthreads();
        if (it + 3 < n_it) load_it(it + 3, RB);
        compute();
        if (it + 2 >= n_it) break;
        store_it(RA);
        __syncthreads();
    }
    }
    // this chunk's part of dK and dV for the wave's keys: lane = d (lane & 15) + 16 dt, keys 4 lg + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = kt * 16 + 4 * lg + i;
        if (k < kexist) {
            const int64_t ro = (((int64_t)b * a.N_alloc + k0 + k) * a.H_kv + h) * D + (lane & 15);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                unsafeAtomicAdd(A.dV + ro + 16 * dt, accV[dt][i]);
                unsafeAtomicAdd(A.dK + ro + 16 * dt, accK[dt][i] * inv_sqrt_d);
            }
        }
    }
}

// Waves loop over (sequence, row, KV head) items with a stride of the grid; lanes
// take (head, 4 d) pieces of the G x D outputs and add the partials of the slots
// whose block holds a visible key, in slot order.
template <int D>
__global__ __launch_bounds__(256) void dq_combine_kernel(AttnBwdArgs A)
{
    constexpr int CH4 = D / 4;
    const AttnClArgs& a = A.c;
    const int lane = threadIdx.x & 63;
    const int64_t total = (int64_t)a.B * a.H_kv * a.N_q;
    const int64_t stride = (int64_t)gridDim.x * 4;
    const int G = a.G, K_top = a.K_top;
    int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    int blk_next = (item < total && lane < K_top) ? a.idx[item * K_top + lane] : -1;
    for (; item < total; item += stride) {
        const int blk = blk_next;  // this item's slot ids; the next item's are read during the merge
        const int64_t next = item + stride;
        blk_next = (next < total && lane < K_top) ? a.idx[next * K_top + lane] : -1;
        const int64_t r = item % a.N_q;
        const int64_t bh = item / a.N_q;
        const int h = (int)(bh % a.H_kv);
        const int b = (int)(bh / a.H_kv);
        int64_t nb = a.kv_len ? a.kv_len[b] : a.N_kv;
        nb = nb < 0 ? 0 : (nb > a.N_alloc ? a.N_alloc : nb);
        const int64_t pos = nb - a.N_q + r;
        bool vis = false;
        if (lane < K_top) {
            const int64_t k0 = (int64_t)blk * a.C;
            int64_t kend = k0 + a.C < nb ? k0 + a.C : nb;
            if (a.causal && kend > pos + 1) kend = pos + 1;
            vis = blk >= 0 && k0 < nb && kend > k0;
        }
        const uint64_t valid = ballot(vis);
        const int64_t prow = item * K_top;  // partial row of slot 0
        for (int pc = lane; pc < G * CH4; pc += 64) {
            const int head = pc / CH4, dc = pc % CH4;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < K_top; s0 += 8) {  // eight slots' loads in flight together, added in slot order
                const uint32_t grp = (uint32_t)(valid >> s0) & 0xffu;
                if (!grp) continue;
                const int sfirst = s0 + __builtin_ctz(grp);
                f32x4 x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int slot = (grp >> j) & 1 ? s0 + j : sfirst;
                    x[j] = *reinterpret_cast<const f32x4*>(A.part_dq + ((prow + slot) * G + head) * D + 4 * dc);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if ((grp >> j) & 1) acc += x[j];
            }
            *reinterpret_cast<f32x4*>(A.dQ + (((int64_t)b * a.N_q + r) * a.H_q + (int64_t)h * G + head) * D + 4 * dc) =
                acc;
        }
    }
}

template <int D, int C>
static hipError_t launch_bwd(const AttnBwdArgs& a, int64_t grid, hipStream_t s)
{
    const size_t lds = BwdGeom<D, C>::BYTES;
    auto k = attn_bwd_kernel<D, C>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(256), lds, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const AttnBwdArgs& a, int64_t grid, hipStream_t s)
{
    return a.c.C == 16 ? launch_bwd<D, 16>(a, grid, s)
                       : (a.c.C == 32 ? launch_bwd<D, 32>(a, grid, s) : launch_bwd<D, 64>(a, grid, s));
}

static hipError_t fill_zero_f32(float* p, int64_t n, hipStream_t s)
{
    const int64_t blocks = std::min<int64_t>((n / 4 + 255) / 256 + 1, 256 * 8);
    hipLaunchKernelGGL(fill_zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace

AttnBwdLayout attn_bwd_layout(int64_t B, int64_t N_q, int64_t N_alloc, int H_q, int H_kv, int d, int C, int K_top)
{
    AttnBwdLayout L;
    L.cl = attn_cl_layout(B, N_q, N_alloc, H_kv, H_q / H_kv, d, C, K_top);
    L.dsum = L.cl.part_lse;  // the forward's partial sections are not used here
    L.part_dq = L.dsum + (((size_t)B * H_q * N_q * 4 + 255) & ~(size_t)255);
    L.bytes = L.part_dq + (size_t)L.cl.n_items * (H_q / H_kv) * d * 4;
    return L;
}

hipError_t launch_attn_bwd(AttnBwdArgs a, int d, char* ws, hipStream_t s)
{
    const AttnBwdLayout L = attn_bwd_layout(a.c.B, a.c.N_q, a.c.N_alloc, a.c.H_q, a.c.H_kv, d, a.c.C, a.c.K_top);
    a.dsum = reinterpret_cast<float*>(ws + L.dsum);
    a.part_dq = reinterpret_cast<float*>(ws + L.part_dq);
    hipError_t e;
    const int64_t nkv = (int64_t)a.c.B * a.c.N_alloc * a.c.H_kv * d;
    if ((e = fill_zero_f32(a.dK, nkv, s)) != hipSuccess) return e;
    if ((e = fill_zero_f32(a.dV, nkv, s)) != hipSuccess) return e;
    {
        const int64_t rows = (int64_t)a.c.B * a.c.N_q * a.c.H_q;
        const int per = 256 / (d / 8);  // (row, head) items per workgroup
        const unsigned grid = (unsigned)((rows + per - 1) / per);
        if (d == 64) hipLaunchKernelGGL(dsum_kernel<64>, dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL(dsum_kernel<128>, dim3(grid), dim3(256), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = launch_attn_cluster(a.c, L.cl, ws, s)) != hipSuccess) return e;
    const int64_t grid = L.cl.n_items / kLeafQC + L.cl.n_clusters;  // bound on the chunks
    if ((e = (d == 64 ? launch_bwd_d<64>(a, grid, s) : launch_bwd_d<128>(a, grid, s))) != hipSuccess) return e;
    const int64_t items = (int64_t)a.c.B * a.c.H_kv * a.c.N_q;
    const int64_t cblocks = std::min<int64_t>((items + 3) / 4, 256 * 8);  // grid-stride, 8 workgroups per CU
    if (d == 64) hipLaunchKernelGGL(dq_combine_kernel<64>, dim3((unsigned)cblocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dq_combine_kernel<128>, dim3((unsigned)cblocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace pisa
