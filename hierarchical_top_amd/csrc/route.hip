// route.hip -- two-stage prefill routing around the stage-1 and stage-2
// kernels: cluster counting sort of (query, retained level-2 node) pairs and
// the final per-query Select_K ("Block Sparse Attention with Log-Linear
// Complexity", section 3.3, "Training/Prefill Stage 2" and the final
// Top-K kernel).
#include "pisa_device.hpp"
#include "pisa_internal.hpp"
#include "route_impl.hpp"

namespace pisa {

// per-dtype entry points (route_bf16.hip, route_f32.hip)
hipError_t route_query_bf16(const RouteArgs& a, int d, int mode, hipStream_t s);
hipError_t route_query_f32(const RouteArgs& a, int d, int mode, hipStream_t s);
hipError_t stage2_bf16(const Stage2Args& a, int d, int64_t grid, hipStream_t s);
hipError_t stage2_f32(const Stage2Args& a, int d, int64_t grid, hipStream_t s);

__global__ void fill_zero_kernel(int32_t* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// Exclusive scans of the cluster sizes and of their chunk counts (one block).
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts, int64_t n,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ chunk_off)
{
    __shared__ int s_w0[16], s_w1[16];
    __shared__ int s_carry[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) { s_carry[0] = 0; s_carry[1] = 0; }
    __syncthreads();
    for (int64_t base = 0; base < n; base += 1024) {
        const int64_t i = base + tid;
        const int cnt = i < n ? counts[i] : 0;
        const int nch = (cnt + kChunkQ - 1) / kChunkQ;
        int x0 = cnt, x1 = nch;
        for (int o = 1; o < 64; o <<= 1) {
            const int y0 = __shfl_up(x0, o, 64), y1 = __shfl_up(x1, o, 64);
            if (lane >= o) { x0 += y0; x1 += y1; }
        }
        if (lane == 63) { s_w0[wave] = x0; s_w1[wave] = x1; }
        __syncthreads();
        int p0 = s_carry[0], p1 = s_carry[1];
        for (int w = 0; w < wave; ++w) { p0 += s_w0[w]; p1 += s_w1[w]; }
        if (i < n) {
            offsets[i] = p0 + x0 - cnt;
            chunk_off[i] = p1 + x1 - nch;
        }
        __syncthreads();
        if (tid == 1023) { s_carry[0] = p0 + x0; s_carry[1] = p1 + x1; }
        __syncthreads();
    }
    if (tid == 0) {
        offsets[n] = s_carry[0];
        chunk_off[n] = s_carry[1];
    }
}

// Cluster membership: every (query, kept level-2 node) pair that has a leaf
// to score is appended to its node's cluster as (t << 6) | slot. The order
// inside a cluster does not affect any result. Block (tile of 256 positions,
// sequence x KV head): the pairs are counted per node in LDS, each node's range
// is reserved with one global atomic per block, and positions inside it are
// handed out from LDS (nodes shared by every query -- the first block's and the
// current path's ancestors -- would otherwise take one global atomic per query).
__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a)
{
    extern __shared__ int s_mem[];
    const int64_t bh = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = t < a.N;
    const int64_t i = bh * a.N + (live ? t : 0);
    const int64_t meta = live ? a.meta[i] : 0;
    const uint64_t mask = (meta & 1) ? (uint64_t)meta >> 1 : 0;
    const int32_t* base_off = a.offsets + bh * a.M2;
    int32_t* cur = a.cursor + bh * a.M2;
    if (a.M2 <= kLdsBins) {
        int* s_cnt = s_mem;
        int* s_pos = s_mem + a.M2;
        for (int64_t k = threadIdx.x; k < a.M2; k += 256) s_cnt[k] = 0;
        __syncthreads();
        for (int k = 0; k < a.K_top; ++k)
            if ((mask >> k) & 1) {
                const int P = a.kept2[i * a.K_top + k];
                lds_add(&s_cnt[P], P, s_cnt);
            }
        __syncthreads();
        for (int64_t k = threadIdx.x; k < a.M2; k += 256) {
            const int v = s_cnt[k];
            s_pos[k] = v ? base_off[k] + atomicAdd(&cur[k], v) : 0;
        }
        __syncthreads();
        for (int k = 0; k < a.K_top; ++k)
            if ((mask >> k) & 1) {
                const int P = a.kept2[i * a.K_top + k];
                const int pos = lds_add(&s_pos[P], P, s_pos);
                a.entries[pos] = (int32_t)((t << 6) | k);
            }
    } else {
        for (int k = 0; k < a.K_top; ++k) {
            if (!((mask >> k) & 1)) continue;
            const int P = a.kept2[i * a.K_top + k];
            a.entries[base_off[P] + atomicAdd(&cur[P], 1)] = (int32_t)((t << 6) | k);
        }
    }
}

// Final Select_K per (query, KV head): forced leaves first, then the best
// K_top - |forced| scored leaves (score desc, id asc); written ascending.
template <int KMAX>
__global__ __launch_bounds__(256) void final_kernel(FinalArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)a.B * a.H * a.N) return;
    const int64_t t = i % a.N;
    const int64_t meta = a.meta[i];
    const bool scored = meta & 1;
    const int32_t* kept = a.kept2 + i * a.K_top;
    const int64_t c = t >> a.c_log2;
    const int64_t M1 = (a.N + a.C - 1) >> a.c_log2;
    const int ucols = a.g * a.K_top;

    int ids[KMAX];
    float val[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) { ids[j] = 0x7fffffff; val[j] = -INFINITY; }
    auto put = [&](int x, float v) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (x < ids[j]) {
                const int ti = ids[j]; ids[j] = x; x = ti;
                const float tv = val[j]; val[j] = v; v = tv;
            }
        }
    };
    if (!scored) {
        for (int k = 0; k < a.K_top; ++k) {
            const int p = kept[k];
            if (p < 0) continue;
            for (int cc = 0; cc < a.g; ++cc) {
                const int64_t leaf = (int64_t)p * a.g + cc;
                if (leaf >= M1 || (a.causal && (leaf << a.c_log2) > t)) break;
                put((int)leaf, INFINITY);
            }
        }
    } else {
        int nF = 0;
        if (a.causal) {
            put(0, INFINITY);
            nF = 1;
            if (c != 0) { put((int)c, INFINITY); ++nF; }
            if (c - 1 >= 1) { put((int)(c - 1), INFINITY); ++nF; }
        }
        const int Rk = a.K_top - nF;
        float bu[KMAX];
        int bi[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) { bu[j] = -INFINITY; bi[j] = 0x7fffffff; }
        for (int k = 0; k < a.K_top; ++k) {
            const int p = kept[k];
            if (p < 0) continue;
            for (int cc = 0; cc < a.g; ++cc) {
                const int64_t leaf = (int64_t)p * a.g + cc;
                if (leaf >= M1 || (a.causal && (leaf << a.c_log2) > t)) break;
                if (a.causal && (leaf == 0 || leaf == c || leaf == c - 1)) continue;
                float xu = a.u[i * ucols + k * a.g + cc];
                int xi = (int)leaf;
#pragma unroll
                for (int j = 0; j < KMAX; ++j) {
                    if (j < Rk && before(xu, xi, bu[j], bi[j])) {
                        const float tu = bu[j]; bu[j] = xu; xu = tu;
                        const int ti = bi[j]; bi[j] = xi; xi = ti;
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < Rk && bi[j] != 0x7fffffff) put(bi[j], bu[j]);
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < a.K_top) {
            const bool ok = ids[j] != 0x7fffffff;
            a.idx[i * a.K_top + j] = ok ? ids[j] : -1;
            if (a.score) a.score[i * a.K_top + j] = ok ? val[j] : -INFINITY;
        }
    }
}

hipError_t launch_route_query(const RouteArgs& a, int dtype, int d, int mode, hipStream_t s)
{
    return dtype == 0 ? route_query_f32(a, d, mode, s) : route_query_bf16(a, d, mode, s);
}

hipError_t launch_two_stage(const RouteArgs& r, const Stage2Args& s2, const FinalArgs& f, const ScatterArgs& sc,
                            int32_t* zero_base, int64_t zero_count, int dtype, int d, hipStream_t s)
{
    hipError_t err;
    // cluster sizes are counted with atomics by the stage-1 kernel: clear them first
    stage_mark(PISA_STAGE_UPPER, false, s);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, s, zero_base, zero_count);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = launch_route_query(r, dtype, d, MODE_STAGE1, s)) != hipSuccess) return err;
    stage_mark(PISA_STAGE_UPPER, true, s);
    stage_mark(PISA_STAGE_CLUSTER, false, s);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, r.counts, s2.n_clusters,
                       const_cast<int32_t*>(s2.offsets), const_cast<int32_t*>(s2.chunk_off));
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t items = (int64_t)f.B * f.H * f.N;
    const unsigned gi = (unsigned)((items + 255) / 256);
    {
        const dim3 grid((unsigned)((f.N + 255) / 256), (unsigned)(f.B * f.H));
        const size_t lds = sc.M2 <= kLdsBins ? (size_t)2 * sc.M2 * 4 : 0;
        hipLaunchKernelGGL(scatter_kernel, grid, dim3(256), lds, s, sc);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    stage_mark(PISA_STAGE_CLUSTER, true, s);
    const int64_t max_chunks = (items * f.K_top + kChunkQ - 1) / kChunkQ + s2.n_clusters;
    stage_mark(PISA_STAGE_LEAF, false, s);
    err = dtype == 0 ? stage2_f32(s2, d, max_chunks, s) : stage2_bf16(s2, d, max_chunks, s);
    if (err != hipSuccess) return err;
    stage_mark(PISA_STAGE_LEAF, true, s);
    stage_mark(PISA_STAGE_FINAL, false, s);
    if (f.K_top <= 8)
        hipLaunchKernelGGL(final_kernel<8>, dim3(gi), dim3(256), 0, s, f);
    else if (f.K_top <= 16)
        hipLaunchKernelGGL(final_kernel<16>, dim3(gi), dim3(256), 0, s, f);
    else if (f.K_top <= 32)
        hipLaunchKernelGGL(final_kernel<32>, dim3(gi), dim3(256), 0, s, f);
    else
        hipLaunchKernelGGL(final_kernel<64>, dim3(gi), dim3(256), 0, s, f);
    stage_mark(PISA_STAGE_FINAL, true, s);
    return hipGetLastError();
}

}  // namespace pisa
