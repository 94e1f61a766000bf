// stream.hpp -- streaming of gathered query rows through an LDS ring, shared
// by the clustered router kernels (levels_impl.hpp) and the clustered
// block-sparse attention (attn_cl.hip). A chunk's entries are (row << 6) | slot;
// every entry brings the G query heads of its row (G * D bf16, contiguous).
#pragma once
#include "pisa_device.hpp"
#include "pisa_internal.hpp"

namespace pisa {

// Streaming of a chunk's query rows through LDS (leaf_kernel, upper_kernel).
// Sub-chunk k holds LDS rows r = entry * G + head for its kSubRows / G
// entries; row r's 16-byte pieces are XOR-swizzled by (r mod D / 8), so the 16
// columns of a B operand read distinct bank groups. Rows are fetched with
// global_load_lds (lane l writes 16 bytes at the wave-uniform base + 16 * l),
// each wave issuing exactly NI instructions per sub-chunk, which lets a wave
// wait for one sub-chunk with an exact vmcnt while later ones are in flight
// (loads complete in order; the loop issues no other memory instruction that
// counts there).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) left at their maxima
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D>
struct StreamGeom {
    static constexpr int CH = D / 8;                    // 16-byte pieces per row
    static constexpr int RPI = 64 / CH;                 // rows per wave instruction
    static constexpr int STEP = 4 * RPI;                // rows between a wave's instructions
    static constexpr int NI = kSubRows / STEP;          // instructions per wave and sub-chunk
    static_assert(STEP % 16 == 0 && 16 % CH == 0, "instructions repeat head and swizzle per lane");
};

// This lane's part of every fetch: instruction i writes LDS row
// wave * RPI + i * STEP + lane / CH, which (G <= 16 dividing STEP) holds
// entry el0 + i * STEP / G, head hd, and the piece `off` addresses.
struct StreamLane {
    int el0;  // entry of instruction 0's row within the sub-chunk
    int off;  // element offset within the entry's G * D query elements: hd * D + 8 * piece
};
template <int D>
__device__ __forceinline__ StreamLane stream_lane(int wave, int lane, int glog)
{
    using S = StreamGeom<D>;
    const int r = wave * S::RPI + lane / S::CH;
    const int c = (lane % S::CH) ^ (r & (S::CH - 1));  // the piece stored at this lane's position
    return StreamLane{r >> glog, (r & ((1 << glog) - 1)) * D + 8 * c};
}

// Issue this wave's NI fetches of one sub-chunk; ent[i] = entry of instruction i.
template <int D>
__device__ __forceinline__ void stream_issue(const bf16* Qb, uint32_t qrow, const int* ent, const StreamLane& sl,
                                             bf16* buf, int wave)
{
    using S = StreamGeom<D>;
#pragma unroll
    for (int i = 0; i < S::NI; ++i) {
        const bf16* src = Qb + (uint64_t)((uint32_t)ent[i] >> 6) * qrow + sl.off;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + (wave * S::RPI + i * S::STEP) * D),
                                         16, 0, 0);
    }
}

// Fetch one sub-chunk (nvalid = its entries; rows past them repeat its last
// entry), the entry ids read from ents (LDS) before any fetch issues.
template <int D>
__device__ __forceinline__ void stream_fetch(const bf16* Qb, uint32_t qrow, const int* ents, int nvalid,
                                             const StreamLane& sl, int glog, bf16* buf, int wave)
{
    using S = StreamGeom<D>;
    int ent[S::NI];
#pragma unroll
    for (int i = 0; i < S::NI; ++i) {
        const int el = sl.el0 + ((i * S::STEP) >> glog);
        ent[i] = ents[el < nvalid ? el : nvalid - 1];
    }
    stream_issue<D>(Qb, qrow, ent, sl, buf, wave);
}

// Start of a chunk: the entry ids of its first NB - 1 sub-chunks and of the
// whole chunk (for the LDS copy) are loaded from memory together, then
// stream_prologue_issue starts the fetches; the caller's A operand loads
// follow them.
template <int D, int NB>
struct StreamPrologue {
    int ent[NB - 1][StreamGeom<D>::NI];
    int own;  // entry e0 + threadIdx.x (if any), copied to LDS
};
template <int D, int NB>
__device__ __forceinline__ void stream_prologue_load(StreamPrologue<D, NB>& pr, const int* entries, int n, int SE,
                                                     const StreamLane& sl, int glog)
{
    static_assert(kLeafQC <= 256, "one entry per thread");
#pragma unroll
    for (int k = 0; k < NB - 1; ++k)
#pragma unroll
        for (int i = 0; i < StreamGeom<D>::NI; ++i) {
            const int el = k * SE + sl.el0 + ((i * StreamGeom<D>::STEP) >> glog);
            const int lim = min(n, (k + 1) * SE) - 1;  // last entry of sub-chunk k (k < nsb)
            pr.ent[k][i] = entries[max(0, min(el, lim))];
        }
    pr.own = entries[min((int)threadIdx.x, n - 1)];
}
template <int D, int NB>
__device__ __forceinline__ void stream_prologue_issue(const StreamPrologue<D, NB>& pr, int* lds_ent,
                                                      const bf16* Qb, uint32_t qrow, const StreamLane& sl, bf16* ring,
                                                      int wave)
{
    wait_vm<0>();  // the entry ids: nothing else outstanding from here on
    // branch-free: sub-chunks past the chunk's end refetch its last entry into buffers no
    // tile reads (the last sub-chunk's wait, vmcnt(0), covers them before the chunk ends)
#pragma unroll
    for (int k = 0; k < NB - 1; ++k) stream_issue<D>(Qb, qrow, pr.ent[k], sl, ring + k * kSubRows * D, wave);
    lds_ent[threadIdx.x] = pr.own;  // slots past n hold copies of the last entry
}

// Wait until this wave's fetch of the current sub-chunk has landed, `later`
// (wave-uniform, <= NB - 2) sub-chunks having been issued after it.
template <int D, int NB, int K = NB - 2>
__device__ __forceinline__ void stream_wait(int later)
{
    constexpr int NI = StreamGeom<D>::NI;
    static_assert(NB >= 2 && (NB - 2) * NI < 64, "ring depth within the vmcnt range");
    if constexpr (K <= 0) {
        wait_vm<0>();
    } else {
        if (later >= K) {
            wait_vm<K * NI>();
            return;
        }
        stream_wait<D, NB, K - 1>(later);
    }
}

// Workgroup barrier after this wave's LDS reads and writes have completed.
// The streamed fetches are waited for explicitly (stream_wait), and nothing
// written to global memory is read back by the workgroup, so no vmcnt wait is
// wanted here (a fence would drain the fetches still in flight: they write
// LDS). The memory clobber keeps the compiler from moving accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace pisa
