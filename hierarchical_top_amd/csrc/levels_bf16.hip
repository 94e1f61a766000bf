// levels_bf16.hip -- bf16 instances of the clustered scoring kernel (levels_impl.hpp).
#include "levels_impl.hpp"

namespace pisa {

template <int D, typename TS, int RC, int WAVES, int SK>
static hipError_t score_launch(const ScoreArgs& a, int64_t grid, hipStream_t s)
{
    const size_t lds = (size_t)Src<TS>::TERMS * ((a.g * RC + 15) & ~15) * (D + 8) * 2 + (size_t)a.qc * 4;
    auto k = score_kernel<D, bf16, TS, RC, WAVES, SK>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64 * WAVES), lds, s, a);
    return hipGetLastError();
}

template <int D, int RC, int SK>
static hipError_t score_reg_launch(const ScoreArgs& a, int64_t grid, hipStream_t s)
{
    hipLaunchKernelGGL((score_reg_kernel<D, bf16, RC, SK>), dim3((unsigned)grid), dim3(64 * kRegWaves), 0, s, a);
    return hipGetLastError();
}

template <int D, int SK>
static hipError_t score_d(const ScoreArgs& a, int kind, int64_t grid, hipStream_t s)
{
    if (kind == 2) return a.rc == 2 ? score_reg_launch<D, 2, SK>(a, grid, s) : score_reg_launch<D, 4, SK>(a, grid, s);
    if (kind == 6) {  // upper levels, one wave per chunk with its own LDS ring: four chunks per workgroup
        const size_t lds = 4 * wave_ring_bytes<D, kUpperWaveNB>();
        const void* k = a.rc == 2 ? (const void*)upper_ring_kernel<D, 2, kUpperWaveNB, SK>
                                  : (const void*)upper_ring_kernel<D, 4, kUpperWaveNB, SK>;
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        ScoreArgs arg = a;
        void* args[] = {&arg};
        hipError_t e = hipLaunchKernel(k, dim3((unsigned)((grid + 3) / 4)), dim3(256), args, lds, s);
        return e != hipSuccess ? e : hipGetLastError();
    }
    if (kind == 3 || kind == 4) {  // queries streamed through LDS: leaf (keys) or upper (grandchildren)
        const size_t lds = stream_lds_bytes(D, kind == 3 ? kLeafNB : kUpperNB);
        const void* k;
        if (kind == 3)
            k = a.rc == 16 ? (const void*)leaf_kernel<D, 16, kLeafNB, SK>
                           : (a.rc == 32 ? (const void*)leaf_kernel<D, 32, kLeafNB, SK> : (const void*)leaf_kernel<D, 64, kLeafNB, SK>);
        else
            k = a.rc == 2 ? (const void*)upper_kernel<D, 2, kUpperNB, SK> : (const void*)upper_kernel<D, 4, kUpperNB, SK>;
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        ScoreArgs arg = a;
        void* args[] = {&arg};
        hipError_t e = hipLaunchKernel(k, dim3((unsigned)grid), dim3(256), args, lds, s);
        return e != hipSuccess ? e : hipGetLastError();
    }
    if (kind == 1) {  // leaf level: rows per candidate = C
        switch (a.rc) {
        case 16: return score_launch<D, bf16, 16, 8, SK>(a, grid, s);
        case 32: return score_launch<D, bf16, 32, 8, SK>(a, grid, s);
        default: return score_launch<D, bf16, 64, 8, SK>(a, grid, s);
        }
    }
    switch (a.rc) {  // upper levels: rows per candidate = g
    case 2: return score_launch<D, float, 2, 4, SK>(a, grid, s);
    case 4: return score_launch<D, float, 4, 4, SK>(a, grid, s);
    case 8: return score_launch<D, float, 8, 4, SK>(a, grid, s);
    default: return score_launch<D, float, 16, 4, SK>(a, grid, s);
    }
}

template <int SK>
static hipError_t score_sk(const ScoreArgs& a, int d, int kind, int64_t grid, hipStream_t s)
{
    return d == 64 ? score_d<64, SK>(a, kind, grid, s) : score_d<128, SK>(a, kind, grid, s);
}

hipError_t score_bf16(const ScoreArgs& a, int d, int kind, int64_t grid, hipStream_t s)
{
    switch (a.sk) {  // block score: LSE, PISA-1 mean, PISA-2 mean + var / 2
    case 1: return score_sk<1>(a, d, kind, grid, s);
    case 2: return score_sk<2>(a, d, kind, grid, s);
    default: return score_sk<0>(a, d, kind, grid, s);
    }
}

template <int D, int GB, int SK>
static hipError_t dense_launch(const DenseArgs& a, hipStream_t s)
{
    const int GT = a.G * Src<bf16>::TERMS, QT = 16 / GT, nct = GT < 4 ? GT : 4;
    const int QW = 4 * nct * QT;
    const int64_t pm = a.causal ? ((a.N - 1) >> a.par_span_log2) + 1 : a.M_par;
    const int npar = (int)(pm < a.M_par ? pm : a.M_par);
    const size_t lds = (size_t)2 * kDenseBatch * 16 * (D + 8) * 2 + (size_t)QW * npar;
    const dim3 grid((unsigned)((a.N + QW - 1) / QW), (unsigned)(a.B * a.H));
    hipLaunchKernelGGL((dense_kernel<D, bf16, GB, SK>), grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

template <int SK>
static hipError_t dense_sk(const DenseArgs& a, int d, hipStream_t s)
{
    if (d == 64) return a.g == 2 ? dense_launch<64, 2, SK>(a, s) : dense_launch<64, 4, SK>(a, s);
    return a.g == 2 ? dense_launch<128, 2, SK>(a, s) : dense_launch<128, 4, SK>(a, s);
}

hipError_t dense_bf16(const DenseArgs& a, int d, hipStream_t s)
{
    switch (a.sk) {
    case 1: return dense_sk<1>(a, d, s);
    case 2: return dense_sk<2>(a, d, s);
    default: return dense_sk<0>(a, d, s);
    }
}

}  // namespace pisa
