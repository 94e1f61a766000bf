// levels_f32.hip -- f32 instances of the clustered scoring kernel (levels_impl.hpp).
#include "levels_impl.hpp"

namespace pisa {

template <int D, typename TS, int RC>
static hipError_t score_launch(const ScoreArgs& a, int64_t grid, hipStream_t s)
{
    const size_t lds = (size_t)Src<TS>::TERMS * ((a.g * a.rc + 15) & ~15) * (D + 8) * 2;
    auto k = score_kernel<D, float, TS, RC>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kScoreThreads), lds, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t score_d(const ScoreArgs& a, bool key_rows, int64_t grid, hipStream_t s)
{
    if (key_rows) return score_launch<D, float, RC16>(a, grid, s);
    switch (a.rc) {
    case 2: return score_launch<D, float, RC2>(a, grid, s);
    case 4: return score_launch<D, float, RC4>(a, grid, s);
    case 8: return score_launch<D, float, RC8>(a, grid, s);
    default: return score_launch<D, float, RC16>(a, grid, s);
    }
}

hipError_t score_f32(const ScoreArgs& a, int d, bool key_rows, int64_t grid, hipStream_t s)
{
    return d == 64 ? score_d<64>(a, key_rows, grid, s) : score_d<128>(a, key_rows, grid, s);
}

}  // namespace pisa
