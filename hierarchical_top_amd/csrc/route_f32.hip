// route_f32.hip -- f32 instances of the routing kernels (see route_impl.hpp).
#include "route_impl.hpp"

namespace pisa {

template <int D, int G, int SK>
static hipError_t route_query_sk(const RouteArgs& a, int mode, hipStream_t s)
{
    if (mode == MODE_DECODE)
        hipLaunchKernelGGL((route_decode_kernel<D, float, G, SK>), dim3((unsigned)(a.p.B * a.p.H)), dim3(64 * kDecodeWaves), 0,
                           s, a);
    else
        hipLaunchKernelGGL((route_query_kernel<D, float, G, MODE_FUSED, SK>), dim3((unsigned)((int64_t)a.p.B * a.p.H * a.N)),
                           dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int D, int G>
static hipError_t route_query_dg(const RouteArgs& a, int mode, hipStream_t s)
{
    if (mode == MODE_STAGE1) {
        hipLaunchKernelGGL((route_query_kernel<D, float, G, MODE_STAGE1>), dim3((unsigned)((int64_t)a.p.B * a.p.H * a.N)),
                           dim3(64), 0, s, a);
        return hipGetLastError();
    }
    switch (a.score_kind) {  // block score: LSE, PISA-1 mean, PISA-2 mean + var / 2
    case 1: return route_query_sk<D, G, 1>(a, mode, s);
    case 2: return route_query_sk<D, G, 2>(a, mode, s);
    default: return route_query_sk<D, G, 0>(a, mode, s);
    }
}

template <int D, int G>
static hipError_t stage2_dg(const Stage2Args& a, int64_t grid, hipStream_t s)
{
    const size_t lds = (size_t)a.p.g * a.p.C * (D + 8) * 2 * Src<float>::TERMS;
    auto k = stage2_kernel<D, float, G>;
    hipError_t err = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(256), lds, s, a);
    return hipGetLastError();
}

#define PISA_G_SWITCH(F, D, ...)                                   \
    switch (G) {                                                   \
    case 1: return F<D, 1>(__VA_ARGS__);                       \
    case 2: return F<D, 2>(__VA_ARGS__);                       \
    case 4: return F<D, 4>(__VA_ARGS__);                       \
    case 8: return F<D, 8>(__VA_ARGS__);                       \
    default: return hipErrorInvalidValue;                          \
    }

hipError_t route_query_f32(const RouteArgs& a, int d, int mode, hipStream_t s)
{
    const int G = a.G;
    if (d == 64) { PISA_G_SWITCH(route_query_dg, 64, a, mode, s) }
    if (d == 128) { PISA_G_SWITCH(route_query_dg, 128, a, mode, s) }
    return hipErrorInvalidValue;
}

hipError_t stage2_f32(const Stage2Args& a, int d, int64_t grid, hipStream_t s)
{
    const int G = a.G;
    if (d == 64) { PISA_G_SWITCH(stage2_dg, 64, a, grid, s) }
    if (d == 128) { PISA_G_SWITCH(stage2_dg, 128, a, grid, s) }
    return hipErrorInvalidValue;
}

}  // namespace pisa
