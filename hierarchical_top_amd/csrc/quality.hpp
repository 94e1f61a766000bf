// quality.hpp -- host-side declarations of the block-selection quality
// evaluation against full attention (quality.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pisa {

struct QualArgs {
    const void* Q;         // [B][N][H_q][d] bf16
    const void* K;         // [B][N][H_kv][d] bf16
    int B, H_q, H_kv, G, C, K_top;
    int64_t N, M1;
    const int32_t* sel;    // [B][H_kv][N][K_top] the selector's blocks
    float* lmass;          // [B][H_q][N][M1] workspace: log mass per (query head, row, block)
    float* mass;           // [B][H_kv][N][M1] or null
    int32_t* ref;          // [B][H_kv][N][K_top] or null
    float* recall;         // [B][H_kv][N]
    float* captured;
    float* ratio;
};

size_t quality_workspace_bytes(int64_t B, int64_t N, int H_q, int C);
hipError_t launch_quality(QualArgs a, int d, hipStream_t s);

}  // namespace pisa
