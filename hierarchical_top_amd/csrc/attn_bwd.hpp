// attn_bwd.hpp -- host-side declarations of the block-sparse attention
// backward (attn_bwd.hip) and of the block clustering it shares with the
// clustered forward (attn_cl.hip).
#pragma once

#include "pisa_internal.hpp"

namespace pisa {

// Count, scan and scatter the (row, selected block) pairs with a visible key
// into entries (row << 6) | slot clustered by (sequence, KV head, block), in
// the tables of L inside ws; fills the table pointers and sizes of a.
hipError_t launch_attn_cluster(AttnClArgs& a, const AttnClLayout& L, char* ws, hipStream_t s);

struct AttnBwdArgs {
    AttnClArgs c;         // Q, K, V, shapes, block_idx, kv_len, cluster tables
    const void* O;        // [B][N_q][H_q][d] forward output
    const void* dO;       // [B][N_q][H_q][d] gradient of the loss w.r.t. O
    const float* lse;     // [B][H_q][N_q] forward log-normaliser (natural log)
    float* dsum;          // [B][H_q][N_q] workspace: sum over d of dO * O
    float* part_dq;       // [B][H_kv][N_q][K_top][G][d] workspace: dQ of each (row, slot, head)
    float* dQ;            // [B][N_q][H_q][d]
    float* dK;            // [B][N_alloc][H_kv][d]
    float* dV;            // [B][N_alloc][H_kv][d]
};

struct AttnBwdLayout {
    AttnClLayout cl;      // cluster tables (the forward's partial-output sections are not used)
    size_t dsum, part_dq, bytes;
};
AttnBwdLayout attn_bwd_layout(int64_t B, int64_t N_q, int64_t N_alloc, int H_q, int H_kv, int d, int C, int K_top);
hipError_t launch_attn_bwd(AttnBwdArgs a, int d, char* ws, hipStream_t s);

}  // namespace pisa
