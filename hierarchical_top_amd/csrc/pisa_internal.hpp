// pisa_internal.hpp -- kernel argument blocks and launchers shared between the
// C ABI layer (capi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pisa.h"

namespace pisa {

// Pyramid geometry and storage, copied from pisa_pyramid (kernel argument).
struct PyrArgs {
    int B, H, d, C, g, g_log2, c_log2, L_cap;
    int64_t N_cap;
    int64_t M_cap[PISA_MAX_LEVELS + 1];
    int64_t off[PISA_MAX_LEVELS + 1];
    float* buf;
};

// Routing of one (query, KV head) item per workgroup (prefill fused,
// prefill stage 1, decode).
struct RouteArgs {
    PyrArgs p;
    const void* Q;        // prefill [B][N][H_q][d]; decode [B][H_q][d]
    const void* K;        // [B][N_cap][H_kv][d]
    int64_t N;            // prefill sequence length (unused for decode)
    const int64_t* seqlen;  // decode: per-sequence length; null for prefill
    int H_q, G, K_top, causal;
    int score_kind;       // level-synchronous router: 0 LSE, 1 mean (PISA-1), 2 mean + var / 2 (PISA-2)
    int32_t* idx;         // fused / decode output
    float* score;         // nullable
    // stage 1 outputs
    int32_t* kept2;       // [B][H][N][K_top]
    int64_t* meta;        // [B][H][N]
    int32_t* counts;      // [B][H][M2] cluster sizes
    int64_t M2;           // level-2 nodes for this N (1 if N <= C * ... see capi)
};

// Leaf scoring of clustered (query, retained level-2 node) pairs.
struct Stage2Args {
    PyrArgs p;
    const void* Q;
    const void* K;
    int64_t N;
    int H_q, G, K_top;
    int64_t n_clusters;          // B * H * M2
    int64_t M2;
    const int32_t* offsets;      // [n_clusters + 1] entry offsets
    const int32_t* chunk_off;    // [n_clusters + 1] chunk offsets
    const int32_t* entries;      // (t << 6) | slot
    float* u;                    // [B][H][N][g * K_top]
};

struct FinalArgs {
    int B, H, C, g, c_log2, g_log2, K_top, causal;
    int64_t N;
    const int32_t* kept2;
    const int64_t* meta;
    const float* u;
    int32_t* idx;
    float* score;
};

struct ScatterArgs {
    int B, H, K_top;
    int64_t N, M2;
    const int32_t* kept2;
    const int64_t* meta;
    const int32_t* offsets;
    int32_t* cursor;
    int32_t* entries;
};

struct AttnArgs {
    const void* Q;
    const void* K;
    const void* V;
    int B, H_q, H_kv, G, C, K_top, causal;
    int64_t N_q, N_kv, N_alloc;
    const int32_t* idx;
    const int64_t* kv_len;
    void* O;
    float* lse;
};

// Clustered attention (attn_cl.hip): arguments as in AttnArgs plus the
// workspace sections (attn_cl_layout).
struct AttnClArgs {
    const void* Q;
    const void* K;
    const void* V;
    int B, H_q, H_kv, G, C, K_top, causal;
    int64_t N_q, N_kv, N_alloc;
    const int32_t* idx;
    const int64_t* kv_len;
    void* O;
    float* lse;
    int64_t M_blk;       // blocks per sequence: ceil(N_alloc / C)
    int64_t n_clusters;  // B * H_kv * M_blk
    int qc;              // entries per chunk
    int32_t* counts;
    int32_t* cursor;
    int32_t* offsets;
    int32_t* chunk_off;
    int32_t* chunk_cl;
    int32_t* block_sums;
    int32_t* entries;    // (row << 6) | slot
    float* part_lse;     // [B][H_kv][N_q][K_top][G][2]: base-2 log-sum-exp of the block's scaled scores, exponent e
    void* part_o;        // [B][H_kv][N_q][K_top][G][d] fp16: the block's normalised output times 2^-e
};

struct AttnClLayout {
    int64_t M_blk, n_clusters, n_items, max_chunks, n_sums;
    size_t counts, offsets, chunk_off, chunk_cl, block_sums, entries, part_lse, part_o, bytes;
};
AttnClLayout attn_cl_layout(int64_t B, int64_t N_q, int64_t N_alloc, int H_kv, int G, int d, int C, int K_top);
hipError_t launch_attn_clustered(AttnClArgs a, int d, char* ws, hipStream_t s);

// Shared clustering steps (levels.hip): zero n ints; exclusive scans of n
// cluster sizes into offsets, chunks of qc entries per cluster into chunk_off
// and the chunk -> cluster map (chunk_cl holds max_chunks, a bound on the chunks).
hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t s);
hipError_t launch_scan_chunks(const int32_t* counts, int64_t n, int qc, int32_t* block_sums, int32_t* offsets,
                              int32_t* chunk_off, int32_t* chunk_cl, int64_t max_chunks, hipStream_t s);

struct BsaArgs {
    PyrArgs p;
    const void* Q;
    int64_t N;
    int H_q, G, K_top, causal;
    int32_t* idx;
    float* score;
};

// Level-synchronous routing: clusters of level l are keyed by (query window,
// sequence and KV head, kept node of level l+1), and cut into chunks of up to 256
// entries. A window trades locality (the queries a cluster gathers) against the fill
// of its chunks: every chunk pays for loading its node's rows and priming its query
// ring, and small windows leave many clusters far below 256 entries. Measured at 256K
// (16 / 4 heads, d=128): leaf windows of 2^18 and level-2 windows of 2^14 beat 2^15 and
// 2^13 by about 4 % each, with identical selections.
inline int cluster_win_log2(int level) { return level == 1 ? 18 : 12; }

// Level-synchronous routing: clustered scoring of one level.
struct ScoreArgs {
    const void* Q;            // [B][N][H_q][d]
    int64_t N;
    int H, H_q, G, K_top, g;
    const void* rows;         // level l-1 data: summaries (float) or keys (dtype of Q)
    int64_t rows_b_stride;    // elements between sequences
    int64_t rows_h_stride;    // elements between KV heads
    int64_t row_stride;       // elements between consecutive rows
    int64_t rows_limit;       // rows that exist (nodes of level l-1, or tokens)
    int rc;                   // rows per candidate (g, or C at the leaf level)
    int qc;                   // entries per chunk
    int64_t n_clusters;       // windows * B * H * M_bins
    int64_t M_bins;           // nodes of level l+1 (cluster keys)
    int64_t BH;               // B * H
    int xcd;                  // 1: give each XCD a contiguous range of chunks
    int sk;                   // block score: 0 LSE, 1 mean (PISA-1), 2 mean + var / 2 (PISA-2)
    const int32_t* offsets;   // [n_clusters + 1]
    const int32_t* chunk_off; // [n_clusters + 1]
    const int32_t* chunk_cl;  // [chunks] cluster of each chunk
    const int32_t* entries;   // (t << 6) | slot
    float* u;                 // [B][H][N][K_top * g]
    // the rows of an upper level as two bf16 terms (split_layout), read by upper_ring_kernel:
    // row r of (b, h) at rows_hl + b * rows_hl_b_stride + h * rows_hl_h_stride + r * 2 d
    const void* rows_hl;
    int64_t rows_hl_b_stride, rows_hl_h_stride;
};

// Dense scoring of an upper level: every query tile scores the children of
// every eligible node of level l+1 (the union of its queries' kept nodes is
// most of them at these sizes), reading each query once per level instead of
// once per kept node. Used for levels whose nodes number at most kDenseParents
// and whose rows (level l-1 summaries) number at most kDenseRows, so the dense
// work stays O(N) per level; g in {2, 4}.
constexpr int kDenseParents = 16;
constexpr int64_t kDenseRows = 256;

// nodes of level l (level 1 = leaf blocks of 2^c_log2 tokens) over n tokens
inline int64_t level_nodes(int64_t n, int c_log2, int g_log2, int l)
{
    const int sh = c_log2 + (l - 1) * g_log2;
    return (n + ((int64_t)1 << sh) - 1) >> sh;
}
// level l is scored densely (see above)
inline bool dense_level(int64_t n, int c_log2, int g_log2, int l)
{
    const int g = 1 << g_log2;
    return l >= 2 && (g == 2 || g == 4) && level_nodes(n, c_log2, g_log2, l + 1) <= kDenseParents &&
           level_nodes(n, c_log2, g_log2, l - 1) <= kDenseRows;
}
// Two dense levels in a row share one pass over the queries: going down from l_top, a dense
// level l whose next level l - 1 is dense too scores both (level l - 1 for every eligible
// level-l node, kept by node id: its kept set is not known yet). Returns whether level l opens
// such a pair, given that level l + 1 did not.
inline bool dense_pair(int64_t n, int c_log2, int g_log2, int l)
{
    return dense_level(n, c_log2, g_log2, l) && dense_level(n, c_log2, g_log2, l - 1);
}
// columns of the by-node score rows of a pair's second level: every child slot of every
// level-l node, rounded up to 4 so that rows stay 16-byte aligned
inline int64_t dense_pair_cols(int64_t n, int c_log2, int g_log2, int l)
{
    return ((level_nodes(n, c_log2, g_log2, l) << g_log2) + 3) & ~(int64_t)3;
}
// the widest by-node score row over the dense pairs of a route from level l_top down (0: none)
inline int64_t dense_pair_max_cols(int64_t n, int c_log2, int g_log2, int l_top)
{
    int64_t cols = 0;
    for (int l = l_top; l >= 2; --l) {
        if (!dense_pair(n, c_log2, g_log2, l)) continue;
        const int64_t c = dense_pair_cols(n, c_log2, g_log2, l);
        if (c > cols) cols = c;
        --l;  // level l - 1 is the pair's second level
    }
    return cols;
}

// The level router splits the fp32 summaries of levels 1 .. l_top - 1 once per call into two
// bf16 terms (hi = the value rounded to bf16, lo = the rest rounded to bf16, as the MFMA
// operands take them): level l holds rows [B * H][nodes(n, l)][hi d | lo d] at off[l] bf16
// elements, each level 256-byte aligned. Returns the total bf16 elements (0 below l_top = 2).
inline int64_t split_layout(int64_t n, int c_log2, int g_log2, int l_top, int64_t BH, int d, int64_t* off)
{
    int64_t e = 0;
    for (int l = 1; l < l_top; ++l) {
        if (off) off[l] = e;
        e += BH * level_nodes(n, c_log2, g_log2, l) * 2 * d;
        e = (e + 127) & ~(int64_t)127;
    }
    return e;
}

struct DenseArgs {
    const void* Q;            // [B][N][H_q][d]
    int64_t N;
    int B, H, H_q, G, K_top, g, causal;
    // level l-1 summaries of (b, h) as two bf16 terms (split_layout): row r at
    // rows_hl + b * rows_hl_b_stride + h * rows_hl_h_stride + r * 2 d (bf16 elements)
    const void* rows_hl;
    int64_t rows_hl_b_stride, rows_hl_h_stride;
    int64_t rows_limit;       // level l-1 nodes that exist
    int par_span_log2;        // log2 of the tokens spanned by a level-(l+1) node
    int64_t M_par;            // level l+1 nodes that exist
    int sk;                   // block score, as in ScoreArgs
    const int32_t* kept;      // [items][K_top] kept nodes of level l+1
    float* u;                 // [items][K_top * g]
    // optional second level l - 1 in the same pass over the queries (rows2 != null): the
    // candidates of every eligible level-l node, written to u2 by node id
    const void* rows2_hl;     // level l-2 summaries, layout as for rows_hl
    int64_t rows2_hl_b_stride, rows2_hl_h_stride, rows2_limit;
    int par2_span_log2;       // log2 of the tokens spanned by a level-l node
    int64_t M_par2;           // level-l nodes that exist
    float* u2;                // [items][u2_cols]: column x = level l-1 node x
    int64_t u2_cols;
};

// Upper levels whose nodes have g * g <= 16 grandchildren: one wave per chunk
// of kRegChunk entries, rows loaded straight into MFMA operand registers.
constexpr int kRegChunk = 32;
constexpr int kRegWaves = 4;

// Leaf and upper levels with bf16 queries and g in {2, 4}: chunks of kLeafQC
// entries whose query rows (entry x head) stream through a ring of LDS
// buffers kSubRows rows at a time, kLeafNB / kUpperNB buffers deep.
constexpr int kLeafQC = 256;
constexpr int kSubRows = 64;
// cluster counters aggregated per workgroup in LDS up to this many bins (else global atomics)
constexpr int kLdsBins = 8192;
constexpr int kLeafNB = 2;
constexpr int kUpperNB = 2;
// Upper levels, one wave per chunk (upper_ring_kernel): chunks of kWaveQC entries, a ring of
// kUpperWaveNB 16-row tiles per wave.
constexpr int kWaveQC = 64;
constexpr int kUpperWaveNB = 2;
// LDS bytes of one such workgroup: the ring, the chunk's entries and its scores
inline size_t stream_lds_bytes(int d, int nb) { return (size_t)nb * kSubRows * d * 2 + (size_t)kLeafQC * (4 + 16); }

// Per-item selection of one level, and counting of the next level's clusters.
struct SelectArgs {
    int B, H, c_log2, g_log2, K_top, causal;
    int64_t N;
    int level;                // the level whose kept set is produced
    int init;                 // 1: the candidates are all eligible nodes of `level`
    const int32_t* kept_in;   // [items][K_top] kept nodes of level + 1
    const float* u;           // [items][K_top * g] scores of the candidates of `level`
    int32_t* kept_out;        // [items][K_top] (level > 1)
    int64_t* flags_out;       // [items] slots of kept_out whose children are scored next
    int32_t* counts;          // [windows][B * H][M_bins] cluster sizes for the next level (level > 1)
    int64_t M_bins;           // nodes of `level`
    int win_log2;             // query window of the next level's clusters
    int32_t* idx;             // level 1: [items][K_top]
    float* score;             // level 1: [items][K_top] or null
    int64_t u_cols;           // 0: u is [items][K_top * g] by kept slot; else [items][u_cols] by node id
};

struct LevelsArgs {
    RouteArgs r;              // pyramid, Q, K, N, heads, K_top, causal, outputs
    int32_t* kept[2];
    int64_t* flags;
    float* u;
    float* u_pair;            // by-node scores of the second level of a dense pair: [items][cols]
    int32_t* counts;          // per scored level, at cnt_off[level]
    int32_t* cursor;          // same layout as counts
    int64_t cnt_total;
    int64_t cnt_off[PISA_MAX_LEVELS + 2];
    int32_t* offsets;
    int32_t* chunk_off;
    int32_t* chunk_cl;        // [max chunks]
    int32_t* block_sums;      // scan partials: 2 * (max clusters / 1024 + 1)
    int32_t* entries;
    void* rows_hl;            // the summaries of levels 1 .. l_top - 1 as two bf16 terms (split_layout)
    int l_top;                // highest scored level (0: nothing is scored)
};

hipError_t launch_build(const PyrArgs& a, const void* K, int dtype, int64_t n, hipStream_t s);
hipError_t launch_append(const PyrArgs& a, const void* K, int dtype, const int64_t* seqlen, hipStream_t s);
hipError_t launch_route_query(const RouteArgs& a, int dtype, int d, int mode, hipStream_t s);
hipError_t launch_two_stage(const RouteArgs& a, const Stage2Args& s2, const FinalArgs& f,
                            const ScatterArgs& sc, int32_t* zero_base, int64_t zero_count, int dtype,
                            int d, hipStream_t s);
hipError_t launch_levels(const LevelsArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_dense(const DenseArgs& a, int dtype, int d, hipStream_t s);
// kind: 0 summary rows staged in LDS, 1 key rows (leaf), 2 summary rows in registers,
// 3 leaf keys in registers with queries through LDS (bf16), 4 upper levels likewise (bf16)
hipError_t launch_score(const ScoreArgs& a, int dtype, int d, int kind, int64_t grid, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_bsa(const BsaArgs& a, int dtype, int d, hipStream_t s);

enum { MODE_FUSED = 0, MODE_STAGE1 = 1, MODE_DECODE = 2 };

// Stage timing (pisa_time_stage): records the caller's armed start / stop
// events on the launch stream around a stage; no-op when nothing is armed.
void stage_mark(int stage, bool stop, hipStream_t s);

}  // namespace pisa
