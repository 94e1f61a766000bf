/*
 * pisa.h -- C ABI of libpisa: PISA pyramid Top-K block selection and
 * block-sparse attention for AMD Instinct MI355X (gfx950).
 *
 * Method: "Block Sparse Attention with Log-Linear Complexity" (PISA), arXiv
 * HTML full text. Section and equation numbers below refer to that page. The
 * page numbers blocks from 1; this interface numbers everything from 0.
 *
 * General conventions
 * -------------------
 * - Every pointer argument named as device memory must point to memory of the
 *   current HIP device. The library never allocates, frees or synchronises:
 *   the caller owns every buffer (inputs, outputs, the pyramid buffer and the
 *   workspace) and keeps them alive until the work queued on `stream` is done.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   All work is queued asynchronously on it.
 * - Arguments are validated on the host before anything is queued; a failed
 *   check returns a negative status and queues nothing. pisa_last_error()
 *   then returns a message naming the argument (per host thread).
 * - Tensors are dense and row-major, innermost dimension last, base pointers
 *   16-byte aligned. dtype PISA_BF16 is bfloat16, PISA_F32 is IEEE float.
 * - Grouped-query heads are contiguous: query head h' reads KV head h' / G_Q,
 *   where G_Q = H_q / H_kv (the `gqa_group` argument).
 * - Block ids are 0-based leaf-block indices; leaf block i holds tokens
 *   [i*C, min(i*C + C, n)).
 * - Supported shapes: d in {64, 128}; C in {16, 32, 64}; g in {2, 4, 8, 16};
 *   G_Q in {1, 2, 4, 8, 16}; G_Q * (2 if f32 else 1) <= 16;
 *   1 <= K_top <= 64 and g * K_top <= 64, or K_top >= the number of leaf
 *   blocks (then every eligible leaf is kept); causal routing needs K_top >= 3.
 *   Other shapes return PISA_EUNSUPPORTED.
 * - Calls do not share mutable state; two calls may run concurrently on
 *   different streams if they do not write the same buffers.
 * - Selection is defined for finite inputs. With NaN or inf in Q or K every
 *   router still returns valid rows (ascending, causal, -1 padded, forced
 *   blocks present); a candidate whose score is NaN is never picked, so a row
 *   may then hold fewer than K_top blocks.
 */
#ifndef PISA_H
#define PISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PISA_ABI_VERSION 1
#define PISA_MAX_LEVELS 32

typedef enum pisa_status {
    PISA_OK = 0,
    PISA_EINVAL = -1,        /* an argument is out of range or inconsistent */
    PISA_EUNSUPPORTED = -2,  /* valid, but no kernel is built for this shape */
    PISA_ENOSPACE = -3,      /* a length exceeds the pyramid capacity, or the workspace is too small */
    PISA_EHIP = -4           /* the HIP runtime reported an error while queueing */
} pisa_status;

/* Element types. Calls take a dtype as int32_t holding one of these values (any other
 * value is rejected with PISA_EINVAL), so that no caller can pass an out-of-range enum. */
typedef enum pisa_dtype { PISA_F32 = 0, PISA_BF16 = 1 } pisa_dtype;

typedef enum pisa_route_mode {
    PISA_ROUTE_TWO_STAGE = 0,  /* section 3.3: intermediate levels per query, then leaf
                                  scoring per retained level-2 node with key reuse */
    PISA_ROUTE_FUSED = 1,      /* all levels of one query in one program (per-query) */
    PISA_ROUTE_LEVELS = 2      /* all queries advance one level at a time; at every level
                                  the (query, kept node) pairs are clustered by node and
                                  scored with the node's data staged once (K_top <= 32) */
} pisa_route_mode;

/*
 * Key pyramid (section 3.2, "Fine-to-coarse block aggregation", eq 7-15).
 * Level 0 is the caller's keys. Level 1 holds one summary per leaf block of C
 * keys, level l+1 one per group of g level-l blocks; M_1 = ceil(n / C),
 * M_{l+1} = ceil(M_l / g), and the top level L is the first with one block.
 * Each summary is the mean of its existing children (the mean of the keys
 * present for a leaf; an unweighted mean of the existing children above).
 *
 * Storage: float32, level l (1 <= l <= L_cap) at float offset off[l] of buf,
 * laid out [B][H_kv][M_cap[l]][d]. Node j of level l for a sequence of n
 * tokens is valid when j < ceil(n / (C * g^(l-1))).
 *
 * The descriptor is plain data owned by the caller: pisa_pyramid_plan() fills
 * the geometry and `floats`; the caller then allocates `floats` float32 of
 * device memory and stores the pointer in `buf`.
 */
typedef struct pisa_pyramid {
    int32_t B, H_kv, d, C, g;
    int32_t L_cap;                        /* levels at capacity */
    int64_t N_cap;                        /* tokens per sequence the buffer holds */
    int64_t M_cap[PISA_MAX_LEVELS + 1];   /* nodes per level at capacity; M_cap[0] = N_cap */
    int64_t off[PISA_MAX_LEVELS + 1];     /* float offset of level l in buf */
    int64_t floats;                       /* size of buf in float32 elements */
    float* buf;                           /* device memory, set by the caller */
} pisa_pyramid;

/* Fill the geometry of a pyramid for B sequences of up to N_cap tokens with
 * H_kv heads of dimension d, leaf size C and branching g. buf is set to NULL.
 * Errors: PISA_EINVAL (non-positive sizes, N_cap too large for
 * PISA_MAX_LEVELS levels), PISA_EUNSUPPORTED (d, C or g not supported). */
pisa_status pisa_pyramid_plan(pisa_pyramid* p, int32_t B, int32_t H_kv, int32_t d, int32_t C,
                              int32_t g, int64_t N_cap);

/* Build every level of the pyramid over the first N tokens of K
 * (section 3.2 eq 15). K: device, dtype dt, [B][N_cap][H_kv][d]. Writes levels
 * 1..L(N) of p->buf. Summaries are fp32 sums in token (or child) order
 * divided by the count. Errors: PISA_EINVAL (null pointers, N < 1),
 * PISA_ENOSPACE (N > N_cap). */
pisa_status pisa_build_pyramid(const pisa_pyramid* p, const void* K, int32_t dt, int64_t N,
                               void* stream);

/* Decode cache update (section 3.3, "Decoding": only the current leaf mean and
 * its ancestor path change when a token is appended). K: device
 * [B][N_cap][H_kv][d] already holding the new token of sequence b at position
 * seqlen[b] - 1. seqlen: device int64 [B], lengths after the append
 * (1 <= seqlen[b] <= N_cap, not checked on the host: lengths live on the
 * device). Recomputes, per (b, h), leaf floor((seqlen[b]-1)/C) and each of its
 * ancestors up to level L(seqlen[b]) in the same order as
 * pisa_build_pyramid, so the result is bit-identical to a rebuild.
 * The previous lengths must have been built or appended one token at a time. */
pisa_status pisa_pyramid_append(const pisa_pyramid* p, const void* K, int32_t dt,
                                const int64_t* seqlen, void* stream);

/* Workspace bytes pisa_route_prefill needs for these arguments (0 for
 * PISA_ROUTE_FUSED). The workspace must be 256-byte aligned. */
pisa_status pisa_route_prefill_workspace(const pisa_pyramid* p, int64_t N, int32_t H_q,
                                         int32_t K_top, int32_t mode, size_t* bytes);

/*
 * Prefill routing (section 3.2 eq 16-22, appendix B). For every sequence b,
 * position t < N and KV head h: starting from the single top block, at each
 * level drop candidates that start after t (causal), keep all candidates if
 * at most K_top remain, otherwise keep the forced nodes (ancestors of the
 * first, previous and current leaf; causal only) plus the best
 * K_top - |forced| others by the grouped LSE score
 *     u_i = sum over the G_Q query heads h' of KV head h of
 *           log sum_{r in children(i)} exp(q_{t,h'} . kbar_r / sqrt(d)),
 * (leaves use their raw keys as children), ties to the lower index; then
 * expand the kept nodes to their children. fp32 dot products and reductions.
 *
 * Q: device [B][N][H_q][d]; K: the keys the pyramid was built from
 * ([B][N_cap][H_kv][d], dtype dt); the pyramid must hold a build over N.
 * idx: device int32 [B][H_kv][N][K_top], ascending block ids, -1 padded.
 * score: device float32 [B][H_kv][N][K_top] or NULL: the leaf-level u of a
 * block kept by ranking, +inf for a block kept without a score, -inf padding.
 * ws: device workspace of ws_bytes >= pisa_route_prefill_workspace().
 * gqa_group must equal H_q / p->H_kv. causal: 1 = causal routing with the
 * forced set, 0 = no eligibility filter and no forced set.
 * Errors: PISA_EINVAL, PISA_EUNSUPPORTED, PISA_ENOSPACE (N > N_cap or the
 * workspace is too small), PISA_EHIP.
 */
pisa_status pisa_route_prefill(const pisa_pyramid* p, const void* Q, const void* K,
                               int32_t dt, int64_t N, int32_t H_q, int32_t K_top,
                               int32_t causal, int32_t gqa_group, int32_t mode, int32_t* idx,
                               float* score, void* ws, size_t ws_bytes, void* stream);

/*
 * Allocation-free prefill routing, for callers that cannot allocate device
 * memory (code under stream capture, serving loops, harnesses that forbid
 * allocation). Same semantics, outputs and errors as pisa_route_prefill with
 * mode PISA_ROUTE_LEVELS and no caller workspace: the workspace is a
 * library-owned device array of PISA_NOALLOC_SCRATCH_BYTES per device (held
 * until the process ends), so the call accepts only shapes whose level-router
 * workspace (pisa_route_prefill_workspace with PISA_ROUTE_LEVELS) fits in it,
 * and returns PISA_ENOSPACE otherwise (e.g. B * H_kv * N up to about 2^18
 * (query, KV head) items at K_top = 8, g = 4). It calls no allocator. Every
 * call on one device shares that array: calls that overlap on one device
 * (concurrent streams or host threads) race and must be serialised by the
 * caller; consecutive calls on one stream are safe (the array needs no
 * clearing between calls).
 */
#define PISA_NOALLOC_SCRATCH_BYTES (64u << 20)
pisa_status pisa_route_prefill_noalloc(const pisa_pyramid* p, const void* Q, const void* K,
                                       int32_t dt, int64_t N, int32_t H_q, int32_t K_top,
                                       int32_t causal, int32_t gqa_group, int32_t* idx,
                                       float* score, void* stream);

/*
 * Block scores (section 4.4 eq 33-34, appendix A.2). PISA scores a candidate
 * by the log-sum-exp of its m valid child logits z_1..z_m (eq 21). Expanding
 * that LSE about the mean zbar gives log m + zbar + Var(z) / 2 + ...;
 * dropping log m and truncating after the first or the second term gives the
 * two ablations of section 4.4, which share PISA's hierarchy, forced set,
 * expansion rule and grouped-query sum (eq 22) and change only the score:
 *   PISA_SCORE_MEAN     (PISA-1): s = zbar = (1/m) sum_j z_j
 *   PISA_SCORE_MEAN_VAR (PISA-2): s = zbar + (1/(2m)) sum_j (z_j - zbar)^2
 * with z_j = q . kbar_j / sqrt(d) over the existing children (raw keys for a
 * leaf, only the keys present in a partial leaf).
 */
typedef enum pisa_score_kind {
    PISA_SCORE_LSE = 0,
    PISA_SCORE_MEAN = 1,
    PISA_SCORE_MEAN_VAR = 2
} pisa_score_kind;

/* pisa_route_prefill with the block score chosen by score_kind (a
 * pisa_score_kind); pisa_route_prefill is this call with PISA_SCORE_LSE.
 * Score outputs hold the chosen score. PISA_SCORE_MEAN and
 * PISA_SCORE_MEAN_VAR need mode PISA_ROUTE_LEVELS or PISA_ROUTE_FUSED
 * (PISA_EUNSUPPORTED for PISA_ROUTE_TWO_STAGE); an unknown score_kind is
 * PISA_EINVAL. Everything else as in pisa_route_prefill. */
pisa_status pisa_route_prefill_scored(const pisa_pyramid* p, const void* Q, const void* K,
                                      int32_t dt, int64_t N, int32_t H_q, int32_t K_top,
                                      int32_t causal, int32_t gqa_group, int32_t mode,
                                      int32_t score_kind, int32_t* idx, float* score, void* ws,
                                      size_t ws_bytes, void* stream);

/*
 * Decode routing (section 3.3, "Decoding"): the single-program selector that
 * continues from the top level down to the leaves, for the newest token of
 * each sequence (position seqlen[b] - 1, sequence length seqlen[b]), causal,
 * with the same rules as pisa_route_prefill.
 * q: device [B][H_q][d]; K: device [B][N_cap][H_kv][d]; seqlen: device int64 [B].
 * idx: device int32 [B][H_kv][K_top]; score: device float32 [B][H_kv][K_top] or NULL.
 */
pisa_status pisa_route_decode(const pisa_pyramid* p, const void* q, const void* K,
                              int32_t dt, const int64_t* seqlen, int32_t H_q, int32_t K_top,
                              int32_t gqa_group, int32_t* idx, float* score, void* stream);

/* pisa_route_decode with the block score chosen by score_kind (a
 * pisa_score_kind, section 4.4); pisa_route_decode is this call with
 * PISA_SCORE_LSE. An unknown score_kind is PISA_EINVAL. */
pisa_status pisa_route_decode_scored(const pisa_pyramid* p, const void* q, const void* K,
                                     int32_t dt, const int64_t* seqlen, int32_t H_q,
                                     int32_t K_top, int32_t gqa_group, int32_t score_kind,
                                     int32_t* idx, float* score, void* stream);

/*
 * Block-sparse attention forward (section 3.1 eq 6). Query row r of sequence
 * b sits at position kv_len[b] - N_q + r (kv_len NULL: every sequence has
 * N_kv keys, so row r is position r when N_q = N_kv). It attends to the keys
 * j < kv_len[b] of the blocks listed for its KV head, and under causal
 * masking only to j <= its position (appendix B).
 * Q: device [B][N_q][H_q][d]; K, V: device [B][N_alloc][H_kv][d];
 * block_idx: device int32 [B][H_kv][N_q][K_top], -1 entries ignored, ids
 * distinct per row; O: device [B][N_q][H_q][d], dtype dt;
 * lse: device float32 [B][H_q][N_q] (natural-log normaliser) or NULL.
 * A row with no visible key gets O = 0 and lse = -inf.
 * fp32 softmax statistics and accumulation.
 */
pisa_status pisa_sparse_attn(const void* Q, const void* K, const void* V, int32_t dt,
                             int32_t B, int64_t N_q, int64_t N_kv, int64_t N_alloc, int32_t H_q,
                             int32_t H_kv, int32_t d, int32_t C, const int32_t* block_idx,
                             int32_t K_top, int32_t causal, const int64_t* kv_len, void* O,
                             float* lse, void* stream);

/*
 * Block-sparse attention forward for many query rows (prefill), clustered by
 * selected block: same arguments, layouts and results as pisa_sparse_attn
 * (section 3.1 eq 6, appendix B masking), computed as one partial softmax per
 * (row, selected block) -- each block's keys and values read once per chunk
 * of up to 256 rows that selected it -- merged per row with the partials'
 * log-sum-exp weights (the softmax factorisation over disjoint key sets).
 * Partial outputs are stored in fp16 scaled by a power of two (11
 * significant bits) before the merge.
 * ws: device workspace of at least pisa_sparse_attn_workspace() bytes,
 * 256-byte aligned, owned by the caller, contents on entry ignored; calls
 * sharing a workspace must not overlap.
 * Supported: dt = PISA_BF16, d in {64, 128}, C in {16, 32, 64}, G_Q in
 * {1, 2, 4, 8, 16}, K_top <= 64, N_q < 2^25.
 * Errors: PISA_EINVAL, PISA_EUNSUPPORTED, PISA_ENOSPACE (ws too small), PISA_EHIP.
 */
pisa_status pisa_sparse_attn_workspace(int32_t B, int64_t N_q, int64_t N_alloc, int32_t H_q, int32_t H_kv,
                                       int32_t d, int32_t C, int32_t K_top, size_t* bytes);
pisa_status pisa_sparse_attn_clustered(const void* Q, const void* K, const void* V, int32_t dt,
                                       int32_t B, int64_t N_q, int64_t N_kv, int64_t N_alloc, int32_t H_q,
                                       int32_t H_kv, int32_t d, int32_t C, const int32_t* block_idx,
                                       int32_t K_top, int32_t causal, const int64_t* kv_len, void* O,
                                       float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of block-sparse attention with fixed block indices (section 3.1
 * eq 6; section 3.3: in training, gradients flow through attention on the
 * selected entries, the selection is not differentiated). With
 * z_j = q . k_j / sqrt(d) over the row's visible selected keys, p = softmax(z),
 * o = sum_j p_j v_j and the upstream gradient dO of o:
 *   dV_j += p_j dO;  dS_j = p_j (dO . v_j - dO . o);
 *   dQ = sum_j dS_j k_j / sqrt(d);  dK_j += dS_j q / sqrt(d).
 * Inputs as for pisa_sparse_attn_clustered, plus O (the forward output,
 * [B][N_q][H_q][d], dtype dt), dO (same layout and dtype) and lse (device
 * float32 [B][H_q][N_q], the forward's natural-log normaliser). Rows with no
 * visible key get dQ = 0. Outputs are device float32: dQ [B][N_q][H_q][d],
 * dK and dV [B][N_alloc][H_kv][d]; the call overwrites all of them (keys no
 * row selected get 0). dK and dV are accumulated with fp32 atomics, so their
 * last bits may differ between runs; dQ is summed in a fixed order. The
 * workspace holds an fp32 dQ per (row, selected block, query head):
 * B * N_q * H_q * K_top * d * 4 bytes plus the block clustering tables.
 * ws: device workspace of at least pisa_sparse_attn_bwd_workspace() bytes,
 * 256-byte aligned, owned by the caller, contents on entry ignored; calls
 * sharing a workspace must not overlap.
 * Supported: dt = PISA_BF16, d in {64, 128}, C in {16, 32, 64}, G_Q in
 * {1, 2, 4, 8, 16}, K_top <= 64, N_q < 2^25, B * N_q * H_q * K_top < 2^31.
 * Errors: PISA_EINVAL, PISA_EUNSUPPORTED, PISA_ENOSPACE (ws too small), PISA_EHIP.
 */
pisa_status pisa_sparse_attn_bwd_workspace(int32_t B, int64_t N_q, int64_t N_alloc, int32_t H_q,
                                           int32_t H_kv, int32_t d, int32_t C, int32_t K_top,
                                           size_t* bytes);
pisa_status pisa_sparse_attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                                 const void* dO, const float* lse, int32_t dt, int32_t B,
                                 int64_t N_q, int64_t N_kv, int64_t N_alloc, int32_t H_q,
                                 int32_t H_kv, int32_t d, int32_t C, const int32_t* block_idx,
                                 int32_t K_top, int32_t causal, const int64_t* kv_len, float* dQ,
                                 float* dK, float* dV, void* ws, size_t ws_bytes, void* stream);

/*
 * Exhaustive single-level selector in the style of BSA (section 3.1 eq 2-5),
 * the comparison point: every eligible leaf (start <= t when causal) except
 * the forced ones is scored by z = q_{t,h'} . kbar_i / sqrt(d) with the level-1
 * summaries of the pyramid; z is normalised by a softmax over those leaves
 * within each query head, and the G_Q probabilities are summed (the grouped
 * rule the page gives for its BSA baseline). Keeps the forced leaves plus the
 * best K_top - |forced| (ties to the lower index); keeps everything eligible
 * when at most K_top leaves are eligible. Q, idx and score as in
 * pisa_route_prefill; score holds the summed probability (+inf for blocks
 * kept without a score). The pyramid must hold a build over N.
 * Supported: K_top <= 16 (bf16 queries with G_Q >= 4 and K_top <= 8 take a faster kernel
 * that keeps the queries in MFMA registers). Errors: PISA_EINVAL, PISA_EUNSUPPORTED, PISA_ENOSPACE.
 */
pisa_status pisa_bsa_select(const pisa_pyramid* p, const void* Q, int32_t dt, int64_t N,
                            int32_t H_q, int32_t K_top, int32_t causal, int32_t gqa_group,
                            int32_t* idx, float* score, void* stream);

/*
 * Block-selection quality against full attention (section 4.4 eq 35-36;
 * appendix D.2 eq 55-57), causal. For row r (position r) of sequence b and KV
 * head h with query heads h', over the eligible leaf blocks B = 0..c, c = r / C:
 *   a_{h'}(B) = log sum_{t in B, t <= r} exp(q_{r,h'} . k_{t,h} / sqrt(d)),
 *   P(B) = (1/G_Q) sum_{h'} exp(a_{h'}(B)) / sum_{B'} exp(a_{h'}(B'))
 * (the block's share of full attention, averaged over the group). The
 * reference set keeps the first, previous and current blocks and the K_top - 3
 * other blocks of highest P (ties to the lower index), or every eligible block
 * when at most K_top are eligible. For the selector's blocks sel:
 *   recall = |sel cap ref| / K_top, captured = sum_{B in sel} P(B),
 *   ratio = captured / sum_{B in ref} P(B).
 * Q: device bf16 [B][N][H_q][d]; K: device bf16 [B][N][H_kv][d];
 * sel: device int32 [B][H_kv][N][K_top] (-1 entries and blocks after the row's
 * block are ignored). Outputs (device): mass float32 [B][H_kv][N][M_1] or NULL
 * (0 past the row's block), ref int32 [B][H_kv][N][K_top] or NULL (ascending,
 * -1 padded), recall, captured, ratio float32 [B][H_kv][N].
 * ws: device workspace of at least pisa_selection_quality_workspace() bytes
 * (B * H_q * N * M_1 * 4: the log masses), contents on entry ignored.
 * The full-attention masses cost O(N^2 d) per head: an evaluation tool for
 * N up to about 64K, not a selector. Supported: d in {64, 128}; C in
 * {16, 32, 64}; G_Q in {1, 2, 4, 8, 16}; 3 <= K_top <= 16.
 * Errors: PISA_EINVAL, PISA_EUNSUPPORTED, PISA_ENOSPACE, PISA_EHIP.
 */
pisa_status pisa_selection_quality_workspace(int32_t B, int64_t N, int32_t H_q, int32_t C,
                                             size_t* bytes);
pisa_status pisa_selection_quality(const void* Q, const void* K, int32_t dt, int32_t B,
                                   int64_t N, int32_t H_q, int32_t H_kv, int32_t d, int32_t C,
                                   const int32_t* sel, int32_t K_top, float* mass, int32_t* ref,
                                   float* recall, float* captured, float* ratio, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * Stage timing, for measurement. The library queues each call as one or more
 * kernel stages; a stage may run several times in one call (once per level).
 * pisa_time_stage appends a pair of caller-created hipEvent_t (passed as
 * void*) to a queue, per host thread and stage id (at most 16 pairs). Each
 * later occurrence of that stage on this thread consumes the oldest pair: it
 * records start_event on its stream just before the stage's first kernel and
 * stop_event just after its last one. The events are the caller's; the
 * library neither creates nor waits on them. NULL events clear the stage's
 * queue. pisa_time_stage_pending returns the pairs not yet consumed (-1 for
 * a bad stage id). Errors: PISA_EINVAL (stage id out of range, or only one
 * event given), PISA_ENOSPACE (queue full).
 */
typedef enum pisa_stage {
    PISA_STAGE_BUILD = 0,         /* pisa_build_pyramid: all levels */
    PISA_STAGE_APPEND = 1,        /* pisa_pyramid_append */
    PISA_STAGE_ROUTE_FUSED = 2,   /* pisa_route_prefill, PISA_ROUTE_FUSED */
    PISA_STAGE_ROUTE_DECODE = 3,  /* pisa_route_decode */
    PISA_STAGE_UPPER = 4,         /* two-stage: levels L..2 per (query, KV head);
                                     level-synchronous: clustered scoring of one level >= 2 */
    PISA_STAGE_CLUSTER = 5,       /* clear, scan and scatter of the query clusters */
    PISA_STAGE_LEAF = 6,          /* leaf scoring of the clustered (query, level-2 node) pairs */
    PISA_STAGE_FINAL = 7,         /* two-stage: final Select_K; level-synchronous: Select_K of one level */
    PISA_STAGE_ATTN = 8,          /* pisa_sparse_attn */
    PISA_STAGE_BSA = 9,           /* pisa_bsa_select */
    PISA_STAGE_ATTN_BWD = 10,     /* pisa_sparse_attn_bwd */
    PISA_STAGE_COUNT = 11
} pisa_stage;

pisa_status pisa_time_stage(int32_t stage, void* start_event, void* stop_event);
int32_t pisa_time_stage_pending(int32_t stage);

/* Static description of a status code. */
const char* pisa_status_str(pisa_status s);

/* Message of the last failed call on this host thread ("" if none). */
const char* pisa_last_error(void);

/* PISA_ABI_VERSION of the library. */
int32_t pisa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H */
