// capi.hip -- the extern "C" boundary of libpisa (include/pisa.h): argument
// validation on the host, workspace layout and kernel dispatch. Nothing here
// allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "attn_bwd.hpp"
#include "quality.hpp"
#include "pisa_internal.hpp"

using namespace pisa;

namespace {

thread_local char g_err[512] = "";

// Library-owned workspace of pisa_route_prefill_noalloc, one copy per device,
// held until the process ends. In host code `scratch` only names the symbol:
// its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)PISA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Armed stage events of this host thread (pisa_time_stage): a queue of up to
// kStageSlots (start, stop) pairs per stage, consumed one per stage occurrence.
constexpr int kStageSlots = 16;
struct StageQueue {
    hipEvent_t ev[kStageSlots][2];
    int head, tail;
};
thread_local StageQueue g_stage[PISA_STAGE_COUNT] = {};

pisa_status fail(pisa_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

pisa_status hip_fail(hipError_t e, const char* what)
{
    return fail(PISA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

pisa_status ok()
{
    g_err[0] = 0;
    return PISA_OK;
}

int log2_exact(int64_t x)
{
    if (x <= 0 || (x & (x - 1))) return -1;
    int k = 0;
    while ((int64_t)1 << k < x) ++k;
    return k;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int64_t nodes_at(int64_t n, int C, int g, int l)
{
    int64_t span = C;
    for (int k = 1; k < l; ++k) span *= g;
    return (n + span - 1) / span;
}

int top_level(int64_t n, int C, int g)
{
    int l = 1;
    while (nodes_at(n, C, g, l) > 1) ++l;
    return l;
}

pisa_status plan(pisa_pyramid* p, int32_t B, int32_t H, int32_t d, int32_t C, int32_t g, int64_t N_cap)
{
    if (B < 1 || H < 1 || N_cap < 1) return fail(PISA_EINVAL, "pyramid: B, H_kv and N_cap must be positive");
    if (d != 64 && d != 128) return fail(PISA_EUNSUPPORTED, "pyramid: d=%d (supported: 64, 128)", d);
    if (C != 16 && C != 32 && C != 64) return fail(PISA_EUNSUPPORTED, "pyramid: C=%d (supported: 16, 32, 64)", C);
    if (g != 2 && g != 4 && g != 8 && g != 16)
        return fail(PISA_EUNSUPPORTED, "pyramid: g=%d (supported: 2, 4, 8, 16)", g);
    if ((int64_t)H * d > 4096) return fail(PISA_EUNSUPPORTED, "pyramid: H_kv * d = %lld > 4096", (long long)H * d);
    if (N_cap > ((int64_t)1 << 40)) return fail(PISA_EINVAL, "pyramid: N_cap too large");
    memset(p, 0, sizeof(*p));
    p->B = B; p->H_kv = H; p->d = d; p->C = C; p->g = g; p->N_cap = N_cap;
    const int L = top_level(N_cap, C, g);
    if (L > PISA_MAX_LEVELS) return fail(PISA_EINVAL, "pyramid: %d levels exceed PISA_MAX_LEVELS", L);
    p->L_cap = L;
    p->M_cap[0] = N_cap;
    int64_t o = 0;
    for (int l = 1; l <= L; ++l) {
        p->M_cap[l] = nodes_at(N_cap, C, g, l);
        p->off[l] = o;
        o += (int64_t)B * H * p->M_cap[l] * d;
        o = (o + 63) & ~(int64_t)63;
    }
    p->floats = o;
    p->buf = nullptr;
    return PISA_OK;
}

// Checks a caller-supplied descriptor's geometry against a fresh plan of it.
pisa_status check_geometry(const pisa_pyramid* p)
{
    if (!p) return fail(PISA_EINVAL, "pyramid descriptor is NULL");
    pisa_pyramid q;
    pisa_status s = plan(&q, p->B, p->H_kv, p->d, p->C, p->g, p->N_cap);
    if (s != PISA_OK) return s;
    if (q.L_cap != p->L_cap || q.floats != p->floats ||
        memcmp(q.M_cap, p->M_cap, sizeof(q.M_cap)) || memcmp(q.off, p->off, sizeof(q.off)))
        return fail(PISA_EINVAL, "pyramid descriptor was not produced by pisa_pyramid_plan");
    return PISA_OK;
}

// ... and that it carries its summary buffer (every call that queues work).
pisa_status check_pyramid(const pisa_pyramid* p)
{
    pisa_status s = check_geometry(p);
    if (s != PISA_OK) return s;
    if (!p->buf || !aligned16(p->buf)) return fail(PISA_EINVAL, "pyramid buf is NULL or not 16-byte aligned");
    return PISA_OK;
}

PyrArgs pyr_args(const pisa_pyramid* p)
{
    PyrArgs a;
    memset(&a, 0, sizeof(a));
    a.B = p->B; a.H = p->H_kv; a.d = p->d; a.C = p->C; a.g = p->g;
    a.g_log2 = log2_exact(p->g);
    a.c_log2 = log2_exact(p->C);
    a.L_cap = p->L_cap;
    a.N_cap = p->N_cap;
    memcpy(a.M_cap, p->M_cap, sizeof(a.M_cap));
    memcpy(a.off, p->off, sizeof(a.off));
    a.buf = p->buf;
    return a;
}

bool dtype_ok(int32_t dt) { return dt == PISA_F32 || dt == PISA_BF16; }

// Routing arguments shared by prefill and decode.
pisa_status check_route(const pisa_pyramid* p, int32_t dt, int32_t H_q, int32_t K_top, int32_t gqa, int causal,
                        int64_t M1)
{
    if (!dtype_ok(dt)) return fail(PISA_EINVAL, "dtype %d is not PISA_F32 or PISA_BF16", (int)dt);
    if (H_q < 1 || H_q % p->H_kv) return fail(PISA_EINVAL, "H_q=%d is not a multiple of H_kv=%d", H_q, p->H_kv);
    if (gqa != H_q / p->H_kv) return fail(PISA_EINVAL, "gqa_group=%d but H_q / H_kv = %d", gqa, H_q / p->H_kv);
    if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8 && gqa != 16)
        return fail(PISA_EUNSUPPORTED, "gqa_group=%d (supported: 1, 2, 4, 8, 16)", gqa);
    if (dt == PISA_F32 && gqa > 8) return fail(PISA_EUNSUPPORTED, "f32 routing supports gqa_group <= 8");
    if (K_top < 1 || K_top > 64) return fail(PISA_EINVAL, "K_top=%d outside [1, 64]", K_top);
    if (causal && K_top < 3)
        return fail(PISA_EINVAL, "causal routing keeps up to three forced blocks: K_top=%d < 3", K_top);
    if ((int64_t)p->g * K_top > 64 && !(K_top >= M1 && M1 <= 64))
        return fail(PISA_EUNSUPPORTED, "g * K_top = %d > 64 candidates (and K_top < leaf blocks)", p->g * K_top);
    return PISA_OK;
}

struct TwoStageLayout {
    size_t kept2, meta, u, counts, cursor, offsets, chunk_off, entries, total;
    int64_t M2, n_clusters;
};

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// Highest level with more than K_top nodes (0: no level is ranked).
int levels_top(int64_t N, int C, int g, int K_top)
{
    int lt = 0;
    for (int l = 1;; ++l) {
        const int64_t M = nodes_at(N, C, g, l);
        if (M > K_top) lt = l;
        if (M <= 1) break;
    }
    return lt;
}

struct LevelsLayout {
    size_t kept0, kept1, flags, u, u_pair, counts, offsets, chunk_off, chunk_cl, block_sums, entries, rows_hl, total;
    int64_t cnt_total, max_clusters;
    int64_t cnt_off[PISA_MAX_LEVELS + 2];
    int l_top;
};

LevelsLayout levels_layout(const pisa_pyramid* p, int64_t N, int K_top)
{
    LevelsLayout w;
    memset(&w, 0, sizeof(w));
    const int64_t items = (int64_t)p->B * p->H_kv * N;
    const int64_t BH = (int64_t)p->B * p->H_kv;
    w.l_top = levels_top(N, p->C, p->g, K_top);
    int64_t c = 0;
    for (int l = 1; l <= w.l_top; ++l) {
        w.cnt_off[l] = c;
        // clusters of level l: (query window, sequence and KV head, kept node of level l + 1)
        const int wl = pisa::cluster_win_log2(l);
        const int64_t n_win = (N + ((int64_t)1 << wl) - 1) >> wl;
        const int64_t nb = n_win * BH * nodes_at(N, p->C, p->g, l + 1);
        c += nb;
        if (nb > w.max_clusters) w.max_clusters = nb;
    }
    w.cnt_total = c;
    size_t o = 0;
    w.kept0 = o; o = al(o + (size_t)items * K_top * 4);
    w.kept1 = o; o = al(o + (size_t)items * K_top * 4);
    w.flags = o; o = al(o + (size_t)items * 8);
    w.u = o; o = al(o + (size_t)items * p->g * K_top * 4);
    // by-node scores of the second level of a dense pair (pisa::dense_pair)
    const int c_log2 = log2_exact(p->C), g_log2 = log2_exact(p->g);
    w.u_pair = o; o = al(o + (size_t)items * pisa::dense_pair_max_cols(N, c_log2, g_log2, w.l_top) * 4);
    w.counts = o; o = al(o + (size_t)2 * c * 4);  // counts, then cursors (cleared together)
    w.offsets = o; o = al(o + (size_t)(w.max_clusters + 1) * 4);
    w.chunk_off = o; o = al(o + (size_t)(w.max_clusters + 1) * 4);
    // chunks of a level: at most entries / chunk + clusters (smallest chunk: kRegChunk entries)
    w.chunk_cl = o; o = al(o + (size_t)(items * K_top / pisa::kRegChunk + w.max_clusters + 1) * 4);
    w.block_sums = o; o = al(o + (size_t)2 * (w.max_clusters / 1024 + 2) * 4);
    w.entries = o; o = al(o + (size_t)items * K_top * 4);
    // the upper levels' summaries as two bf16 terms (pisa::split_layout): 4 bytes per value
    w.rows_hl = o; o = al(o + (size_t)pisa::split_layout(N, c_log2, g_log2, w.l_top, BH, p->d, nullptr) * 2);
    w.total = o;
    return w;
}

TwoStageLayout two_stage_layout(const pisa_pyramid* p, int64_t N, int K_top)
{
    TwoStageLayout w;
    const int64_t items = (int64_t)p->B * p->H_kv * N;
    w.M2 = nodes_at(N, p->C, p->g, 2);
    w.n_clusters = (int64_t)p->B * p->H_kv * w.M2;
    size_t o = 0;
    w.kept2 = o; o = al(o + (size_t)items * K_top * 4);
    w.meta = o; o = al(o + (size_t)items * 8);
    w.u = o; o = al(o + (size_t)items * p->g * K_top * 4);
    w.counts = o; o += (size_t)w.n_clusters * 4;  // counts and cursor are zeroed as one range
    w.cursor = o; o = al(o + (size_t)w.n_clusters * 4);
    w.offsets = o; o = al(o + (size_t)(w.n_clusters + 1) * 4);
    w.chunk_off = o; o = al(o + (size_t)(w.n_clusters + 1) * 4);
    w.entries = o; o = al(o + (size_t)items * K_top * 4);
    w.total = o;
    return w;
}

}  // namespace

namespace pisa {

void stage_mark(int stage, bool stop, hipStream_t s)
{
    if (stage < 0 || stage >= PISA_STAGE_COUNT) return;
    StageQueue& q = g_stage[stage];
    if (q.head == q.tail) return;
    hipEventRecord(q.ev[q.head % kStageSlots][stop ? 1 : 0], s);
    if (stop) ++q.head;  // this pair is consumed
}

}  // namespace pisa

extern "C" {

pisa_status pisa_time_stage(int32_t stage, void* start_event, void* stop_event)
{
    if (stage < 0 || stage >= PISA_STAGE_COUNT) return fail(PISA_EINVAL, "stage id %d out of range", stage);
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(PISA_EINVAL, "pisa_time_stage needs both events or neither");
    StageQueue& q = g_stage[stage];
    if (!start_event) {
        q.head = q.tail = 0;
        return ok();
    }
    if (q.tail - q.head >= kStageSlots) return fail(PISA_ENOSPACE, "more than %d event pairs armed", kStageSlots);
    q.ev[q.tail % kStageSlots][0] = (hipEvent_t)start_event;
    q.ev[q.tail % kStageSlots][1] = (hipEvent_t)stop_event;
    ++q.tail;
    return ok();
}

int32_t pisa_time_stage_pending(int32_t stage)
{
    if (stage < 0 || stage >= PISA_STAGE_COUNT) return -1;
    return g_stage[stage].tail - g_stage[stage].head;
}

int32_t pisa_abi_version(void) { return PISA_ABI_VERSION; }

const char* pisa_status_str(pisa_status s)
{
    switch (s) {
    case PISA_OK: return "ok";
    case PISA_EINVAL: return "invalid argument";
    case PISA_EUNSUPPORTED: return "unsupported shape";
    case PISA_ENOSPACE: return "capacity or workspace too small";
    case PISA_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* pisa_last_error(void) { return g_err; }

pisa_status pisa_pyramid_plan(pisa_pyramid* p, int32_t B, int32_t H_kv, int32_t d, int32_t C, int32_t g,
                              int64_t N_cap)
{
    if (!p) return fail(PISA_EINVAL, "pyramid descriptor is NULL");
    pisa_status s = plan(p, B, H_kv, d, C, g, N_cap);
    return s == PISA_OK ? ok() : s;
}

pisa_status pisa_build_pyramid(const pisa_pyramid* p, const void* K, int32_t dt, int64_t N, void* stream)
{
    pisa_status s = check_pyramid(p);
    if (s != PISA_OK) return s;
    if (!dtype_ok(dt)) return fail(PISA_EINVAL, "dtype %d is not PISA_F32 or PISA_BF16", (int)dt);
    if (!K || !aligned16(K)) return fail(PISA_EINVAL, "K is NULL or not 16-byte aligned");
    if (N < 1) return fail(PISA_EINVAL, "N=%lld < 1", (long long)N);
    if (N > p->N_cap) return fail(PISA_ENOSPACE, "N=%lld exceeds N_cap=%lld", (long long)N, (long long)p->N_cap);
    stage_mark(PISA_STAGE_BUILD, false, (hipStream_t)stream);
    hipError_t e = launch_build(pyr_args(p), K, dt == PISA_F32 ? 0 : 1, N, (hipStream_t)stream);
    stage_mark(PISA_STAGE_BUILD, true, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "pisa_build_pyramid");
}

pisa_status pisa_pyramid_append(const pisa_pyramid* p, const void* K, int32_t dt, const int64_t* seqlen,
                                void* stream)
{
    pisa_status s = check_pyramid(p);
    if (s != PISA_OK) return s;
    if (!dtype_ok(dt)) return fail(PISA_EINVAL, "dtype %d is not PISA_F32 or PISA_BF16", (int)dt);
    if (!K || !aligned16(K)) return fail(PISA_EINVAL, "K is NULL or not 16-byte aligned");
    if (!seqlen) return fail(PISA_EINVAL, "seqlen is NULL");
    stage_mark(PISA_STAGE_APPEND, false, (hipStream_t)stream);
    hipError_t e = launch_append(pyr_args(p), K, dt == PISA_F32 ? 0 : 1, seqlen, (hipStream_t)stream);
    stage_mark(PISA_STAGE_APPEND, true, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "pisa_pyramid_append");
}

pisa_status pisa_route_prefill_workspace(const pisa_pyramid* p, int64_t N, int32_t H_q, int32_t K_top, int32_t mode,
                                         size_t* bytes)
{
    (void)H_q;
    if (!bytes) return fail(PISA_EINVAL, "NULL argument");
    pisa_status s = check_geometry(p);  /* the layouts divide by C and g and walk the levels */
    if (s != PISA_OK) return s;
    if (N < 1 || K_top < 1 || K_top > 64) return fail(PISA_EINVAL, "N or K_top out of range");
    if (N > p->N_cap) return fail(PISA_ENOSPACE, "N=%lld exceeds N_cap=%lld", (long long)N, (long long)p->N_cap);
    if (mode != PISA_ROUTE_FUSED && mode != PISA_ROUTE_TWO_STAGE && mode != PISA_ROUTE_LEVELS)
        return fail(PISA_EINVAL, "mode=%d", mode);
    if (mode == PISA_ROUTE_FUSED) *bytes = 0;
    else if (mode == PISA_ROUTE_LEVELS) *bytes = levels_layout(p, N, K_top).total;
    else *bytes = two_stage_layout(p, N, K_top).total;
    return ok();
}

pisa_status pisa_route_prefill_noalloc(const pisa_pyramid* p, const void* Q, const void* K, int32_t dt,
                                       int64_t N, int32_t H_q, int32_t K_top, int32_t causal, int32_t gqa_group,
                                       int32_t* idx, float* score, void* stream)
{
    pisa_status s = check_pyramid(p);
    if (s != PISA_OK) return s;
    if (N < 1 || K_top < 1 || K_top > 64) return fail(PISA_EINVAL, "N or K_top out of range");
    if (N > p->N_cap) return fail(PISA_ENOSPACE, "N=%lld exceeds N_cap=%lld", (long long)N, (long long)p->N_cap);
    const size_t need = levels_layout(p, N, K_top).total;
    if (need > kScratchBytes)
        return fail(PISA_ENOSPACE, "pisa_route_prefill_noalloc: %zu bytes of workspace needed, the library's "
                    "scratch holds %zu (use pisa_route_prefill with a workspace)", need, kScratchBytes);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "pisa_route_prefill_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(PISA_EUNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
    void* ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            // the current device's copy of the array (each device holds its own)
            e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
            if (e != hipSuccess) {
                g_scratch_ptr[dev] = nullptr;
                return hip_fail(e, "pisa_route_prefill_noalloc: hipGetSymbolAddress");
            }
        }
        ws = g_scratch_ptr[dev];
    }
    return pisa_route_prefill_scored(p, Q, K, dt, N, H_q, K_top, causal, gqa_group, PISA_ROUTE_LEVELS,
                                     PISA_SCORE_LSE, idx, score, ws, kScratchBytes, stream);
}

pisa_status pisa_route_prefill(const pisa_pyramid* p, const void* Q, const void* K, int32_t dt, int64_t N,
                               int32_t H_q, int32_t K_top, int32_t causal, int32_t gqa_group, int32_t mode,
                               int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream)
{
    return pisa_route_prefill_scored(p, Q, K, dt, N, H_q, K_top, causal, gqa_group, mode, PISA_SCORE_LSE, idx, score,
                                     ws, ws_bytes, stream);
}

pisa_status pisa_route_prefill_scored(const pisa_pyramid* p, const void* Q, const void* K, int32_t dt, int64_t N,
                                      int32_t H_q, int32_t K_top, int32_t causal, int32_t gqa_group, int32_t mode,
                                      int32_t score_kind, int32_t* idx, float* score, void* ws, size_t ws_bytes,
                                      void* stream)
{
    if (score_kind != PISA_SCORE_LSE && score_kind != PISA_SCORE_MEAN && score_kind != PISA_SCORE_MEAN_VAR)
        return fail(PISA_EINVAL, "score_kind=%d", score_kind);
    if (score_kind != PISA_SCORE_LSE && mode == PISA_ROUTE_TWO_STAGE)
        return fail(PISA_EUNSUPPORTED, "PISA-1 / PISA-2 scores need mode PISA_ROUTE_LEVELS or PISA_ROUTE_FUSED");
    pisa_status s = check_pyramid(p);
    if (s != PISA_OK) return s;
    if (N < 1) return fail(PISA_EINVAL, "N=%lld < 1", (long long)N);
    if (N > p->N_cap) return fail(PISA_ENOSPACE, "N=%lld exceeds N_cap=%lld", (long long)N, (long long)p->N_cap);
    s = check_route(p, dt, H_q, K_top, gqa_group, causal, nodes_at(N, p->C, p->g, 1));
    if (s != PISA_OK) return s;
    if (!Q || !K || !idx) return fail(PISA_EINVAL, "Q, K and idx must be non-NULL");
    if (!aligned16(Q) || !aligned16(K)) return fail(PISA_EINVAL, "Q and K must be 16-byte aligned");
    if (mode != PISA_ROUTE_FUSED && mode != PISA_ROUTE_TWO_STAGE && mode != PISA_ROUTE_LEVELS)
        return fail(PISA_EINVAL, "mode=%d", mode);
    const int64_t items = (int64_t)p->B * p->H_kv * N;
    if (items > ((int64_t)1 << 31) - 1) return fail(PISA_EUNSUPPORTED, "B * H_kv * N exceeds 2^31 - 1");

    RouteArgs r;
    memset(&r, 0, sizeof(r));
    r.p = pyr_args(p);
    r.Q = Q; r.K = K; r.N = N; r.seqlen = nullptr;
    r.H_q = H_q; r.G = gqa_group; r.K_top = K_top; r.causal = causal ? 1 : 0;
    r.score_kind = score_kind;
    r.idx = idx; r.score = score;
    const int dti = dt == PISA_F32 ? 0 : 1;
    hipStream_t st = (hipStream_t)stream;
    if (mode == PISA_ROUTE_FUSED) {
        stage_mark(PISA_STAGE_ROUTE_FUSED, false, st);
        hipError_t e = launch_route_query(r, dti, p->d, MODE_FUSED, st);
        stage_mark(PISA_STAGE_ROUTE_FUSED, true, st);
        return e == hipSuccess ? ok() : hip_fail(e, "pisa_route_prefill (fused)");
    }

    if (N >= ((int64_t)1 << 25)) return fail(PISA_EUNSUPPORTED, "clustered routing needs N < 2^25");
    if (mode == PISA_ROUTE_LEVELS) {
        if (K_top > 32 && levels_top(N, p->C, p->g, K_top) > 0)
            return fail(PISA_EUNSUPPORTED, "level-synchronous routing ranks at most K_top = 32 blocks");
        if (items * K_top > ((int64_t)1 << 31) - 1)
            return fail(PISA_EUNSUPPORTED, "B * H_kv * N * K_top exceeds 2^31 - 1");
        const size_t lds_leaf = (size_t)p->g * p->C * (p->d + 8) * 2 * (dt == PISA_F32 ? 2 : 1);
        const size_t lds_up = (size_t)p->g * p->g * (p->d + 8) * 2 * 2;
        if (lds_leaf > 160 * 1024 || lds_up > 160 * 1024)
            return fail(PISA_EUNSUPPORTED, "a node's rows do not fit in LDS for level-synchronous routing");
        const LevelsLayout w = levels_layout(p, N, K_top);
        if (!ws || ws_bytes < w.total)
            return fail(PISA_ENOSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, w.total);
        if (((uintptr_t)ws & 255) != 0) return fail(PISA_EINVAL, "workspace must be 256-byte aligned");
        char* base = (char*)ws;
        LevelsArgs la;
        memset(&la, 0, sizeof(la));
        la.r = r;
        la.kept[0] = (int32_t*)(base + w.kept0);
        la.kept[1] = (int32_t*)(base + w.kept1);
        la.flags = (int64_t*)(base + w.flags);
        la.u = (float*)(base + w.u);
        la.u_pair = (float*)(base + w.u_pair);
        la.counts = (int32_t*)(base + w.counts);
        la.cursor = la.counts + w.cnt_total;
        la.cnt_total = w.cnt_total;
        memcpy(la.cnt_off, w.cnt_off, sizeof(la.cnt_off));
        la.offsets = (int32_t*)(base + w.offsets);
        la.chunk_off = (int32_t*)(base + w.chunk_off);
        la.chunk_cl = (int32_t*)(base + w.chunk_cl);
        la.block_sums = (int32_t*)(base + w.block_sums);
        la.entries = (int32_t*)(base + w.entries);
        la.rows_hl = base + w.rows_hl;
        la.l_top = w.l_top;
        hipError_t e = launch_levels(la, dti, p->d, st);
        return e == hipSuccess ? ok() : hip_fail(e, "pisa_route_prefill (levels)");
    }
    if (items * K_top > ((int64_t)1 << 31) - 1) return fail(PISA_EUNSUPPORTED, "B * H_kv * N * K_top exceeds 2^31 - 1");
    const size_t lds = (size_t)p->g * p->C * (p->d + 8) * 2 * (dt == PISA_F32 ? 2 : 1);
    if (lds > 160 * 1024) return fail(PISA_EUNSUPPORTED, "g * C keys do not fit in LDS for two-stage routing");
    const TwoStageLayout w = two_stage_layout(p, N, K_top);
    if (!ws || ws_bytes < w.total)
        return fail(PISA_ENOSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, w.total);
    if (((uintptr_t)ws & 255) != 0) return fail(PISA_EINVAL, "workspace must be 256-byte aligned");
    char* base = (char*)ws;
    r.kept2 = (int32_t*)(base + w.kept2);
    r.meta = (int64_t*)(base + w.meta);
    r.counts = (int32_t*)(base + w.counts);
    r.M2 = w.M2;

    Stage2Args s2;
    memset(&s2, 0, sizeof(s2));
    s2.p = r.p; s2.Q = Q; s2.K = K; s2.N = N; s2.H_q = H_q; s2.G = gqa_group; s2.K_top = K_top;
    s2.n_clusters = w.n_clusters; s2.M2 = w.M2;
    s2.offsets = (const int32_t*)(base + w.offsets);
    s2.chunk_off = (const int32_t*)(base + w.chunk_off);
    s2.entries = (const int32_t*)(base + w.entries);
    s2.u = (float*)(base + w.u);

    FinalArgs f;
    memset(&f, 0, sizeof(f));
    f.B = p->B; f.H = p->H_kv; f.C = p->C; f.g = p->g; f.c_log2 = r.p.c_log2; f.g_log2 = r.p.g_log2;
    f.K_top = K_top; f.causal = r.causal; f.N = N;
    f.kept2 = r.kept2; f.meta = r.meta; f.u = s2.u; f.idx = idx; f.score = score;

    ScatterArgs sc;
    memset(&sc, 0, sizeof(sc));
    sc.B = p->B; sc.H = p->H_kv; sc.K_top = K_top; sc.N = N; sc.M2 = w.M2;
    sc.kept2 = r.kept2; sc.meta = r.meta; sc.offsets = s2.offsets;
    sc.cursor = (int32_t*)(base + w.cursor);
    sc.entries = (int32_t*)(base + w.entries);

    hipError_t e = launch_two_stage(r, s2, f, sc, r.counts, 2 * w.n_clusters, dti, p->d, st);
    return e == hipSuccess ? ok() : hip_fail(e, "pisa_route_prefill (two-stage)");
}

pisa_status pisa_route_decode(const pisa_pyramid* p, const void* q, const void* K, int32_t dt,
                              const int64_t* seqlen, int32_t H_q, int32_t K_top, int32_t gqa_group, int32_t* idx,
                              float* score, void* stream)
{
    return pisa_route_decode_scored(p, q, K, dt, seqlen, H_q, K_top, gqa_group, PISA_SCORE_LSE, idx, score, stream);
}

pisa_status pisa_route_decode_scored(const pisa_pyramid* p, const void* q, const void* K, int32_t dt,
                                     const int64_t* seqlen, int32_t H_q, int32_t K_top, int32_t gqa_group,
                                     int32_t score_kind, int32_t* idx, float* score, void* stream)
{
    if (score_kind != PISA_SCORE_LSE && score_kind != PISA_SCORE_MEAN && score_kind != PISA_SCORE_MEAN_VAR)
        return fail(PISA_EINVAL, "score_kind=%d", score_kind);
    pisa_status s = check_pyramid(p);
    if (s != PISA_OK) return s;
    s = check_route(p, dt, H_q, K_top, gqa_group, 1, nodes_at(p->N_cap, p->C, p->g, 1));
    if (s != PISA_OK) return s;
    if (!q || !K || !seqlen || !idx) return fail(PISA_EINVAL, "q, K, seqlen and idx must be non-NULL");
    if (!aligned16(q) || !aligned16(K)) return fail(PISA_EINVAL, "q and K must be 16-byte aligned");
    RouteArgs r;
    memset(&r, 0, sizeof(r));
    r.p = pyr_args(p);
    r.Q = q; r.K = K; r.N = 0; r.seqlen = seqlen;
    r.H_q = H_q; r.G = gqa_group; r.K_top = K_top; r.causal = 1;
    r.score_kind = score_kind;
    r.idx = idx; r.score = score;
    stage_mark(PISA_STAGE_ROUTE_DECODE, false, (hipStream_t)stream);
    hipError_t e = launch_route_query(r, dt == PISA_F32 ? 0 : 1, p->d, MODE_DECODE, (hipStream_t)stream);
    stage_mark(PISA_STAGE_ROUTE_DECODE, true, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "pisa_route_decode");
}

pisa_status pisa_sparse_attn(const void* Q, const void* K, const void* V, int32_t dt, int32_t B, int64_t N_q,
                             int64_t N_kv, int64_t N_alloc, int32_t H_q, int32_t H_kv, int32_t d, int32_t C,
                             const int32_t* block_idx, int32_t K_top, int32_t causal, const int64_t* kv_len, void* O,
                             float* lse, void* stream)
{
    if (!dtype_ok(dt)) return fail(PISA_EINVAL, "dtype %d is not PISA_F32 or PISA_BF16", (int)dt);
    if (!Q || !K || !V || !block_idx || !O) return fail(PISA_EINVAL, "Q, K, V, block_idx and O must be non-NULL");
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
        return fail(PISA_EINVAL, "Q, K, V and O must be 16-byte aligned");
    if (B < 1 || N_q < 1 || N_kv < 1 || N_alloc < N_kv || N_q > N_kv)
        return fail(PISA_EINVAL, "need B >= 1, 1 <= N_q <= N_kv <= N_alloc");
    if (H_kv < 1 || H_q < 1 || H_q % H_kv) return fail(PISA_EINVAL, "H_q must be a positive multiple of H_kv");
    const int G = H_q / H_kv;
    if (d != 64 && d != 128) return fail(PISA_EUNSUPPORTED, "d=%d (supported: 64, 128)", d);
    if (C != 16 && C != 32 && C != 64) return fail(PISA_EUNSUPPORTED, "C=%d (supported: 16, 32, 64)", C);
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return fail(PISA_EUNSUPPORTED, "G_Q=%d", G);
    if (dt == PISA_F32 && G > 8) return fail(PISA_EUNSUPPORTED, "f32 attention supports G_Q <= 8");
    if (K_top < 1 || K_top > 1024) return fail(PISA_EINVAL, "K_top=%d outside [1, 1024]", K_top);
    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.Q = Q; a.K = K; a.V = V; a.B = B; a.H_q = H_q; a.H_kv = H_kv; a.G = G; a.C = C; a.K_top = K_top;
    a.causal = causal ? 1 : 0; a.N_q = N_q; a.N_kv = N_kv; a.N_alloc = N_alloc; a.idx = block_idx;
    a.kv_len = kv_len; a.O = O; a.lse = lse;
    stage_mark(PISA_STAGE_ATTN, false, (hipStream_t)stream);
    hipError_t e = launch_attn(a, dt == PISA_F32 ? 0 : 1, d, (hipStream_t)stream);
    stage_mark(PISA_STAGE_ATTN, true, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "pisa_sparse_attn");
}

static pisa_status check_attn_cl(int32_t B, int64_t N_q, int64_t N_alloc, int32_t H_q, int32_t H_kv, int32_t d,
                                 int32_t C, int32_t K_top)
{
    if (B < 1 || N_q < 1 || N_alloc < 1) return fail(PISA_EINVAL, "need B >= 1, N_q >= 1, N_alloc >= 1");
    if (H_kv < 1 || H_q < 1 || H_q % H_kv) return fail(PISA_EINVAL, "H_q must be a positive multiple of H_kv");
    const int G = H_q / H_kv;
    if (d != 64 && d != 128) return fail(PISA_EUNSUPPORTED, "d=%d (supported: 64, 128)", d);
    if (C != 16 && C != 32 && C != 64) return fail(PISA_EUNSUPPORTED, "C=%d (supported: 16, 32, 64)", C);
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return fail(PISA_EUNSUPPORTED, "G_Q=%d", G);
    if (K_top < 1 || K_top > 64) return fail(PISA_EUNSUPPORTED, "clustered attention: K_top=%d outside [1, 64]", K_top);
    if (N_q >= ((int64_t)1 << 25)) return fail(PISA_EUNSUPPORTED, "clustered attention needs N_q < 2^25");
    return PISA_OK;
}

pisa_status pisa_sparse_attn_workspace(int32_t B, int64_t N_q, int64_t N_alloc, int32_t H_q, int32_t H_kv, int32_t d,
                                       int32_t C, int32_t K_top, size_t* bytes)
{
    if (!bytes) return fail(PISA_EINVAL, "bytes must be non-NULL");
    pisa_status st = check_attn_cl(B, N_q, N_alloc, H_q, H_kv, d, C, K_top);
    if (st != PISA_OK) return st;
    *bytes = attn_cl_layout(B, N_q, N_alloc, H_kv, H_q / H_kv, d, C, K_top).bytes;
    return ok();
}

pisa_status pisa_sparse_attn_clustered(const void* Q, const void* K, const void* V, int32_t dt, int32_t B,
                                       int64_t N_q, int64_t N_kv, int64_t N_alloc, int32_t H_q, int32_t H_kv,
                                       int32_t d, int32_t C, const int32_t* block_idx, int32_t K_top, int32_t causal,
                                       const int64_t* kv_len, void* O, float* lse, void* ws, size_t ws_bytes,
                                       void* stream)
{
    if (!dtype_ok(dt)) return fail(PISA_EINVAL, "dtype %d is not PISA_F32 or PISA_BF16", (int)dt);
    if (dt != PISA_BF16) return fail(PISA_EUNSUPPORTED, "clustered attention takes bf16 inputs");
    if (!Q || !K || !V || !block_idx || !O || !ws)
        return fail(PISA_EINVAL, "Q, K, V, block_idx, O and ws must be non-NULL");
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
        return fail(PISA_EINVAL, "Q, K, V and O must be 16-byte aligned");
    if (((uintptr_t)ws & 255) != 0) return fail(PISA_EINVAL, "ws must be 256-byte aligned");
    if (N_kv < 1 || N_alloc < N_kv || N_q > N_kv) return fail(PISA_EINVAL, "need 1 <= N_q <= N_kv <= N_alloc");
    pisa_status st = check_attn_cl(B, N_q, N_alloc, H_q, H_kv, d, C, K_top);
    if (st != PISA_OK) return st;
    const AttnClLayout L = attn_cl_layout(B, N_q, N_alloc, H_kv, H_q / H_kv, d, C, K_top);
    if (ws_bytes < L.bytes)
        return fail(PISA_ENOSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, L.bytes);
    AttnClArgs a;
    memset(&a, 0, sizeof(a));
    a.Q = Q; a.K = K; a.V = V; a.B = B; a.H_q = H_q; a.H_kv = H_kv; a.G = H_q / H_kv; a.C = C; a.K_top = K_top;
    a.causal = causal ? 1 : 0; a.N_q = N_q; a.N_kv = N_kv; a.N_alloc = N_alloc; a.idx = block_idx;
    a.kv_len = kv_len; a.O = O; a.lse = lse;
    stage_mark(PISA_STAGE_ATTN, false, (hipStream_t)stream);
    hipError_t e = launch_attn_clustered(a, d, (char*)ws, (hipStream_t)stream);
    stage_mark(PISA_STAGE_ATTN, true, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "pisa_sparse_attn_clustered");
}

pisa_status pisa_sparse_attn_bwd_workspace(int32_t B, int64_t N_q, int64_t N_alloc, int32_t H_q, int32_t H_kv,
                                           int32_t d, int32_t C, int32_t K_top, size_t* bytes)
{
    if (!bytes) return fail(PISA_EINVAL, "bytes must be non-NULL");
    pisa_status st = check_attn_cl(B, N_q, N_alloc, H_q, H_kv, d, C, K_top);
    if (st != PISA_OK) return st;
    *bytes = attn_bwd_layout(B, N_q, N_alloc, H_q, H_kv, d, C, K_top).bytes;
    return ok();
}

pisa_status pisa_sparse_attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                 const float* lse, int32_t dt, int32_t B, int64_t N_q, int64_t N_kv,
                                 int64_t N_alloc, int32_t H_q, int32_t H_kv, int32_t d, int32_t C,
                                 const int32_t* block_idx, int32_t K_top, int32_t causal, const int64_t* kv_len,
                                 float* dQ, float* dK, float* dV, void* ws, size_t ws_bytes, void* stream)
{
    if (!dtype_ok(dt)) return fail(PISA_EINVAL, "dtype %d is not PISA_F32 or PISA_BF16", (int)dt);
    if (dt != PISA_BF16) return fail(PISA_EUNSUPPORTED, "attention backward takes bf16 inputs");
    if (!Q || !K || !V || !O || !dO || !lse || !block_idx || !dQ || !dK || !dV || !ws)
        return fail(PISA_EINVAL, "Q, K, V, O, dO, lse, block_idx, dQ, dK, dV and ws must be non-NULL");
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(dQ) ||
        !aligned16(dK) || !aligned16(dV))
        return fail(PISA_EINVAL, "Q, K, V, O, dO, dQ, dK and dV must be 16-byte aligned");
    if (((uintptr_t)ws & 255) != 0) return fail(PISA_EINVAL, "ws must be 256-byte aligned");
    if (N_kv < 1 || N_alloc < N_kv || N_q > N_kv) return fail(PISA_EINVAL, "need 1 <= N_q <= N_kv <= N_alloc");
    pisa_status st = check_attn_cl(B, N_q, N_alloc, H_q, H_kv, d, C, K_top);
    if (st != PISA_OK) return st;
    if ((int64_t)B * N_q * H_q * K_top >= ((int64_t)1 << 31))
        return fail(PISA_EUNSUPPORTED, "B * N_q * H_q * K_top >= 2^31");
    const AttnBwdLayout L = attn_bwd_layout(B, N_q, N_alloc, H_q, H_kv, d, C, K_top);
    if (ws_bytes < L.bytes) return fail(PISA_ENOSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, L.bytes);
    AttnBwdArgs a;
    memset(&a, 0, sizeof(a));
    AttnClArgs& c = a.c;
    c.Q = Q; c.K = K; c.V = V; c.B = B; c.H_q = H_q; c.H_kv = H_kv; c.G = H_q / H_kv; c.C = C; c.K_top = K_top;
    c.causal = causal ? 1 : 0; c.N_q = N_q; c.N_kv = N_kv; c.N_alloc = N_alloc; c.idx = block_idx; c.kv_len = kv_len;
    a.O = O; a.dO = dO; a.lse = lse; a.dQ = dQ; a.dK = dK; a.dV = dV;
    stage_mark(PISA_STAGE_ATTN_BWD, false, (hipStream_t)stream);
    hipError_t e = launch_attn_bwd(a, d, (char*)ws, (hipStream_t)stream);
    stage_mark(PISA_STAGE_ATTN_BWD, true, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "pisa_sparse_attn_bwd");
}

static pisa_status check_quality(int32_t B, int64_t N, int32_t H_q, int32_t C)
{
    if (B < 1 || N < 1 || H_q < 1) return fail(PISA_EINVAL, "need B, N, H_q >= 1");
    if (C != 16 && C != 32 && C != 64) return fail(PISA_EUNSUPPORTED, "C=%d (supported: 16, 32, 64)", C);
    if (N > ((int64_t)1 << 20)) return fail(PISA_EUNSUPPORTED, "selection quality needs N <= 2^20");
    return PISA_OK;
}

pisa_status pisa_selection_quality_workspace(int32_t B, int64_t N, int32_t H_q, int32_t C, size_t* bytes)
{
    if (!bytes) return fail(PISA_EINVAL, "bytes must be non-NULL");
    pisa_status st = check_quality(B, N, H_q, C);
    if (st != PISA_OK) return st;
    *bytes = quality_workspace_bytes(B, N, H_q, C);
    return ok();
}

pisa_status pisa_selection_quality(const void* Q, const void* K, int32_t dt, int32_t B, int64_t N, int32_t H_q,
                                   int32_t H_kv, int32_t d, int32_t C, const int32_t* sel, int32_t K_top, float* mass,
                                   int32_t* ref, float* recall, float* captured, float* ratio, void* ws,
                                   size_t ws_bytes, void* stream)
{
    if (!dtype_ok(dt)) return fail(PISA_EINVAL, "dtype %d is not PISA_F32 or PISA_BF16", (int)dt);
    if (dt != PISA_BF16) return fail(PISA_EUNSUPPORTED, "selection quality takes bf16 inputs");
    pisa_status st = check_quality(B, N, H_q, C);
    if (st != PISA_OK) return st;
    if (H_kv < 1 || H_q % H_kv) return fail(PISA_EINVAL, "H_q must be a positive multiple of H_kv");
    const int G = H_q / H_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return fail(PISA_EUNSUPPORTED, "G_Q=%d", G);
    if (d != 64 && d != 128) return fail(PISA_EUNSUPPORTED, "d=%d (supported: 64, 128)", d);
    if (K_top < 3) return fail(PISA_EINVAL, "K_top=%d < 3 (the forced blocks)", K_top);
    if (K_top > 16) return fail(PISA_EUNSUPPORTED, "selection quality supports K_top <= 16");
    if (!Q || !K || !sel || !recall || !captured || !ratio || !ws)
        return fail(PISA_EINVAL, "Q, K, sel, recall, captured, ratio and ws must be non-NULL");
    if (!aligned16(Q) || !aligned16(K)) return fail(PISA_EINVAL, "Q and K must be 16-byte aligned");
    const size_t need = quality_workspace_bytes(B, N, H_q, C);
    if (ws_bytes < need) return fail(PISA_ENOSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
    if (((uintptr_t)ws & 15) != 0) return fail(PISA_EINVAL, "ws must be 16-byte aligned");
    QualArgs a;
    memset(&a, 0, sizeof(a));
    a.Q = Q; a.K = K; a.B = B; a.H_q = H_q; a.H_kv = H_kv; a.G = G; a.C = C; a.K_top = K_top;
    a.N = N; a.M1 = (N + C - 1) / C; a.sel = sel; a.lmass = (float*)ws; a.mass = mass; a.ref = ref;
    a.recall = recall; a.captured = captured; a.ratio = ratio;
    hipError_t e = launch_quality(a, d, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "pisa_selection_quality");
}

pisa_status pisa_bsa_select(const pisa_pyramid* p, const void* Q, int32_t dt, int64_t N, int32_t H_q,
                            int32_t K_top, int32_t causal, int32_t gqa_group, int32_t* idx, float* score,
                            void* stream)
{
    pisa_status s = check_pyramid(p);
    if (s != PISA_OK) return s;
    if (N < 1) return fail(PISA_EINVAL, "N=%lld < 1", (long long)N);
    if (N > p->N_cap) return fail(PISA_ENOSPACE, "N=%lld exceeds N_cap=%lld", (long long)N, (long long)p->N_cap);
    if (!dtype_ok(dt)) return fail(PISA_EINVAL, "dtype %d is not PISA_F32 or PISA_BF16", (int)dt);
    if (H_q < 1 || H_q % p->H_kv) return fail(PISA_EINVAL, "H_q=%d is not a multiple of H_kv=%d", H_q, p->H_kv);
    if (gqa_group != H_q / p->H_kv) return fail(PISA_EINVAL, "gqa_group does not equal H_q / H_kv");
    const int G = gqa_group;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return fail(PISA_EUNSUPPORTED, "gqa_group=%d", G);
    if (dt == PISA_F32 && G > 8) return fail(PISA_EUNSUPPORTED, "f32 selection supports gqa_group <= 8");
    if (K_top < 1) return fail(PISA_EINVAL, "K_top=%d < 1", K_top);
    if (K_top > 16) return fail(PISA_EUNSUPPORTED, "exhaustive selector supports K_top <= 16");
    if (causal && K_top < 3) return fail(PISA_EINVAL, "causal selection needs K_top >= 3");
    if (!Q || !idx || !aligned16(Q)) return fail(PISA_EINVAL, "Q and idx must be non-NULL, Q 16-byte aligned");
    BsaArgs a;
    memset(&a, 0, sizeof(a));
    a.p = pyr_args(p); a.Q = Q; a.N = N; a.H_q = H_q; a.G = G; a.K_top = K_top; a.causal = causal ? 1 : 0;
    a.idx = idx; a.score = score;
    stage_mark(PISA_STAGE_BSA, false, (hipStream_t)stream);
    hipError_t e = launch_bsa(a, dt == PISA_F32 ? 0 : 1, p->d, (hipStream_t)stream);
    stage_mark(PISA_STAGE_BSA, true, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "pisa_bsa_select");
}

}  // extern "C"
