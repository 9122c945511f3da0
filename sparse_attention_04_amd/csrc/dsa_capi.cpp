// C ABI of the DSA forward path: argument validation, dispatch to the gfx950
// kernels, and the query-row tiling of the fused forward.  Every check runs
// before any launch; failures return a status and leave a message in a
// thread-local buffer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/dsa.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

dsa_status ok()
{
    g_err[0] = '\0';
    return DSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE_PTR(p)                                                              \
    do {                                                                            \
        if ((p) == nullptr) return fail(DSA_ERR_NULL, "%s: %s is NULL", fn, #p);    \
        if (!aligned16(p)) return fail(DSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)

#define OPTIONAL_PTR(p)                                                             \
    do {                                                                            \
        if ((p) != nullptr && !aligned16(p))                                        \
            return fail(DSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p);    \
    } while (0)

// Shared position checks.  Returns DSA_OK and sets *empty for B*Lq == 0.
dsa_status check_positions(const char* fn, int B, int Lq, int Lk, int q_pos0, bool* empty)
{
    if (B < 0 || Lq < 0 || Lk < 0 || q_pos0 < 0)
        return fail(DSA_ERR_SHAPE, "%s: negative size (B=%d Lq=%d Lk=%d q_pos0=%d)", fn, B, Lq, Lk, q_pos0);
    if (B > 65535)
        return fail(DSA_ERR_UNSUPPORTED, "%s: B=%d exceeds 65535", fn, B);
    *empty = (B == 0 || Lq == 0);
    if (*empty) return DSA_OK;
    if ((int64_t)q_pos0 + Lq > Lk)
        return fail(DSA_ERR_SHAPE, "%s: q_pos0 + Lq = %lld exceeds Lk = %d", fn,
                    (long long)q_pos0 + Lq, Lk);
    return DSA_OK;
}

dsa_status check_indexer(const char* fn, const void* q_idx, const float* q_scale, const void* k_idx,
                         const float* k_scale, const float* w, int n_idx_heads, int idx_dim,
                         dsa_dtype idx_dtype)
{
    REQUIRE_PTR(q_idx);
    REQUIRE_PTR(k_idx);
    REQUIRE_PTR(w);
    if (n_idx_heads < 1 || idx_dim < 1)
        return fail(DSA_ERR_SHAPE, "%s: n_idx_heads=%d idx_dim=%d must be >= 1", fn, n_idx_heads, idx_dim);
    if (idx_dtype == DSA_FP8_E4M3) {
        REQUIRE_PTR(q_scale);
        REQUIRE_PTR(k_scale);
        if (idx_dim != 128 || n_idx_heads != 64)
            return fail(DSA_ERR_UNSUPPORTED, "%s: FP8 indexer implemented for 64 heads x 128 dims, got %d x %d",
                        fn, n_idx_heads, idx_dim);
    } else if (idx_dtype == DSA_F32) {
        if (q_scale != nullptr || k_scale != nullptr)
            return fail(DSA_ERR_DTYPE, "%s: scales are only defined for FP8 inputs; pass NULL for F32", fn);
        if (idx_dim % 4 != 0 || idx_dim > 256 || n_idx_heads > 64 || n_idx_heads * idx_dim > 8192)
            return fail(DSA_ERR_UNSUPPORTED,
                        "%s: F32 indexer needs idx_dim %% 4 == 0, idx_dim <= 256, heads <= 64, heads*dim <= 8192", fn);
    } else {
        return fail(DSA_ERR_DTYPE, "%s: idx_dtype must be DSA_FP8_E4M3 or DSA_F32", fn);
    }
    return DSA_OK;
}

dsa_status check_attn(const char* fn, const void* q, const void* kv, void* out, float* lse,
                      int n_heads, int d_qk, int d_v, int k, float softmax_scale, dsa_dtype io_dtype)
{
    REQUIRE_PTR(q);
    REQUIRE_PTR(kv);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(lse);
    if (n_heads < 1 || d_qk < 1 || d_v < 1 || d_v > d_qk)
        return fail(DSA_ERR_SHAPE, "%s: need n_heads >= 1 and 1 <= d_v <= d_qk (got %d, %d, %d)", fn,
                    n_heads, d_qk, d_v);
    if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
        return fail(DSA_ERR_SHAPE, "%s: softmax_scale must be finite and > 0", fn);
    if (io_dtype == DSA_BF16) {
        if (n_heads % 16 != 0 || n_heads > 128)
            return fail(DSA_ERR_UNSUPPORTED, "%s: bf16 attention needs n_heads %% 16 == 0 and <= 128 (got %d)", fn, n_heads);
        if (!dsa::sparse_attn_bf16_supported(d_qk, d_v))
            return fail(DSA_ERR_UNSUPPORTED, "%s: bf16 attention built for (d_qk, d_v) in {(576,512),(128,128),(64,64)}, got (%d,%d)",
                        fn, d_qk, d_v);
    } else if (io_dtype == DSA_F32) {
        if (n_heads > 256 || d_qk > 1024 || k > 4096)
            return fail(DSA_ERR_UNSUPPORTED, "%s: f32 attention needs n_heads <= 256, d_qk <= 1024, k <= 4096", fn);
    } else {
        return fail(DSA_ERR_DTYPE, "%s: io_dtype must be DSA_BF16 or DSA_F32", fn);
    }
    return DSA_OK;
}

dsa_status check_k(const char* fn, int k, int Lk)
{
    if (k < 1 || k > Lk) return fail(DSA_ERR_SHAPE, "%s: k=%d must satisfy 1 <= k <= Lk=%d", fn, k, Lk);
    return DSA_OK;
}

dsa_status hip_status(const char* fn, hipError_t e)
{
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    return ok();
}

int auto_tile_rows(int B, int Lq, int Lk)
{
    const uint64_t per_row = (uint64_t)B * (uint64_t)Lk * 4u;   // bytes of scores per query row
    const uint64_t cap = 4ull << 30;
    uint64_t t = per_row ? cap / per_row : (uint64_t)Lq;
    if (t < 1) t = 1;
    if (t > (uint64_t)Lq) t = (uint64_t)Lq;
    return (int)t;
}

size_t round256(size_t x) { return (x + 255u) & ~(size_t)255u; }

// Parameters of the candidate route (dsa_select in dsa.h): sample every
// 2^kshift-th key, tau = the need-th largest sample score, lists of at most
// cap = 2k entries.  The sample is about k / 128 keys apart, so a row's need
// is about 192 sample scores: the relative spread of the number of keys that
// score >= tau is then about 1/sqrt(192), and 1.5 k sits 4.6 spreads from
// both k and 2k.
struct CandPlan {
    int kshift, need, cap, Ls, Ls_pad;
    bool applies;       // DSA_SELECT_CANDIDATES takes the problem
    bool automatic;     // DSA_SELECT_AUTO picks it
};

CandPlan cand_plan(int B, int Lq, int Lk, int k, bool fp8)
{
    CandPlan c{};
    while ((128 << (c.kshift + 1)) <= k) ++c.kshift;
    const int R = 1 << c.kshift;
    c.need = (3 * k + 2 * R - 1) / (2 * R);
    c.cap = 2 * k;
    c.Ls = ((Lk - 1) >> c.kshift) + 1;
    c.Ls_pad = (c.Ls + 3) & ~3;
    c.applies = fp8 && Lq >= 8 && k <= dsa::kSelectMaxCap / 2 && c.Ls <= dsa::kSelectMaxSample;
    // AUTO: candidates where the sample is at most 1/8 of the keys and the
    // list pass fills the GPU without splitting keys over workgroups (at least
    // 1024 blocks of 16 rows).  At L = 32768 they measured 23.39 ms per forward
    // against 23.81 ms by score tiles.
    c.automatic = c.applies && k >= 1024 && (int64_t)B * ((Lq + 15) / 16) >= 1024;
    return c;
}

// The route a call takes: 1 = score tiles, 2 = candidates, 0 = not taken
// (candidates asked for where they do not apply), -1 = unknown value.
int forward_route(int select, const CandPlan& c)
{
    switch (select) {
    case DSA_SELECT_AUTO: return c.automatic ? 2 : 1;
    case DSA_SELECT_SCORE_TILES: return 1;
    case DSA_SELECT_CANDIDATES: return c.applies ? 2 : 0;
    default: return -1;
    }
}

// Workspace of the forward for query tiles of T rows: one tile of scores,
// the selected sets of every row (the attention runs once over all rows
// after the last tile), and the attention's split partials (decided by the
// whole problem's rows, as dsa_sparse_attn decides); for the candidate
// route, per row the sample scores, tau, the list length, the flag and the
// list.
struct ForwardLayout {
    size_t scores, idx, part, sample, tau, cnt, flag, cand, ctr, total;
};

ForwardLayout forward_layout(int B, int Lq, int Lk, int k, int n_heads, int d_qk, int d_v, dsa_dtype io_dtype,
                             int T, bool idx_in_workspace = true, const CandPlan* cand = nullptr)
{
    ForwardLayout L{};
    L.scores = round256((size_t)B * (size_t)T * (size_t)Lk * sizeof(float));
    L.idx = idx_in_workspace ? round256((size_t)B * (size_t)Lq * (size_t)k * sizeof(int32_t)) : 0;
    const int ns = dsa::sparse_attn_split((int64_t)B * Lq, n_heads, d_qk, d_v, k, io_dtype == DSA_BF16);
    // the attention's split partials, or (unsplit) its row counter
    L.part = round256(ns > 1 ? dsa::sparse_attn_split_bytes((int64_t)B * Lq, n_heads, d_v, ns)
                             : dsa::sparse_attn_counter_bytes((int64_t)B * Lq, n_heads, d_qk, d_v, k,
                                                              io_dtype == DSA_BF16));
    if (cand) {
        const size_t rows = (size_t)B * (size_t)Lq;
        L.sample = round256(rows * (size_t)cand->Ls_pad * sizeof(float));
        L.tau = round256(rows * sizeof(float));
        L.cnt = round256(rows * sizeof(int32_t));
        L.flag = round256(rows * sizeof(int32_t));
        L.cand = round256(rows * (size_t)cand->cap * 2 * sizeof(uint32_t));
        L.ctr = 256;                                         // the list pass's block counter
    }
    L.total = L.scores + L.idx + L.part + L.sample + L.tau + L.cnt + L.flag + L.cand + L.ctr;
    return L;
}

dsa_status check_forward(const char* fn, const void* q_idx, const float* q_scale, const void* k_idx,
                         const float* k_scale, const float* w, int n_idx_heads, int idx_dim, dsa_dtype idx_dtype,
                         const void* q, const void* kv, int n_heads, int d_qk, int d_v, dsa_dtype io_dtype,
                         float softmax_scale, int B, int Lq, int Lk, int q_pos0, int k, const int32_t* idx_out,
                         void* out, float* lse, bool* empty)
{
    dsa_status st = check_positions(fn, B, Lq, Lk, q_pos0, empty);
    if (st != DSA_OK || *empty) return st;
    st = check_indexer(fn, q_idx, q_scale, k_idx, k_scale, w, n_idx_heads, idx_dim, idx_dtype);
    if (st != DSA_OK) return st;
    st = check_k(fn, k, Lk);
    if (st != DSA_OK) return st;
    st = check_attn(fn, q, kv, out, lse, n_heads, d_qk, d_v, k, softmax_scale, io_dtype);
    if (st != DSA_OK) return st;
    OPTIONAL_PTR(idx_out);
    return DSA_OK;
}

// The forward on checked arguments.  Score-tile route: per tile of T query
// rows the indexer scores (no masked entries written; rows that select every
// preceding token skipped) and the top-k into the selected sets of all rows.
// Candidate route: the sample scores, the thresholds, the lists and the
// selection over the whole problem, then the score tiles for the flagged rows
// only (launches whose rows are all unflagged return at once).  Then one
// attention launch over every row.  Nothing here allocates: `ws` holds
// forward_layout(..., T, idx_out == nullptr, cand or nullptr).total bytes.
dsa_status forward_run(const char* fn, const void* q_idx, const float* q_scale, const void* k_idx,
                       const float* k_scale, const float* w, int n_idx_heads, int idx_dim, dsa_dtype idx_dtype,
                       const void* q, const void* kv, int n_heads, int d_qk, int d_v, dsa_dtype io_dtype,
                       float softmax_scale, int B, int Lq, int Lk, int q_pos0, int k, int32_t* idx_out, void* out,
                       float* lse, int T, const CandPlan* cand, void* ws, hipStream_t s)
{
    const ForwardLayout L = forward_layout(B, Lq, Lk, k, n_heads, d_qk, d_v, io_dtype, T, idx_out == nullptr, cand);
    char* p = (char*)ws;
    float* ws_scores = (float*)p;
    p += L.scores;
    int32_t* idx_all = idx_out ? idx_out : (int32_t*)p;
    p += L.idx;
    float* ws_part = (float*)p;
    p += L.part;
    float* ws_sample = (float*)p;
    p += L.sample;
    float* ws_tau = (float*)p;
    p += L.tau;
    int32_t* ws_cnt = (int32_t*)p;
    p += L.cnt;
    int32_t* ws_flag = (int32_t*)p;
    p += L.flag;
    uint32_t* ws_cand = (uint32_t*)p;
    p += L.cand;
    int* ws_ctr = (int*)p;
    const int64_t idx_bstride = (int64_t)Lq * k;

    dsa::IndexerLaunch base{};
    base.q = q_idx; base.q_scale = q_scale; base.k = k_idx; base.k_scale = k_scale; base.w = w;
    base.B = B; base.Lq = Lq; base.Lk = Lk; base.q_pos0 = q_pos0;
    base.H = n_idx_heads; base.D = idx_dim; base.fp8 = (idx_dtype == DSA_FP8_E4M3);
    base.write_masked = false; base.skip_upto_k = k;
    hipError_t e = hipSuccess;

    if (cand) {
        // sample scores of the rows with t_pos + 1 > cap, every 2^kshift-th key
        dsa::IndexerLaunch sa = base;
        sa.scores = ws_sample; sa.t_begin = 0; sa.t_count = Lq;
        sa.sc_bstride = (int64_t)Lq * cand->Ls_pad; sa.sc_rstride = cand->Ls_pad;
        sa.kshift = cand->kshift; sa.skip_upto_k = cand->cap;
        if ((e = dsa::launch_indexer(sa, s)) != hipSuccess) return hip_status(fn, e);
        dsa::SelectLaunch sl{};
        sl.B = B; sl.Lq = Lq; sl.q_pos0 = q_pos0; sl.k = k;
        sl.sample = ws_sample; sl.s_rstride = cand->Ls_pad; sl.kshift = cand->kshift; sl.need = cand->need;
        sl.tau = ws_tau; sl.cand = ws_cand; sl.cand_cnt = ws_cnt; sl.cap = cand->cap;
        sl.idx = idx_all; sl.idx_bstride = idx_bstride; sl.flag = ws_flag;
        if ((e = dsa::launch_select_threshold(sl, s)) != hipSuccess) return hip_status(fn, e);
        // every key's score against tau, the lists
        dsa::IndexerLaunch fa = base;
        fa.t_begin = 0; fa.t_count = Lq;
        fa.tau = ws_tau; fa.cand = ws_cand; fa.cand_cnt = ws_cnt; fa.cap = cand->cap;
        fa.blk_ctr = ws_ctr;
        if ((e = dsa::launch_indexer(fa, s)) != hipSuccess) return hip_status(fn, e);
        if ((e = dsa::launch_select_candidates(sl, s)) != hipSuccess) return hip_status(fn, e);
    }

    for (int t0 = 0; t0 < Lq; t0 += T) {
        const int tc = (Lq - t0 < T) ? (Lq - t0) : T;
        dsa::IndexerLaunch ia = base;
        ia.scores = ws_scores; ia.t_begin = t0; ia.t_count = tc;
        ia.sc_bstride = (int64_t)T * Lk; ia.sc_rstride = Lk;
        ia.flag = cand ? ws_flag : nullptr;
        if ((e = dsa::launch_indexer(ia, s)) != hipSuccess) return hip_status(fn, e);

        dsa::TopkLaunch ta{};
        ta.scores = ws_scores; ta.idx = idx_all + (int64_t)t0 * k; ta.B = B; ta.Lq = Lq; ta.Lk = Lk;
        ta.q_pos0 = q_pos0; ta.t_begin = t0; ta.t_count = tc; ta.sc_bstride = (int64_t)T * Lk; ta.sc_rstride = Lk;
        ta.idx_bstride = idx_bstride; ta.k = k;
        ta.flag = cand ? ws_flag : nullptr;
        if ((e = dsa::launch_topk(ta, s)) != hipSuccess) return hip_status(fn, e);
    }

    dsa::AttnLaunch aa{};
    aa.q = q; aa.kv = kv; aa.idx = idx_all; aa.out = out; aa.lse = lse;
    aa.B = B; aa.Lq = Lq; aa.Lk = Lk; aa.t_begin = 0; aa.t_count = Lq; aa.idx_bstride = idx_bstride;
    aa.H = n_heads; aa.Dqk = d_qk; aa.Dv = d_v; aa.k = k; aa.scale = softmax_scale;
    aa.bf16 = (io_dtype == DSA_BF16);
    aa.nsplit = dsa::sparse_attn_split((int64_t)B * Lq, n_heads, d_qk, d_v, k, aa.bf16);
    aa.part = aa.nsplit > 1 ? ws_part : nullptr;
    if (aa.nsplit == 1 && dsa::sparse_attn_counter_bytes((int64_t)B * Lq, n_heads, d_qk, d_v, k, aa.bf16) > 0)
        aa.row_ctr = (int*)ws_part;
    return hip_status(fn, dsa::launch_sparse_attn(aa, s));
}

// The no-allocation forward's workspace: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends.  In host code
// `scratch` names a host-side stand-in, never a device address: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up on the
// first use on that device.
dsa_status scratch_address(const char* fn, void** ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(DSA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status s)
{
    switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "null pointer";
    case DSA_ERR_SHAPE: return "inconsistent sizes";
    case DSA_ERR_DTYPE: return "invalid dtype";
    case DSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSA_ERR_ALIGN: return "misaligned pointer";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* dsa_last_error(void) { return g_err; }

dsa_status dsa_indexer_scores(const void* q_idx, const float* q_scale, const void* k_idx,
                              const float* k_scale, const float* w, float* scores, int B, int Lq,
                              int Lk, int q_pos0, int n_idx_heads, int idx_dim,
                              dsa_dtype idx_dtype, void* stream)
{
    const char* fn = "dsa_indexer_scores";
    bool empty = false;
    dsa_status st = check_positions(fn, B, Lq, Lk, q_pos0, &empty);
    if (st != DSA_OK || empty) return st == DSA_OK ? ok() : st;
    st = check_indexer(fn, q_idx, q_scale, k_idx, k_scale, w, n_idx_heads, idx_dim, idx_dtype);
    if (st != DSA_OK) return st;
    REQUIRE_PTR(scores);
    dsa::IndexerLaunch a{};
    a.q = q_idx; a.q_scale = q_scale; a.k = k_idx; a.k_scale = k_scale; a.w = w; a.scores = scores;
    a.B = B; a.Lq = Lq; a.Lk = Lk; a.q_pos0 = q_pos0; a.t_begin = 0; a.t_count = Lq;
    a.sc_bstride = (int64_t)Lq * Lk; a.sc_rstride = Lk;
    a.H = n_idx_heads; a.D = idx_dim; a.fp8 = (idx_dtype == DSA_FP8_E4M3);
    a.write_masked = true; a.skip_upto_k = 0;
    return hip_status(fn, dsa::launch_indexer(a, (hipStream_t)stream));
}

dsa_status dsa_topk(const float* scores, int32_t* idx, int B, int Lq, int Lk, int q_pos0, int k,
                    void* stream)
{
    const char* fn = "dsa_topk";
    bool empty = false;
    dsa_status st = check_positions(fn, B, Lq, Lk, q_pos0, &empty);
    if (st != DSA_OK || empty) return st == DSA_OK ? ok() : st;
    REQUIRE_PTR(scores);
    REQUIRE_PTR(idx);
    st = check_k(fn, k, Lk);
    if (st != DSA_OK) return st;
    dsa::TopkLaunch a{};
    a.scores = scores; a.idx = idx; a.B = B; a.Lq = Lq; a.Lk = Lk; a.q_pos0 = q_pos0;
    a.t_begin = 0; a.t_count = Lq;
    a.sc_bstride = (int64_t)Lq * Lk; a.sc_rstride = Lk; a.idx_bstride = (int64_t)Lq * k; a.k = k;
    return hip_status(fn, dsa::launch_topk(a, (hipStream_t)stream));
}

size_t dsa_sparse_attn_workspace_size(int B, int Lq, int n_heads, int d_qk, int d_v, int k, dsa_dtype io_dtype)
{
    if (B <= 0 || Lq <= 0 || n_heads <= 0 || d_v <= 0 || k <= 0) return 0;
    const int64_t rows = (int64_t)B * Lq;
    const bool bf16 = io_dtype == DSA_BF16;
    const int ns = dsa::sparse_attn_split(rows, n_heads, d_qk, d_v, k, bf16);
    const size_t bytes = ns > 1 ? dsa::sparse_attn_split_bytes(rows, n_heads, d_v, ns)
                                : dsa::sparse_attn_counter_bytes(rows, n_heads, d_qk, d_v, k, bf16);
    return bytes ? round256(bytes) : 0;
}

dsa_status dsa_sparse_attn(const void* q, const void* kv, const int32_t* idx, void* out, float* lse,
                           int B, int Lq, int Lk, int q_pos0, int n_heads, int d_qk, int d_v, int k,
                           float softmax_scale, dsa_dtype io_dtype, void* workspace, size_t workspace_bytes,
                           void* stream)
{
    const char* fn = "dsa_sparse_attn";
    bool empty = false;
    dsa_status st = check_positions(fn, B, Lq, Lk, q_pos0, &empty);
    if (st != DSA_OK || empty) return st == DSA_OK ? ok() : st;
    REQUIRE_PTR(idx);
    if (k < 1) return fail(DSA_ERR_SHAPE, "%s: k=%d must be >= 1", fn, k);
    st = check_attn(fn, q, kv, out, lse, n_heads, d_qk, d_v, k, softmax_scale, io_dtype);
    if (st != DSA_OK) return st;
    dsa::AttnLaunch a{};
    a.q = q; a.kv = kv; a.idx = idx; a.out = out; a.lse = lse;
    a.B = B; a.Lq = Lq; a.Lk = Lk; a.t_begin = 0; a.t_count = Lq; a.idx_bstride = (int64_t)Lq * k;
    a.H = n_heads; a.Dqk = d_qk; a.Dv = d_v; a.k = k; a.scale = softmax_scale;
    a.bf16 = (io_dtype == DSA_BF16);
    // the split over the selected set (few rows) or the row counter (many)
    // runs only with a large enough workspace
    const size_t need = dsa_sparse_attn_workspace_size(B, Lq, n_heads, d_qk, d_v, k, io_dtype);
    if (need > 0 && workspace != nullptr && workspace_bytes >= need) {
        if (((uintptr_t)workspace & 255u) != 0)
            return fail(DSA_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
        a.nsplit = dsa::sparse_attn_split((int64_t)B * Lq, n_heads, d_qk, d_v, k, a.bf16);
        if (a.nsplit > 1) a.part = (float*)workspace;
        else a.row_ctr = (int*)workspace;
    }
    return hip_status(fn, dsa::launch_sparse_attn(a, (hipStream_t)stream));
}

dsa_status dsa_sparse_attn_fp8kv(const void* q, const void* kv_fp8, const int32_t* idx, void* out, float* lse,
                                 int B, int Lq, int Lk, int q_pos0, int n_heads, int k, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, void* stream)
{
    const char* fn = "dsa_sparse_attn_fp8kv";
    bool empty = false;
    dsa_status st = check_positions(fn, B, Lq, Lk, q_pos0, &empty);
    if (st != DSA_OK || empty) return st == DSA_OK ? ok() : st;
    REQUIRE_PTR(idx);
    if (k < 1) return fail(DSA_ERR_SHAPE, "%s: k=%d must be >= 1", fn, k);
    st = check_attn(fn, q, kv_fp8, out, lse, n_heads, 576, 512, k, softmax_scale, DSA_BF16);
    if (st != DSA_OK) return st;
    if (n_heads != 32 && n_heads != 64 && n_heads != 128)
        return fail(DSA_ERR_UNSUPPORTED, "%s: n_heads must be 32, 64 or 128 (got %d)", fn, n_heads);
    if (k > 2048) return fail(DSA_ERR_UNSUPPORTED, "%s: k=%d exceeds 2048", fn, k);
    dsa::AttnLaunch a{};
    a.q = q; a.kv = kv_fp8; a.idx = idx; a.out = out; a.lse = lse;
    a.B = B; a.Lq = Lq; a.Lk = Lk; a.t_begin = 0; a.t_count = Lq; a.idx_bstride = (int64_t)Lq * k;
    a.H = n_heads; a.Dqk = 576; a.Dv = 512; a.k = k; a.scale = softmax_scale;
    a.bf16 = true; a.kv_fp8 = true;
    const size_t need = dsa_sparse_attn_workspace_size(B, Lq, n_heads, 576, 512, k, DSA_BF16);
    if (need > 0 && workspace != nullptr && workspace_bytes >= need) {
        if (((uintptr_t)workspace & 255u) != 0)
            return fail(DSA_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
        a.nsplit = dsa::sparse_attn_split((int64_t)B * Lq, n_heads, 576, 512, k, true);
        if (a.nsplit > 1) a.part = (float*)workspace;     // the FP8-row kernel takes no row counter
    }
    return hip_status(fn, dsa::launch_sparse_attn(a, (hipStream_t)stream));
}

dsa_status dsa_indexer_kl(const void* q, const void* kv, const float* scores, float* kl, int B, int Lq, int Lk,
                          int q_pos0, int n_heads, int d_qk, float softmax_scale, void* stream)
{
    const char* fn = "dsa_indexer_kl";
    bool empty = false;
    dsa_status st = check_positions(fn, B, Lq, Lk, q_pos0, &empty);
    if (st != DSA_OK || empty) return st == DSA_OK ? ok() : st;
    REQUIRE_PTR(q);
    REQUIRE_PTR(kv);
    REQUIRE_PTR(scores);
    REQUIRE_PTR(kl);
    if (d_qk != 576) return fail(DSA_ERR_UNSUPPORTED, "%s: d_qk must be 576 (got %d)", fn, d_qk);
    if (n_heads != 32 && n_heads != 64 && n_heads != 128)
        return fail(DSA_ERR_UNSUPPORTED, "%s: n_heads must be 32, 64 or 128 (got %d)", fn, n_heads);
    if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
        return fail(DSA_ERR_SHAPE, "%s: softmax_scale must be finite and > 0", fn);
    dsa::KlLaunch a{};
    a.q = q; a.kv = kv; a.scores = scores; a.kl = kl; a.B = B; a.Lq = Lq; a.Lk = Lk; a.q_pos0 = q_pos0;
    a.H = n_heads; a.scale = softmax_scale;
    return hip_status(fn, dsa::launch_indexer_kl(a, (hipStream_t)stream));
}

size_t dsa_sparse_attn_bwd_workspace_size(int B, int Lq, int Lk, int n_heads, int k)
{
    if (B <= 0 || Lq <= 0 || Lk <= 0 || n_heads <= 0 || k <= 0) return 0;
    return round256(dsa::attn_bwd_workspace_bytes(B, Lq, Lk, n_heads, k));
}

dsa_status dsa_sparse_attn_bwd(const void* q, const void* kv, const int32_t* idx, const void* out,
                               const float* lse, const void* dout, float* dq, float* dkv, int B, int Lq, int Lk,
                               int q_pos0, int n_heads, int d_qk, int d_v, int k, float softmax_scale,
                               void* workspace, size_t workspace_bytes, void* stream)
{
    const char* fn = "dsa_sparse_attn_bwd";
    bool empty = false;
    dsa_status st = check_positions(fn, B, Lq, Lk, q_pos0, &empty);
    if (st != DSA_OK || empty) return st == DSA_OK ? ok() : st;
    REQUIRE_PTR(q);
    REQUIRE_PTR(kv);
    REQUIRE_PTR(idx);
    REQUIRE_PTR(out);
    REQUIRE_PTR(lse);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(dq);
    REQUIRE_PTR(dkv);
    if (d_qk != 576 || d_v != 512)
        return fail(DSA_ERR_UNSUPPORTED, "%s: built for (d_qk, d_v) = (576, 512), got (%d, %d)", fn, d_qk, d_v);
    if (n_heads != 16 && n_heads != 32 && n_heads != 64 && n_heads != 128)
        return fail(DSA_ERR_UNSUPPORTED, "%s: n_heads must be 16, 32, 64 or 128 (got %d)", fn, n_heads);
    if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "%s: k=%d outside [1, 2048]", fn, k);
    if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
        return fail(DSA_ERR_SHAPE, "%s: softmax_scale must be finite and > 0", fn);
    if ((int64_t)B * Lq * k >= ((int64_t)1 << 31) || (int64_t)B * Lk >= ((int64_t)1 << 31))
        return fail(DSA_ERR_UNSUPPORTED, "%s: B * Lq * k and B * Lk must be below 2^31", fn);
    const size_t need = dsa_sparse_attn_bwd_workspace_size(B, Lq, Lk, n_heads, k);
    if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
        return fail(DSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu at %p)", fn, need,
                    workspace_bytes, workspace);
    dsa::AttnBwdLaunch a{};
    a.q = q; a.kv = kv; a.idx = idx; a.out = out; a.lse = lse; a.dout = dout; a.dq = dq; a.dkv = dkv;
    a.workspace = workspace; a.B = B; a.Lq = Lq; a.Lk = Lk; a.H = n_heads; a.k = k; a.scale = softmax_scale;
    return hip_status(fn, dsa::launch_attn_bwd(a, (hipStream_t)stream));
}

dsa_status dsa_kv_pack_fp8(const void* kv, void* kv_fp8, int64_t n_tok, void* stream)
{
    const char* fn = "dsa_kv_pack_fp8";
    if (n_tok < 0) return fail(DSA_ERR_SHAPE, "%s: negative n_tok (%lld)", fn, (long long)n_tok);
    if (n_tok == 0) return ok();
    if (n_tok > ((int64_t)1 << 33)) return fail(DSA_ERR_UNSUPPORTED, "%s: n_tok too large", fn);
    REQUIRE_PTR(kv);
    REQUIRE_PTR(kv_fp8);
    dsa::KvPackLaunch a{};
    a.kv = kv; a.out = kv_fp8; a.n_tok = n_tok;
    return hip_status(fn, dsa::launch_kv_pack_fp8(a, (hipStream_t)stream));
}

size_t dsa_forward_workspace_size(int B, int Lq, int Lk, int k, int n_heads, int d_qk, int d_v,
                                  dsa_dtype io_dtype, int q_tile_rows, dsa_select select)
{
    if (B <= 0 || Lq <= 0 || Lk <= 0 || k <= 0 || q_tile_rows < 0) return 0;
    const CandPlan c = cand_plan(B, Lq, Lk, k, true);
    const int route = forward_route((int)select, c);
    if (route <= 0) return 0;
    const int T = q_tile_rows > 0 ? (q_tile_rows < Lq ? q_tile_rows : Lq) : auto_tile_rows(B, Lq, Lk);
    return forward_layout(B, Lq, Lk, k, n_heads, d_qk, d_v, io_dtype, T, true, route == 2 ? &c : nullptr).total;
}

dsa_status dsa_forward(const void* q_idx, const float* q_scale, const void* k_idx,
                       const float* k_scale, const float* w, int n_idx_heads, int idx_dim,
                       dsa_dtype idx_dtype, const void* q, const void* kv, int n_heads, int d_qk,
                       int d_v, dsa_dtype io_dtype, float softmax_scale, int B, int Lq, int Lk,
                       int q_pos0, int k, int32_t* idx_out, void* out, float* lse,
                       int q_tile_rows, dsa_select select, void* workspace, size_t workspace_bytes,
                       void* stream)
{
    const char* fn = "dsa_forward";
    bool empty = false;
    dsa_status st = check_forward(fn, q_idx, q_scale, k_idx, k_scale, w, n_idx_heads, idx_dim, idx_dtype, q, kv,
                                  n_heads, d_qk, d_v, io_dtype, softmax_scale, B, Lq, Lk, q_pos0, k, idx_out, out,
                                  lse, &empty);
    if (st != DSA_OK || empty) return st == DSA_OK ? ok() : st;
    if (q_tile_rows < 0) return fail(DSA_ERR_SHAPE, "%s: q_tile_rows=%d must be >= 0", fn, q_tile_rows);
    const CandPlan c = cand_plan(B, Lq, Lk, k, idx_dtype == DSA_FP8_E4M3);
    const int route = forward_route((int)select, c);
    if (route < 0) return fail(DSA_ERR_SHAPE, "%s: select=%d is not a dsa_select value", fn, (int)select);
    if (route == 0)
        return fail(DSA_ERR_UNSUPPORTED,
                    "%s: the candidate route needs FP8 indexer inputs, Lq >= 8, k <= %d and (Lk - 1) / %d + 1 <= %d "
                    "(Lq=%d, k=%d, Lk=%d)", fn, dsa::kSelectMaxCap / 2, 1 << c.kshift, dsa::kSelectMaxSample,
                    Lq, k, Lk);
    const CandPlan* cp = route == 2 ? &c : nullptr;
    const int T = q_tile_rows > 0 ? (q_tile_rows < Lq ? q_tile_rows : Lq) : auto_tile_rows(B, Lq, Lk);
    const size_t need = forward_layout(B, Lq, Lk, k, n_heads, d_qk, d_v, io_dtype, T, idx_out == nullptr, cp).total;
    if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
        return fail(DSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu at %p)",
                    fn, need, workspace_bytes, workspace);
    return forward_run(fn, q_idx, q_scale, k_idx, k_scale, w, n_idx_heads, idx_dim, idx_dtype, q, kv, n_heads,
                       d_qk, d_v, io_dtype, softmax_scale, B, Lq, Lk, q_pos0, k, idx_out, out, lse, T, cp, workspace,
                       (hipStream_t)stream);
}

dsa_status dsa_forward_noalloc(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                               const float* w, int n_idx_heads, int idx_dim, dsa_dtype idx_dtype, const void* q,
                               const void* kv, int n_heads, int d_qk, int d_v, dsa_dtype io_dtype,
                               float softmax_scale, int B, int Lq, int Lk, int q_pos0, int k, int32_t* idx_out,
                               void* out, float* lse, void* stream)
{
    const char* fn = "dsa_forward_noalloc";
    bool empty = false;
    dsa_status st = check_forward(fn, q_idx, q_scale, k_idx, k_scale, w, n_idx_heads, idx_dim, idx_dtype, q, kv,
                                  n_heads, d_qk, d_v, io_dtype, softmax_scale, B, Lq, Lk, q_pos0, k, idx_out, out,
                                  lse, &empty);
    if (st != DSA_OK || empty) return st == DSA_OK ? ok() : st;
    // the largest query tile (at most the automatic one) whose workspace fits
    // the scratch array; the result does not depend on the tile
    const bool idx_ws = idx_out == nullptr;
    const size_t cap = (size_t)DSA_NOALLOC_SCRATCH_BYTES;
    const ForwardLayout fixed = forward_layout(B, Lq, Lk, k, n_heads, d_qk, d_v, io_dtype, 0, idx_ws);
    const size_t per_row = (size_t)B * (size_t)Lk * sizeof(float);
    if (fixed.total + round256(per_row) > cap)
        return fail(DSA_ERR_UNSUPPORTED,
                    "%s: even a one-row query tile needs %zu bytes of workspace, above the %zu-byte scratch array "
                    "(pass idx_out, or use dsa_forward with a caller workspace)",
                    fn, fixed.total + round256(per_row), cap);
    int T = (int)std::min<size_t>((cap - fixed.total) / per_row, (size_t)auto_tile_rows(B, Lq, Lk));
    while (T > 1 && forward_layout(B, Lq, Lk, k, n_heads, d_qk, d_v, io_dtype, T, idx_ws).total > cap) --T;
    void* ws = nullptr;
    st = scratch_address(fn, &ws);
    if (st != DSA_OK) return st;
    return forward_run(fn, q_idx, q_scale, k_idx, k_scale, w, n_idx_heads, idx_dim, idx_dtype, q, kv, n_heads,
                       d_qk, d_v, io_dtype, softmax_scale, B, Lq, Lk, q_pos0, k, idx_out, out, lse, T, nullptr, ws,
                       (hipStream_t)stream);
}

dsa_status dsa_quantize_e4m3(const void* x, dsa_dtype x_dtype, uint8_t* codes, float* scales,
                             int64_t n_tok, int tok_len, int scale_repeat, float margin, void* stream)
{
    const char* fn = "dsa_quantize_e4m3";
    if (n_tok < 0)
        return fail(DSA_ERR_SHAPE, "%s: negative n_tok (%lld)", fn, (long long)n_tok);
    if (tok_len < 8 || tok_len > 16384 || tok_len % 8 != 0)
        return fail(DSA_ERR_UNSUPPORTED, "%s: tok_len=%d must be a multiple of 8 in [8, 16384]", fn, tok_len);
    if (scale_repeat < 1 || scale_repeat > 65536)
        return fail(DSA_ERR_SHAPE, "%s: scale_repeat=%d outside [1, 65536]", fn, scale_repeat);
    if (!(margin > 0.f) || !std::isfinite(margin))
        return fail(DSA_ERR_SHAPE, "%s: margin must be finite and > 0", fn);
    if (x_dtype != DSA_F32 && x_dtype != DSA_BF16)
        return fail(DSA_ERR_DTYPE, "%s: x must be fp32 or bf16", fn);
    if (n_tok == 0) return ok();
    if (n_tok > (int64_t)1 << 40)
        return fail(DSA_ERR_UNSUPPORTED, "%s: n_tok=%lld too large", fn, (long long)n_tok);
    REQUIRE_PTR(x);
    REQUIRE_PTR(codes);
    REQUIRE_PTR(scales);
    dsa::QuantLaunch a{};
    a.x = x; a.codes = codes; a.scales = scales; a.n_tok = n_tok; a.tok_len = tok_len;
    a.repeat = scale_repeat; a.margin = margin; a.bf16 = (x_dtype == DSA_BF16);
    return hip_status(fn, dsa::launch_quantize_e4m3(a, (hipStream_t)stream));
}

dsa_status dsa_rope_assemble(const void* nope, const void* rope, void* out, int B, int L, int heads,
                             int d_nope, int d_rope, int pos0, double rope_base, void* stream)
{
    const char* fn = "dsa_rope_assemble";
    if (B < 0 || L < 0 || heads < 1 || d_nope < 0 || pos0 < 0)
        return fail(DSA_ERR_SHAPE, "%s: bad sizes (B=%d L=%d heads=%d d_nope=%d pos0=%d)", fn, B, L, heads,
                    d_nope, pos0);
    if (d_nope % 8 != 0 || d_rope % 8 != 0 || d_rope < 8 || d_rope > 128)
        return fail(DSA_ERR_UNSUPPORTED, "%s: d_nope=%d and d_rope=%d must be multiples of 8, 8 <= d_rope <= 128",
                    fn, d_nope, d_rope);
    if (!(rope_base > 1.0) || !std::isfinite(rope_base))
        return fail(DSA_ERR_SHAPE, "%s: rope_base must be finite and > 1", fn);
    if ((int64_t)pos0 + L > ((int64_t)1 << 31) - 1)
        return fail(DSA_ERR_SHAPE, "%s: positions exceed the int range", fn);
    if ((int64_t)B * L > ((int64_t)1 << 31) - 1)
        return fail(DSA_ERR_UNSUPPORTED, "%s: B*L=%lld too large", fn, (long long)B * L);
    if ((int64_t)heads * (d_nope + d_rope) > ((int64_t)1 << 24))
        return fail(DSA_ERR_UNSUPPORTED, "%s: heads * (d_nope + d_rope) too large", fn);
    if (B == 0 || L == 0) return ok();
    if (d_nope > 0) REQUIRE_PTR(nope);
    REQUIRE_PTR(rope);
    REQUIRE_PTR(out);
    dsa::RopeLaunch a{};
    a.nope = nope; a.rope = rope; a.out = out; a.B = B; a.L = L; a.heads = heads;
    a.d_nope = d_nope; a.d_rope = d_rope; a.pos0 = pos0; a.base = rope_base;
    return hip_status(fn, dsa::launch_rope_assemble(a, (hipStream_t)stream));
}

}  // extern "C"
