// Host-side launch descriptors shared by the C ABI (dsa_capi.cpp) and the
// kernel files.  All row addressing is relative to a tile of query rows
// [t_begin, t_begin + t_count) of every batch entry.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

struct IndexerLaunch {
    const void* q;          // [B,Lq,H,D] fp8 codes or fp32
    const float* q_scale;   // [B,Lq,H] (fp8 only)
    const void* k;          // [B,Lk,D]
    const float* k_scale;   // [B,Lk] (fp8 only)
    const float* w;         // [B,Lq,H]
    float* scores;          // row (b, t) at scores + b*sc_bstride + (t - t_begin)*sc_rstride
    int B, Lq, Lk, q_pos0;
    int t_begin, t_count;
    int64_t sc_bstride, sc_rstride;
    int H, D;
    bool fp8;
    bool write_masked;      // write -inf for t_pos < s < Lk
    int skip_upto_k;        // > 0: skip query blocks whose rows all have t_pos + 1 <= this
    // FP8 block kernel only (B * Lq rows indexed b * Lq + t):
    int kshift = 0;         // > 0: sample pass over keys s = j << kshift; score column j, j <= t_pos >> kshift
    const int32_t* flag = nullptr;   // non-null: only query blocks holding a row with flag != 0 run
    // Candidate pass (tau non-null; no scores stored, keys not split over
    // workgroups): the keys of row (b, t) with score >= tau[row] are appended,
    // in ascending s, to cand + 2 * row * cap as (score bits, s) pairs, the
    // first cap of them stored; cand_cnt[row] gets their number.
    const float* tau = nullptr;
    uint32_t* cand = nullptr;
    int32_t* cand_cnt = nullptr;
    int cap = 0;
    // FP8 block kernel, keys not split over workgroups: a device counter
    // (cleared by the launch) from which workgroups take their row blocks,
    // longest first; null: one workgroup per row block, fixed
    int* blk_ctr = nullptr;
};

struct TopkLaunch {
    const float* scores;    // as IndexerLaunch::scores
    int32_t* idx;           // row (b, t) at idx + b*idx_bstride + (t - t_begin)*k
    int B, Lq, Lk, q_pos0;
    int t_begin, t_count;
    int64_t sc_bstride, sc_rstride, idx_bstride;
    int k;
    const int32_t* flag = nullptr;   // non-null: only rows with flag[b * Lq + t] != 0 run
};

// Selection over per-row candidate lists (select.hip), rows [0, Lq) of every
// batch entry, row (b, t) at index b * Lq + t.
struct SelectLaunch {
    int B, Lq, q_pos0, k;
    // thresholds: rows with t_pos + 1 <= cap get tau = -inf (every key is a
    // candidate); the others the need-th largest of their (t_pos >> kshift) + 1
    // sample scores, row (b, t) at sample + (b * Lq + t) * s_rstride
    const float* sample;
    int64_t s_rstride;
    int kshift, need;
    float* tau;
    // selection: the k entries of the row's list with the largest scores
    // (lowest s among equal scores), written in ascending s to
    // idx + b * idx_bstride + t * k; flag[row] = 1 when the list cannot
    // hold them (fewer than k entries, or more than cap), else 0
    const uint32_t* cand;
    const int32_t* cand_cnt;
    int cap;
    int32_t* idx;
    int64_t idx_bstride;
    int32_t* flag;
};

struct AttnLaunch {
    const void* q;          // [B,Lq,H,Dqk]
    const void* kv;         // [B,Lk,Dqk]
    const int32_t* idx;     // as TopkLaunch::idx
    void* out;              // [B,Lq,H,Dv]
    float* lse;             // [B,Lq,H] or null
    int B, Lq, Lk;
    int t_begin, t_count;
    int64_t idx_bstride;
    int H, Dqk, Dv, k;
    float scale;
    bool bf16;
    bool kv_fp8;            // kv holds 656-byte FP8 rows (576/512 rows, 32-head kernel only)
    int nsplit;             // > 1: split each row's selected set (32-head kernel only)
    float* part;            // split partials, sparse_attn_split_bytes(B * t_count, H, Dv, nsplit) bytes
    int* row_ctr = nullptr; // unsplit 576/512 rows: a device counter (zeroed by the launch) from which
                            // workgroups take their rows in turn; null: one workgroup per row, fixed
};

struct QuantLaunch {
    const void* x;          // [n_tok, tok_len] fp32 or bf16
    uint8_t* codes;         // [n_tok, tok_len] e4m3
    float* scales;          // [n_tok, repeat]
    int64_t n_tok;
    int tok_len, repeat;    // tok_len % 8 == 0, tok_len <= 16384
    float margin;
    bool bf16;
};

struct AttnBwdLaunch {
    const void* q;          // [B, Lq, H, 576] bf16
    const void* kv;         // [B, Lk, 576] bf16
    const int32_t* idx;     // [B, Lq, k]
    const void* out;        // [B, Lq, H, 512] bf16 (forward output)
    const float* lse;       // [B, Lq, H] (forward log-sum-exp, natural log)
    const void* dout;       // [B, Lq, H, 512] bf16
    float* dq;              // [B, Lq, H, 576]
    float* dkv;             // [B, Lk, 576]
    void* workspace;        // attn_bwd_workspace_bytes(B, Lq, Lk, H, k)
    int B, Lq, Lk, H, k;
    float scale;
};

struct KlLaunch {
    const void* q;          // [B, Lq, H, 576] bf16
    const void* kv;         // [B, Lk, 576] bf16
    const float* scores;    // [B, Lq, Lk] indexer scores (s <= t_pos read)
    float* kl;              // [B, Lq]
    int B, Lq, Lk, q_pos0, H;
    float scale;
};

struct KvPackLaunch {
    const void* kv;         // [n_tok, 576] bf16
    void* out;              // [n_tok, 656] packed FP8 rows
    int64_t n_tok;
};

struct RopeLaunch {
    const void* nope;       // [B, L, heads, d_nope] bf16
    const void* rope;       // [B, L, heads, d_rope] bf16
    void* out;              // [B, L, heads, d_nope + d_rope] bf16
    int B, L, heads, d_nope, d_rope, pos0;
    double base;
};

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t s);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t s);
hipError_t launch_select_threshold(const SelectLaunch& a, hipStream_t s);
hipError_t launch_select_candidates(const SelectLaunch& a, hipStream_t s);
// largest sample row and list the selection kernels take
constexpr int kSelectMaxSample = 8192;
constexpr int kSelectMaxCap = 4096;
hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s);
// bf16 576/512 rows, 32/64/128 heads, k <= 2048 (attn_mla.hip): ns splits
// of cps chunks each (ns > 1: partials to part_o / part_lse for the merge)
hipError_t launch_sparse_attn_mla(const AttnLaunch& a, hipStream_t s, int ns, int cps, float* part_o,
                                  float* part_lse);
// bf16 rows of D = d_qk = d_v in {64, 128}, H / 16 waves (1, 2, 4 or 8 and
// dividing D / 16), k <= 2048, rows addressable by 32-bit byte offsets
// (attn_mqa.hip)
bool sparse_attn_mqa_supported(int H, int D, int k, int Lk);
hipError_t launch_sparse_attn_mqa(const AttnLaunch& a, hipStream_t s);
hipError_t launch_quantize_e4m3(const QuantLaunch& a, hipStream_t s);
hipError_t launch_rope_assemble(const RopeLaunch& a, hipStream_t s);
hipError_t launch_kv_pack_fp8(const KvPackLaunch& a, hipStream_t s);
hipError_t launch_indexer_kl(const KlLaunch& a, hipStream_t s);
hipError_t launch_attn_bwd(const AttnBwdLaunch& a, hipStream_t s);
size_t attn_bwd_workspace_bytes(int B, int Lq, int Lk, int H, int k);

// Split factor for the selected set when few query rows are attended (1 = no
// split), and the bytes of partial results it needs.
int sparse_attn_split(int64_t rows, int H, int Dqk, int Dv, int k, bool bf16);
size_t sparse_attn_split_bytes(int64_t rows, int H, int Dv, int nsplit);
// Bytes of the row counter the unsplit 576/512 kernel takes its rows from
// (0 where that kernel does not run unsplit).
size_t sparse_attn_counter_bytes(int64_t rows, int H, int Dqk, int Dv, int k, bool bf16);

// Which (Dqk, Dv) pairs the bf16 attention kernel is instantiated for.
bool sparse_attn_bf16_supported(int Dqk, int Dv);

}  // namespace dsa
