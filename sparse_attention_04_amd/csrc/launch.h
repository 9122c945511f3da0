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
};

struct TopkLaunch {
    const float* scores;    // as IndexerLaunch::scores
    int32_t* idx;           // row (b, t) at idx + b*idx_bstride + (t - t_begin)*k
    int B, Lq, Lk, q_pos0;
    int t_begin, t_count;
    int64_t sc_bstride, sc_rstride, idx_bstride;
    int k;
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
    void* workspace;        // attn_bwd_workspace_bytes(B, Lq, H, k)
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
hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s);
hipError_t launch_quantize_e4m3(const QuantLaunch& a, hipStream_t s);
hipError_t launch_rope_assemble(const RopeLaunch& a, hipStream_t s);
hipError_t launch_kv_pack_fp8(const KvPackLaunch& a, hipStream_t s);
hipError_t launch_indexer_kl(const KlLaunch& a, hipStream_t s);
hipError_t launch_attn_bwd(const AttnBwdLaunch& a, hipStream_t s);
// MFMA issue-rate probe (measurement only): kind 0 = FP8 16x16x128, 1 = BF16
// 32x32x16; n_cu * waves_per_simd workgroups of four waves; sink holds one
// float per wave.
hipError_t launch_mfma_probe(int kind, int waves_per_simd, int iters, int n_cu, float* sink, hipStream_t s);
int mfma_probe_mfmas_per_iter(int kind);
double mfma_probe_flop_per_mfma(int kind);
size_t attn_bwd_workspace_bytes(int B, int Lq, int H, int k);

// Split factor for the selected set when few query rows are attended (1 = no
// split), and the bytes of partial results it needs.
int sparse_attn_split(int64_t rows, int H, int Dqk, int Dv, int k, bool bf16);
size_t sparse_attn_split_bytes(int64_t rows, int H, int Dv, int nsplit);

// Which (Dqk, Dv) pairs the bf16 attention kernel is instantiated for.
bool sparse_attn_bf16_supported(int Dqk, int Dv);

}  // namespace dsa
