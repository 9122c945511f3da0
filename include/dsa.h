/*
 * dsa.h — C ABI of the MI355X (gfx950) DeepSeek Sparse Attention forward path.
 *
 * The method ("DeepseekV3.2 拆解", section 核心组件):
 *   1. lightning-indexer score  I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j] . k_I[s])
 *      over the tokens s that precede query t (s <= t), computed in FP8;
 *   2. fine-grained token selection: per query, the k (= 2048) tokens with the
 *      largest I[t,:];
 *   3. attention of the query over the latent rows c_s of the selected tokens
 *      only.  All query heads share one selected set and one latent row per
 *      token (MQA over the MLA latent cache, "DeepSeek模型架构创新解析" section
 *      1.1): the key is the row's first d_qk columns, the value its first d_v.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor is a dense row-major array; the last dimension is unit-stride.
 *    Device pointers must be 16-byte aligned.  The caller owns every buffer; the
 *    library never allocates device memory except where a function says so.
 *  - Positions: query row t of a batch entry sits at absolute position
 *    t_pos = q_pos0 + t and may attend to keys 0..t_pos; q_pos0 + Lq <= Lk.
 *    Prefill is q_pos0 = 0, Lq = Lk; decode of one new token is q_pos0 = Lk-1,
 *    Lq = 1.
 *  - Outputs are fully overwritten (callers need not clear them).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).  No
 *    entry point synchronises or copies between host and device.
 *  - Argument errors are detected before any launch and returned as a status;
 *    dsa_last_error() then holds a message (per thread).  A failed launch
 *    returns DSA_ERR_HIP.  Device faults surface at the caller's next
 *    synchronisation.  No C++ exception crosses this interface.
 *  - Entry points keep no state between calls; concurrent calls on different
 *    streams are safe.
 *  - B == 0 or Lq == 0 is a valid empty call: nothing is launched, DSA_OK.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
    DSA_OK = 0,
    DSA_ERR_NULL = 1,         /* a required pointer is NULL                      */
    DSA_ERR_SHAPE = 2,        /* sizes inconsistent (e.g. q_pos0 + Lq > Lk)      */
    DSA_ERR_DTYPE = 3,        /* dtype not valid for this argument               */
    DSA_ERR_UNSUPPORTED = 4,  /* valid, but outside what the kernels implement   */
    DSA_ERR_ALIGN = 5,        /* a pointer is not 16-byte aligned                */
    DSA_ERR_WORKSPACE = 6,    /* workspace missing or too small                  */
    DSA_ERR_HIP = 7           /* the HIP runtime reported an error at launch     */
} dsa_status;

typedef enum dsa_dtype {
    DSA_F32 = 0,
    DSA_BF16 = 1,
    DSA_FP8_E4M3 = 2          /* OCP e4m3fn: bias 7, max 448, no inf, 0x7F = NaN */
} dsa_dtype;

/*
 * Lightning-indexer scores ("DeepseekV3.2 拆解", section 核心组件, indexer
 * equation; FP8 and ReLU chosen there for throughput):
 *
 *   scores[b,t,s] = k_scale[b,s] * sum_j (w[b,t,j] * q_scale[b,t,j])
 *                                 * ReLU(sum_d q_idx[b,t,j,d] * k_idx[b,s,d])
 *     for s <= t_pos,  and -INFINITY for t_pos < s < Lk.
 *
 * With positive scales this equals sum_j w * ReLU(qhat . khat) of the
 * dequantised vectors.  The key vector k_idx[s] has no head index: one key per
 * token serves every indexer head.
 *
 *   q_idx   [B,Lq,n_idx_heads,idx_dim]  FP8 e4m3 codes or fp32 (idx_dtype)
 *   q_scale [B,Lq,n_idx_heads] fp32 > 0  (FP8 only; must be NULL for F32)
 *   k_idx   [B,Lk,idx_dim]              same dtype as q_idx
 *   k_scale [B,Lk] fp32 > 0             (FP8 only; must be NULL for F32)
 *   w       [B,Lq,n_idx_heads] fp32     head weights, any sign
 *   scores  [B,Lq,Lk] fp32              output
 *
 * Supported: FP8 with idx_dim == 128 and n_idx_heads == 64;
 *            F32 with idx_dim % 4 == 0, idx_dim <= 256, n_idx_heads <= 64 and
 *            n_idx_heads * idx_dim <= 8192.
 */
dsa_status dsa_indexer_scores(const void* q_idx, const float* q_scale,
                              const void* k_idx, const float* k_scale,
                              const float* w, float* scores,
                              int B, int Lq, int Lk, int q_pos0,
                              int n_idx_heads, int idx_dim, dsa_dtype idx_dtype,
                              void* stream);

/*
 * Per-query top-k selection ("DeepseekV3.2 拆解", section 核心组件, the
 * token-selection equation; k = 2048 in the section 创新点 table):
 *
 *   idx[b,t,:] = the min(k, t_pos+1) positions s <= t_pos with the largest
 *                scores[b,t,s], ties resolved to the smaller s, written in
 *                ascending s and padded with -1 up to k entries.
 *
 * -0.0 and +0.0 rank as one value.  Only scores[b,t,0..t_pos] is read (rows
 * with t_pos + 1 <= k read nothing).  Scores must not be NaN.
 *
 *   scores [B,Lq,Lk] fp32;  idx [B,Lq,k] int32 (output).   Requires 1 <= k <= Lk.
 */
dsa_status dsa_topk(const float* scores, int32_t* idx,
                    int B, int Lq, int Lk, int q_pos0, int k, void* stream);

/*
 * Sparse attention over the selected latent rows ("DeepseekV3.2 拆解",
 * section 核心组件, u_t = Attn(h_t, {c_s : s selected})):
 *
 *   z_s        = softmax_scale * sum_{d<d_qk} q[b,t,h,d] * kv[b,s,d]
 *   out[b,t,h] = sum_s softmax(z)_s * kv[b,s,0:d_v]
 *   lse[b,t,h] = log sum_s exp(z_s)        (natural log; optional)
 * over s in { idx[b,t,i] : 0 <= idx[b,t,i] < Lk }.  Entries outside [0, Lk)
 * (such as the -1 padding) are skipped; an empty set gives out = 0 and
 * lse = -inf.  Duplicate entries count once per occurrence.
 *
 *   q   [B,Lq,n_heads,d_qk]  bf16 or fp32 (io_dtype)
 *   kv  [B,Lk,d_qk]          same dtype; one latent row per token shared by
 *                            every head, value = its first d_v columns
 *   idx [B,Lq,k] int32
 *   out [B,Lq,n_heads,d_v]   same dtype (bf16 rounded to nearest even)
 *   lse [B,Lq,n_heads] fp32  may be NULL
 *
 * Accumulation is fp32.  softmax_scale must be finite and > 0 (the MLA rows use
 * 1/sqrt(d_h + d^R_h) = 1/sqrt(192), "DeepSeek模型架构创新解析" section 4.3).
 * Supported: BF16 with n_heads % 16 == 0, n_heads <= 128, and
 *            (d_qk, d_v) in {(576,512), (128,128), (64,64)};
 *            F32 with d_qk <= 1024, d_v <= d_qk, n_heads <= 256.
 *
 * Workspace (bf16 576/512 rows with 32, 64 or 128 heads and k <= 2048): when
 * dsa_sparse_attn_workspace_size() is non-zero and `workspace` (256-byte
 * aligned) holds that many bytes,
 *  - few query rows (decode): each row's selected set is split over several
 *    workgroups whose normalised partial outputs and log-sum-exps are merged
 *    in fp32 (in a fixed order, so the result is deterministic).  Unsplit
 *    (workspace NULL or too small) the result agrees within fp32 rounding
 *    before the bf16 rounding of out;
 *  - many query rows: the workspace holds a counter from which workgroups
 *    take their rows in turn, so the GPU's dies share the rows by speed.  The
 *    result is the same bit for bit as without the workspace (one workgroup
 *    per row, fixed).
 * The workspace's contents on entry do not matter.  Calls that share a
 * workspace must not run at the same time.
 */
dsa_status dsa_sparse_attn(const void* q, const void* kv, const int32_t* idx,
                           void* out, float* lse,
                           int B, int Lq, int Lk, int q_pos0,
                           int n_heads, int d_qk, int d_v, int k,
                           float softmax_scale, dsa_dtype io_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace dsa_sparse_attn can use (0: none).  For the bf16 576/512
 * rows with 32, 64 or 128 heads and k <= 2048: with fewer than 128 query rows
 * (B * Lq) in all, the split partials; otherwise 256 bytes for the row
 * counter.
 */
size_t dsa_sparse_attn_workspace_size(int B, int Lq, int n_heads, int d_qk, int d_v, int k,
                                      dsa_dtype io_dtype);

/*
 * FP8 latent rows (the cache at 656 instead of 1152 bytes per token;
 * "DeepSeek模型架构创新解析" section 2.3: FP8 storage with a scale calibrated
 * per block).  Row layout, per token:
 *   bytes [0, 512)    e4m3 codes of dims 0..511
 *   bytes [512, 528)  four fp32 scales, scale g for dims 128g .. 128g+127
 *   bytes [528, 656)  dims 512..575 (the rotary part) as bf16, unchanged
 * Scale of a block: t = (amax / 448) in fp32, rounded up to a power of two (1
 * for an all-zero block); codes = e4m3(clamp(x / scale, -448, 448)), round to
 * nearest even.  Because the scale is a power of two, code * scale is exact in
 * bf16.
 *
 *   kv     [n_tok, 576] bf16 (input)
 *   kv_fp8 [n_tok, 656] bytes (output)
 */
dsa_status dsa_kv_pack_fp8(const void* kv, void* kv_fp8, int64_t n_tok, void* stream);

/*
 * dsa_sparse_attn over FP8 latent rows: the same computation with key row
 * [code * scale ; rotary part] (576 wide) and value its first 512 dims, taken
 * exactly (the kernel widens code * scale to bf16 without rounding).
 *   q      [B,Lq,n_heads,576] bf16
 *   kv_fp8 [B,Lk,656] packed rows (dsa_kv_pack_fp8)
 *   idx, out [B,Lq,n_heads,512] bf16, lse: as for dsa_sparse_attn
 * Supported: n_heads in {32, 64, 128}, k <= 2048.  The workspace rule is that
 * of dsa_sparse_attn with d_qk = 576, d_v = 512 (dsa_sparse_attn_workspace_size).
 */
dsa_status dsa_sparse_attn_fp8kv(const void* q, const void* kv_fp8, const int32_t* idx,
                                 void* out, float* lse,
                                 int B, int Lq, int Lk, int q_pos0, int n_heads, int k,
                                 float softmax_scale, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Indexer distillation loss of the dense warm-up ("DeepseekV3.2 拆解", section
 * 预训练策略: L^I = sum_t KL(p_t || Softmax(I_t))), one value per query row:
 *
 *   z[h,s]     = softmax_scale * q[b,t,h,:] . kv[b,s,0:d_qk]
 *   p[s]       = (1/n_heads) sum_h exp(z[h,s] - LSE_s' z[h,s'])      (dense, s <= t_pos)
 *   kl[b,t]    = sum_{s <= t_pos} p[s] (log p[s] - (scores[b,t,s] - LSE_s' scores[b,t,s']))
 *
 * p is the mean over heads of the main attention's dense distributions (the
 * pages leave the head aggregation open).  L^I is the sum of kl over rows.
 *   q      [B,Lq,n_heads,d_qk] bf16;  kv [B,Lk,d_qk] bf16
 *   scores [B,Lq,Lk] fp32 (as dsa_indexer_scores writes them; s <= t_pos read)
 *   kl     [B,Lq] fp32 (output)
 * Accumulation is fp32.  Supported: d_qk = 576, n_heads in {32, 64, 128}.
 * The work is two dense QK^T products per query row.
 */
dsa_status dsa_indexer_kl(const void* q, const void* kv, const float* scores, float* kl,
                          int B, int Lq, int Lk, int q_pos0, int n_heads, int d_qk,
                          float softmax_scale, void* stream);

/*
 * Backward of dsa_sparse_attn (the sparse training stage of "DeepseekV3.2
 * 拆解", section 预训练策略, trains the main model through the selected
 * sets).  Given dout = dL/dout, for each row and head over the selected
 * entries i (rows s_i, once per occurrence):
 *   P_i = exp(z_i - lse),  dP_i = dout . kv[s_i][0:d_v],  D = dout . out
 *   dZ_i = P_i (dP_i - D)
 *   dq          = softmax_scale * sum_i dZ_i kv[s_i][0:d_qk]
 *   dkv[s_i]   += softmax_scale * dZ_i q   (all d_qk columns)
 *   dkv[s_i]   += P_i dout                 (first d_v columns)
 * out and lse are the forward's outputs for the same inputs.
 *   q [B,Lq,n_heads,576] bf16; kv [B,Lk,576] bf16; idx [B,Lq,k] int32
 *   out, dout [B,Lq,n_heads,512] bf16; lse [B,Lq,n_heads] fp32
 *   dq [B,Lq,n_heads,576] fp32 (output); dkv [B,Lk,576] fp32 (output, overwritten)
 * P and dZ pass through the workspace in bf16 (the MFMA operand precision).
 * dkv: each entry's 576 fp32 contributions go to a slot of a key-major buffer
 * in the workspace (B * Lq * k slots of 2304 bytes), and each key's slots are
 * summed in slot order.  An entry's slot among its key's comes from an atomic
 * counter, so dkv's last bits vary between runs; dq is deterministic.
 * Supported: (d_qk, d_v) = (576, 512), n_heads in {16, 32, 64, 128}, k <= 2048,
 * B * Lq * k and B * Lk below 2^31.
 */
size_t dsa_sparse_attn_bwd_workspace_size(int B, int Lq, int Lk, int n_heads, int k);

dsa_status dsa_sparse_attn_bwd(const void* q, const void* kv, const int32_t* idx, const void* out,
                               const float* lse, const void* dout, float* dq, float* dkv,
                               int B, int Lq, int Lk, int q_pos0, int n_heads, int d_qk, int d_v, int k,
                               float softmax_scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * How dsa_forward finds each row's k largest scores.  Both routes give the
 * same selected sets, bit for bit (the k largest scores, the lowest s first
 * among equal ones); they differ in memory traffic.
 *
 * DSA_SELECT_SCORE_TILES: the indexer writes every row's scores (s <= t_pos)
 *   in tiles of q_tile_rows query rows, and dsa_topk reads them back.
 *
 * DSA_SELECT_CANDIDATES: no row's full scores are written.  With R = 2^r,
 *   r = max(0, floor(log2(k / 128))), the indexer first scores every R-th key
 *   (s = 0, R, 2R, ...) of each row with t_pos + 1 > 2k; each such row takes
 *   tau = the ceil(1.5 k / R)-th largest of those sample scores (about 1.5 k
 *   of its keys score at least that), the other rows tau = -inf.  The indexer
 *   then scores every key and keeps, per row, the list of keys scoring >= tau
 *   (at most cap = 2k stored), and the k largest of the list are selected.
 *   A list of at least k and at most 2k entries contains every key scoring at
 *   least the row's k-th largest score, so this selection is the exact top k.
 *   Rows whose list is shorter than k or longer than 2k are recomputed from
 *   their full scores, in tiles of q_tile_rows rows, by the first route (only
 *   those rows' scores are written).  Requires FP8 indexer inputs, Lq >= 8,
 *   k <= 2048, and (Lk - 1) / R + 1 <= 8192.
 *
 * DSA_SELECT_AUTO: candidates when they apply, k >= 1024 (the sample is then
 *   at most 1/8 of the keys) and the problem has at least 1024 blocks of 16
 *   query rows (B * ceil(Lq / 16)); score tiles otherwise.  For the workspace
 *   size, AUTO assumes FP8 inputs.
 */
typedef enum dsa_select {
    DSA_SELECT_AUTO = 0,
    DSA_SELECT_SCORE_TILES = 1,
    DSA_SELECT_CANDIDATES = 2
} dsa_select;

/*
 * Bytes of device workspace dsa_forward needs for these sizes and route, laid
 * out in this order: one tile of B * T * Lk fp32 scores (T = the query-tile
 * rows; at the start of the workspace), the selected sets
 * of all B * Lq rows (int32, k each), the attention's workspace (split
 * partials or row counter) when dsa_sparse_attn_workspace_size(B, Lq, ...)
 * is non-zero, and for the
 * candidate route per row: the sample scores ((Lk - 1) / R + 1 fp32, padded
 * to a multiple of 4), tau, the list (2k pairs of 4-byte words), its length and
 * a flag, then 256 bytes for the list pass's block counter.  q_tile_rows = 0
 * picks T automatically (the largest T whose score tile fits the automatic
 * tile budget, at most Lq).  Returns 0 for an empty
 * problem, for q_tile_rows < 0, and for DSA_SELECT_CANDIDATES on a problem the
 * candidate route does not take (with any idx_dtype).
 */
size_t dsa_forward_workspace_size(int B, int Lq, int Lk, int k, int n_heads, int d_qk, int d_v,
                                  dsa_dtype io_dtype, int q_tile_rows, dsa_select select);

/*
 * The whole forward ("DeepseekV3.2 拆解", section 核心组件: the output u_t of
 * query t is the attention of h_t over the latent rows c_s of the tokens whose
 * indexer scores I[t,s] are among its k largest):
 *
 *   out[b,t] = dsa_sparse_attn(q, kv, dsa_topk(dsa_indexer_scores(...), k))[b,t]
 *
 * The selected sets come from the route `select` names (dsa_select above).
 * With score tiles, the scores are formed in tiles of q_tile_rows query rows,
 * each tile's top-k following at once, so that at most B * q_tile_rows * Lk
 * scores exist at a time (the full Lq x Lk score matrix is never held when
 * q_tile_rows < Lq).  With candidates, only the sample scores and the lists are
 * written, and score tiles only for rows whose list misses.  The attention
 * then runs once over every row.  Rows with t_pos + 1 <= k select every
 * preceding token, so their scores are not computed.
 *
 * Results are identical, bit for bit, to calling dsa_indexer_scores, dsa_topk
 * and dsa_sparse_attn (with its workspace) in turn on the whole problem, for
 * every q_tile_rows and route.
 *
 * Arguments are those of the three calls; idx_out [B,Lq,k] and lse may be
 * NULL (without idx_out the selected sets stay in the workspace).  workspace
 * must hold dsa_forward_workspace_size(B, Lq, Lk, k, n_heads, d_qk, d_v,
 * io_dtype, q_tile_rows, select) bytes, 256-byte aligned; its contents on
 * entry do not matter.  Errors: those of the three calls; DSA_ERR_WORKSPACE
 * for a missing, short or misaligned workspace; DSA_ERR_SHAPE for
 * q_tile_rows < 0 or an unknown route; DSA_ERR_UNSUPPORTED for
 * DSA_SELECT_CANDIDATES on a problem it does not take.
 */
dsa_status dsa_forward(const void* q_idx, const float* q_scale,
                       const void* k_idx, const float* k_scale, const float* w,
                       int n_idx_heads, int idx_dim, dsa_dtype idx_dtype,
                       const void* q, const void* kv,
                       int n_heads, int d_qk, int d_v, dsa_dtype io_dtype,
                       float softmax_scale,
                       int B, int Lq, int Lk, int q_pos0, int k,
                       int32_t* idx_out, void* out, float* lse,
                       int q_tile_rows, dsa_select select, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * dsa_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It calls no allocating routine.  Its workspace is a
 * device array of DSA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held from the first call on that GPU until the process ends.
 *
 * Arguments and results are those of dsa_forward (bit for bit the same
 * output), by the score-tile route: the query tile is the largest one whose
 * workspace fits the array.
 * Problems for which even a one-row tile does not fit (B * Lk * 4 bytes of
 * scores, plus B * Lq * k * 4 for the selected sets when idx_out is NULL,
 * plus the attention's split partials) return DSA_ERR_UNSUPPORTED before any
 * launch.  All calls on one GPU share its array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and must not be made.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

dsa_status dsa_forward_noalloc(const void* q_idx, const float* q_scale,
                               const void* k_idx, const float* k_scale, const float* w,
                               int n_idx_heads, int idx_dim, dsa_dtype idx_dtype,
                               const void* q, const void* kv,
                               int n_heads, int d_qk, int d_v, dsa_dtype io_dtype,
                               float softmax_scale,
                               int B, int Lq, int Lk, int q_pos0, int k,
                               int32_t* idx_out, void* out, float* lse, void* stream);

/*
 * Per-token FP8 e4m3 quantisation of the indexer vectors ("DeepseekV3.2 拆解",
 * section 核心组件: the indexer computes in FP8; "DeepSeek模型架构创新解析"
 * section 4.3: enlarge the scale's safety margin, e.g. 1.2x, against FP8
 * overflow).  For each token i, the tok_len consecutive values x[i,:]:
 *
 *   amax           = max_j |x[i,j]|
 *   scale          = (amax * margin) / 448 in fp32 arithmetic; 1 if amax == 0
 *   codes[i,j]     = e4m3(clamp(x[i,j] / scale, -448, 448)), fp32 IEEE
 *                    division, round to nearest even
 *   scales[i*scale_repeat + r] = scale  for r < scale_repeat
 *
 * Decoding code * scale gives back x to within half an e4m3 step.  Layouts for
 * the indexer inputs of dsa_indexer_scores:
 *   k_I [B,Lk,d_I]:      n_tok = B*Lk, tok_len = d_I, scale_repeat = 1
 *                        -> k_scale [B,Lk];
 *   q_I [B,Lq,H_I,d_I]:  n_tok = B*Lq, tok_len = H_I*d_I, scale_repeat = H_I
 *                        -> q_scale [B,Lq,H_I] (one scale per token, broadcast
 *                        to its heads); or n_tok = B*Lq*H_I, tok_len = d_I,
 *                        scale_repeat = 1 for one scale per head.
 *
 *   x      [n_tok, tok_len] fp32 or bf16 (x_dtype), finite values
 *   codes  [n_tok, tok_len] e4m3 (output)
 *   scales [n_tok, scale_repeat] fp32 (output)
 * Requires tok_len % 8 == 0, 8 <= tok_len <= 16384, 1 <= scale_repeat <=
 * 65536, margin finite and > 0 (margin < 1 saturates the largest values).
 */
dsa_status dsa_quantize_e4m3(const void* x, dsa_dtype x_dtype, uint8_t* codes, float* scales,
                             int64_t n_tok, int tok_len, int scale_repeat, float margin,
                             void* stream);

/*
 * Row assembly with the decoupled rotary part ("DeepSeek模型架构创新解析",
 * section 1.1: the rotary position code lives in a separate d^R_h = d_h/2
 * wide part, one key part k^R shared by all heads per token and one query part
 * per head, beside the compressed latent c^KV / the absorbed query).  For
 * batch entry b, token t at position pos0 + t and head h:
 *
 *   out[b,t,h, 0:d_nope]              = nope[b,t,h, :]
 *   out[b,t,h, d_nope+2p], [.. +2p+1] = (r0 cos a - r1 sin a, r0 sin a + r1 cos a)
 *       (r0, r1) = rope[b,t,h, 2p:2p+2],  a = (pos0 + t) * rope_base^(-2p/d_rope),
 *       p < d_rope/2  (the rotary embedding of adjacent pairs).
 *
 * heads = 1 builds the cached latent rows kv = [c^KV ; RoPE(k^R)] (576 = 512 +
 * 64 on the MLA rows); heads = n_h builds the attention queries.
 *   nope [B,L,heads,d_nope] bf16 (NULL when d_nope == 0)
 *   rope [B,L,heads,d_rope] bf16
 *   out  [B,L,heads,d_nope+d_rope] bf16 (output, round to nearest even)
 * Angles are evaluated in fp64, the rotation in fp32.  Requires
 * d_nope % 8 == 0, d_rope % 8 == 0, 8 <= d_rope <= 128, pos0 >= 0 and
 * rope_base finite and > 1.
 */
dsa_status dsa_rope_assemble(const void* nope, const void* rope, void* out,
                             int B, int L, int heads, int d_nope, int d_rope, int pos0,
                             double rope_base, void* stream);

/* Static description of a status code. */
const char* dsa_status_string(dsa_status s);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
