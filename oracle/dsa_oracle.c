/*
 * Plain CPU oracle for the DeepSeek Sparse Attention (DSA) forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no code, header or table with the HIP path.
 *
 * It evaluates the definitions literally, by brute force, in double precision:
 *
 *  - indexer score ("DeepseekV3.2 拆解", section 核心组件, lightning indexer
 *    equation):  I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]) over the preceding
 *    tokens s <= t (self included);
 *  - fine-grained token selection (same section, the u_t equation): the k
 *    largest I[t,s]; ties go to the lower s; the set is emitted in ascending s
 *    and padded with -1 when fewer than k tokens precede t;
 *  - attention of the query over the selected latent rows only, with the row's
 *    first d_qk columns as key and first d_v columns as value ("DeepSeek模型架构
 *    创新解析" section 1.1: the up-projection is absorbed so attention runs on the
 *    latent row) and a softmax scale supplied by the caller;
 *  - on the input side, per-token FP8 e4m3 quantisation (nearest code by
 *    exhaustive search, scale and division in fp32, the precision the codes
 *    are decided in) and the assembly of a row from its compressed part and
 *    its rotary part (section 1.1 of the same page);
 *  - the 656-byte FP8 form of a latent row (per-128-column power-of-two block
 *    scales) and the exact values it stands for;
 *  - the indexer's distillation loss, KL(dense attention distribution ||
 *    softmax of the indexer scores) per query row;
 *  - the backward of the sparse attention (gradients of q and of the latent
 *    rows through the selected sets).
 *
 * Inputs are the same bytes the GPU consumes.  FP8 e4m3fn codes are decoded
 * with a table built here from the OCP E4M3 definition (1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits, subnormals at exponent 0, S.1111.111 = NaN,
 * no infinities, largest finite 448), then multiplied by their fp32 scale in
 * fp32.  bf16 is decoded by placing its 16 bits at the top of an fp32 word.
 *
 * Rows are independent; OpenMP parallelises over rows only, so the arithmetic
 * order within a row is exactly the order written below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2 };

/* ---- decoding ----------------------------------------------------------- */

double orc_e4m3_value(int code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, 1 - 7);           /* subnormal: 2^(1-bias) * 0.m */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);     /* normal: 2^(e-bias) * 1.m */
    return sign ? -v : v;
}

static float g_e4m3[256];
static int g_e4m3_ready = 0;

static void e4m3_table_init(void)
{
    if (g_e4m3_ready)
        return;
    for (int c = 0; c < 256; ++c)
        g_e4m3[c] = (float)orc_e4m3_value(c);
    g_e4m3_ready = 1;
}

void orc_e4m3_table(float* out256)
{
    e4m3_table_init();
    memcpy(out256, g_e4m3, sizeof(g_e4m3));
}

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Element i of a row stored as dtype, optionally multiplied by an fp32 scale
 * in fp32 arithmetic (dequantisation). */
static float load_elem(const void* base, int dtype, int64_t i)
{
    switch (dtype) {
    case ORC_F32: return ((const float*)base)[i];
    case ORC_BF16: return bf16_to_float(((const uint16_t*)base)[i]);
    default: return g_e4m3[((const uint8_t*)base)[i]];
    }
}

/* ---- indexer scores ------------------------------------------------------ */

/*
 * scores[r][s] for r < n_rows, s < Lk:
 *   I = sum_j w[r][j] * max(0, sum_d qhat[r][j][d] * khat[s][d])   for s <= t_pos[r]
 *   -INFINITY                                                     for s >  t_pos[r]
 * q_idx: [n_rows][H][D], q_scale: [n_rows][H] (NULL when dtype is F32),
 * k_idx: [Lk][D], k_scale: [Lk] (NULL when F32), w: [n_rows][H].
 * qhat = fp32(decode(q) * q_scale), khat = fp32(decode(k) * k_scale).
 * Returns 0, or -1 on bad arguments.
 */
int orc_indexer(const void* q_idx, const float* q_scale, const void* k_idx,
                const float* k_scale, const float* w, int dtype,
                const int64_t* t_pos, int n_rows, int Lk, int H, int D,
                double* scores)
{
    if (dtype != ORC_F32 && dtype != ORC_E4M3)
        return -1;
    if (dtype == ORC_E4M3 && (!q_scale || !k_scale))
        return -1;
    e4m3_table_init();

    float* khat = (float*)malloc(sizeof(float) * (size_t)Lk * (size_t)D);
    if (!khat)
        return -1;
    for (int64_t s = 0; s < Lk; ++s)
        for (int d = 0; d < D; ++d) {
            float v = load_elem(k_idx, dtype, s * D + d);
            khat[s * D + d] = (dtype == ORC_E4M3) ? v * k_scale[s] : v;
        }

    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|: bad)
    for (int r = 0; r < n_rows; ++r) {
        if (t_pos[r] < 0 || t_pos[r] >= Lk) {
            bad = 1;
            continue;
        }
        float* qhat = (float*)malloc(sizeof(float) * (size_t)H * (size_t)D);
        for (int j = 0; j < H; ++j)
            for (int d = 0; d < D; ++d) {
                int64_t i = ((int64_t)r * H + j) * D + d;
                float v = load_elem(q_idx, dtype, i);
                qhat[j * D + d] = (dtype == ORC_E4M3) ? v * q_scale[(int64_t)r * H + j] : v;
            }
        double* row = scores + (int64_t)r * Lk;
        for (int64_t s = 0; s < Lk; ++s) {
            if (s > t_pos[r]) {
                row[s] = -INFINITY;
                continue;
            }
            double I = 0.0;
            for (int j = 0; j < H; ++j) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += (double)qhat[j * D + d] * (double)khat[s * D + d];
                double relu = dot > 0.0 ? dot : 0.0;
                I += (double)w[(int64_t)r * H + j] * relu;
            }
            row[s] = I;
        }
        free(qhat);
    }
    free(khat);
    return bad ? -1 : 0;
}

/* ---- top-k selection ---------------------------------------------------- */

typedef struct { double v; int32_t s; } scored_t;

/* Order: larger score first; equal scores (−0 == +0) by smaller index. */
static int by_score_then_index(const void* a, const void* b)
{
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->s > y->s) - (x->s < y->s);
}

static int by_index(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/*
 * idx[r][0..k): the min(k, t_pos[r]+1) indices s <= t_pos[r] of the largest
 * scores[r][s] (ties to the smaller s), in ascending s, then -1 padding.
 * scores: [n_rows][ld]; only s <= t_pos[r] is read.
 */
int orc_topk(const double* scores, int64_t ld, const int64_t* t_pos, int n_rows,
             int k, int32_t* idx)
{
    if (k < 1)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|: bad)
    for (int r = 0; r < n_rows; ++r) {
        int64_t n = t_pos[r] + 1;
        int32_t* out = idx + (int64_t)r * k;
        if (n < 1 || n > ld) {
            bad = 1;
            continue;
        }
        int m = n < k ? (int)n : k;
        scored_t* all = (scored_t*)malloc(sizeof(scored_t) * (size_t)n);
        for (int64_t s = 0; s < n; ++s) {
            double v = scores[(int64_t)r * ld + s];
            all[s].v = (v == 0.0) ? 0.0 : v;   /* −0 and +0 are one value */
            all[s].s = (int32_t)s;
        }
        qsort(all, (size_t)n, sizeof(scored_t), by_score_then_index);
        for (int i = 0; i < m; ++i)
            out[i] = all[i].s;
        qsort(out, (size_t)m, sizeof(int32_t), by_index);
        for (int i = m; i < k; ++i)
            out[i] = -1;
        free(all);
    }
    return bad ? -1 : 0;
}

/* ---- sparse attention over the selected rows ---------------------------- */

/*
 * For each row r and head h, over the selected set S = {idx[r][i] : idx >= 0}:
 *   z_s  = scale * sum_d q[r][h][d] * kv[s][d]            (d < d_qk)
 *   o[d] = sum_s exp(z_s - max z) * kv[s][d] / sum_s exp(z_s - max z)   (d < d_v)
 *   lse  = max z + log(sum_s exp(z_s - max z))
 * q: [n_rows][H][d_qk], kv: [Lk][d_qk] (both F32 or BF16), idx: [n_rows][k].
 * out: [n_rows][H][d_v], lse: [n_rows][H] (may be NULL).  An empty set gives
 * o = 0 and lse = -inf.
 */
int orc_sparse_attn(const void* q, const void* kv, int dtype, const int32_t* idx,
                    int n_rows, int k, int Lk, int H, int d_qk, int d_v,
                    double scale, double* out, double* lse)
{
    if (dtype != ORC_F32 && dtype != ORC_BF16)
        return -1;
    if (d_v > d_qk)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|: bad)
    for (int r = 0; r < n_rows; ++r) {
        const int32_t* sel = idx + (int64_t)r * k;
        int n = 0;
        for (int i = 0; i < k; ++i) {
            if (sel[i] >= Lk) bad = 1;
            if (sel[i] >= 0 && sel[i] < Lk) ++n;
        }
        double* z = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
        n = 0;
        for (int i = 0; i < k; ++i)
            if (sel[i] >= 0 && sel[i] < Lk)
                rows[n++] = sel[i];
        for (int h = 0; h < H; ++h) {
            double* o = out + ((int64_t)r * H + h) * d_v;
            const int64_t qoff = ((int64_t)r * H + h) * d_qk;
            if (n == 0) {
                for (int d = 0; d < d_v; ++d) o[d] = 0.0;
                if (lse) lse[(int64_t)r * H + h] = -INFINITY;
                continue;
            }
            double zmax = -INFINITY;
            for (int i = 0; i < n; ++i) {
                double dot = 0.0;
                for (int d = 0; d < d_qk; ++d)
                    dot += (double)load_elem(q, dtype, qoff + d) *
                           (double)load_elem(kv, dtype, (int64_t)rows[i] * d_qk + d);
                z[i] = scale * dot;
                if (z[i] > zmax) zmax = z[i];
            }
            double denom = 0.0;
            for (int i = 0; i < n; ++i) {
                z[i] = exp(z[i] - zmax);          /* z now holds the weight p_s */
                denom += z[i];
            }
            for (int d = 0; d < d_v; ++d) {
                double acc = 0.0;
                for (int i = 0; i < n; ++i)
                    acc += z[i] * (double)load_elem(kv, dtype, (int64_t)rows[i] * d_qk + d);
                o[d] = acc / denom;
            }
            if (lse) lse[(int64_t)r * H + h] = zmax + log(denom);
        }
        free(z);
        free(rows);
    }
    return bad ? -1 : 0;
}

/* ---- input side: FP8 quantisation, latent-row assembly ------------------ */

/*
 * e4m3fn code nearest to y, ties to the even code (round to nearest even),
 * magnitudes beyond 448 saturating to 448.  Found by exhaustive search over
 * the 127 non-negative finite codes of the table above; the sign bit is y's
 * (so -0.0 and negative values that round to zero give 0x80).  NaN gives 0x7F.
 */
int orc_e4m3_encode(float y)
{
    e4m3_table_init();
    if (isnan(y))
        return 0x7F;
    double a = fabs((double)y);
    int best = 0;
    double bd = a;                                   /* distance to code 0 (= 0.0) */
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(a - (double)g_e4m3[c]);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return signbit(y) ? (best | 0x80) : best;
}

/*
 * Per-token FP8 quantisation ("DeepseekV3.2 拆解", section 核心组件: the
 * indexer runs in FP8; "DeepSeek模型架构创新解析" section 4.3: an optional
 * safety margin on the scale against FP8 overflow).  For each token i of
 * tok_len values x:
 *   amax  = max |x|
 *   scale = fp32(fp32(amax * margin) / 448), or 1 when amax == 0
 *   code  = e4m3(clamp(fp32(x / scale), -448, 448))
 * and the scale is written `repeat` times (scales[i * repeat + r]).  The
 * scale and the division are fp32 operations, the precision the codes are
 * decided in.  x is fp32 or bf16 (dtype).  Returns 0, or -1 on bad arguments.
 */
int orc_quantize_e4m3(const void* x, int dtype, int64_t n_tok, int tok_len, int repeat,
                      float margin, uint8_t* codes, float* scales)
{
    if ((dtype != ORC_F32 && dtype != ORC_BF16) || n_tok < 0 || tok_len < 1 || repeat < 1)
        return -1;
    e4m3_table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_tok; ++i) {
        const int64_t off = i * tok_len;
        float amax = 0.0f;
        for (int j = 0; j < tok_len; ++j) {
            float a = fabsf(load_elem(x, dtype, off + j));
            if (a > amax) amax = a;
        }
        float scale = 1.0f;
        if (amax > 0.0f) {
            float t = amax * margin;
            scale = t / 448.0f;
        }
        for (int j = 0; j < tok_len; ++j) {
            float y = load_elem(x, dtype, off + j) / scale;
            if (y > 448.0f) y = 448.0f;
            if (y < -448.0f) y = -448.0f;
            codes[off + j] = (uint8_t)orc_e4m3_encode(y);
        }
        for (int r = 0; r < repeat; ++r)
            scales[i * repeat + r] = scale;
    }
    return 0;
}

/*
 * Row assembly with the decoupled rotary part ("DeepSeek模型架构创新解析",
 * section 1.1: the rotary part is a separate d^R_h-wide vector, one shared
 * key per token and one query part per head, concatenated to the compressed
 * part).  For token i at position pos[i] and head h:
 *   out[i][h][0:d_nope]          = nope[i][h][:]
 *   out[i][h][d_nope + 2p]       = r[2p] cos(a_p) - r[2p+1] sin(a_p)
 *   out[i][h][d_nope + 2p + 1]   = r[2p] sin(a_p) + r[2p+1] cos(a_p)
 *   a_p = pos[i] * base^(-2p / d_rope),  p < d_rope / 2,   r = rope[i][h][:]
 * (the rotary embedding of adjacent pairs; the pages name RoPE without
 * restating it).  Inputs are bf16 bit patterns; out is float64.
 */
int orc_rope_rows(const uint16_t* nope, const uint16_t* rope, int64_t n_tok, int heads,
                  int d_nope, int d_rope, const int64_t* pos, double base, double* out)
{
    if (n_tok < 0 || heads < 1 || d_nope < 0 || d_rope < 0 || (d_rope & 1) || !(base > 0.0))
        return -1;
    const int w = d_nope + d_rope;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_tok; ++i) {
        for (int h = 0; h < heads; ++h) {
            const int64_t row = i * heads + h;
            double* o = out + row * w;
            for (int d = 0; d < d_nope; ++d)
                o[d] = (double)bf16_to_float(nope[row * d_nope + d]);
            for (int p = 0; p < d_rope / 2; ++p) {
                double a = (double)pos[i] * pow(base, -2.0 * p / (double)d_rope);
                double x0 = (double)bf16_to_float(rope[row * d_rope + 2 * p]);
                double x1 = (double)bf16_to_float(rope[row * d_rope + 2 * p + 1]);
                o[d_nope + 2 * p] = x0 * cos(a) - x1 * sin(a);
                o[d_nope + 2 * p + 1] = x0 * sin(a) + x1 * cos(a);
            }
        }
    }
    return 0;
}

/*
 * FP8 latent rows (NEXT row of the path: the cache at half the bytes;
 * "DeepSeek模型架构创新解析" section 2.3 gives FP8 storage with a scale
 * calibrated per block).  A 576-wide bf16 row becomes 656 bytes:
 *   [0, 512)    e4m3 codes of dims 0..511
 *   [512, 528)  four fp32 block scales, dims 128g .. 128g + 127
 *   [528, 656)  dims 512..575 (the rotary part) as the original bf16
 * Block scale: t = fp32(amax / 448); scale = the smallest power of two >= t
 * (1 when amax == 0); code = e4m3(clamp(fp32(x / scale), -448, 448)).  With a
 * power-of-two scale, code * scale is exact in bf16 and fp32.
 */
static float pow2_ceil(float t)
{
    int e;
    float f = frexpf(t, &e);                         /* t = f * 2^e, f in [0.5, 1) */
    return (f == 0.5f) ? t : ldexpf(1.0f, e);
}

int orc_kv_pack_fp8(const uint16_t* kv, int64_t n_tok, uint8_t* out)
{
    if (n_tok < 0)
        return -1;
    e4m3_table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_tok; ++i) {
        const uint16_t* row = kv + i * 576;
        uint8_t* o = out + i * 656;
        for (int g = 0; g < 4; ++g) {
            float amax = 0.0f;
            for (int d = 128 * g; d < 128 * g + 128; ++d) {
                float a = fabsf(bf16_to_float(row[d]));
                if (a > amax) amax = a;
            }
            float scale = 1.0f;
            if (amax > 0.0f) {
                float t = amax / 448.0f;
                scale = pow2_ceil(t);
            }
            memcpy(o + 512 + 4 * g, &scale, 4);
            for (int d = 128 * g; d < 128 * g + 128; ++d) {
                float y = bf16_to_float(row[d]) / scale;
                if (y > 448.0f) y = 448.0f;
                if (y < -448.0f) y = -448.0f;
                o[d] = (uint8_t)orc_e4m3_encode(y);
            }
        }
        memcpy(o + 528, row + 512, 128);
    }
    return 0;
}

/* The 576 fp32 values a packed row stands for: code * scale, then the bf16 tail. */
int orc_kv_unpack_fp8(const uint8_t* packed, int64_t n_tok, float* out)
{
    if (n_tok < 0)
        return -1;
    e4m3_table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_tok; ++i) {
        const uint8_t* p = packed + i * 656;
        float* o = out + i * 576;
        for (int g = 0; g < 4; ++g) {
            float scale;
            memcpy(&scale, p + 512 + 4 * g, 4);
            for (int d = 128 * g; d < 128 * g + 128; ++d)
                o[d] = g_e4m3[p[d]] * scale;
        }
        for (int d = 0; d < 64; ++d) {
            uint16_t h;
            memcpy(&h, p + 528 + 2 * d, 2);
            o[512 + d] = bf16_to_float(h);
        }
    }
    return 0;
}

/*
 * Indexer distillation loss of the dense warm-up ("DeepseekV3.2 拆解", section
 * 预训练策略, dense warm-up stage): per query row r, KL(p || Softmax(I[r,:]))
 * over the keys s <= t_pos[r], where p is the dense attention distribution of
 * the main attention over the same rows, taken as the mean over the H heads
 * of each head's softmax (the pages leave the head aggregation open):
 *   z[h][s] = scale * q[r][h][:] . kv[s][0:d_qk]
 *   p[s]    = (1/H) sum_h exp(z[h][s] - LSE_h(z[h][:]))
 *   KL[r]   = sum_s p[s] (log p[s] - (I[r][s] - LSE(I[r][:])))   (0 log 0 = 0)
 * q [n_rows][H][d_qk] and kv [Lk][d_qk] are F32 or BF16 (dtype); scores
 * [n_rows][Lk] float64.  Returns 0, or -1 on bad arguments.
 */
int orc_indexer_kl(const void* q, const void* kv, int dtype, const double* scores,
                   const int64_t* t_pos, int n_rows, int Lk, int H, int d_qk, double scale,
                   double* kl)
{
    if ((dtype != ORC_F32 && dtype != ORC_BF16) || H < 1 || d_qk < 1)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|: bad)
    for (int r = 0; r < n_rows; ++r) {
        const int64_t n = t_pos[r] + 1;
        if (n < 1 || n > Lk) {
            bad = 1;
            continue;
        }
        double* z = (double*)malloc(sizeof(double) * (size_t)n);
        double* p = (double*)calloc((size_t)n, sizeof(double));
        for (int h = 0; h < H; ++h) {
            const int64_t qoff = ((int64_t)r * H + h) * d_qk;
            double zmax = -INFINITY;
            for (int64_t s = 0; s < n; ++s) {
                double dot = 0.0;
                for (int d = 0; d < d_qk; ++d)
                    dot += (double)load_elem(q, dtype, qoff + d) * (double)load_elem(kv, dtype, s * d_qk + d);
                z[s] = scale * dot;
                if (z[s] > zmax) zmax = z[s];
            }
            double sum = 0.0;
            for (int64_t s = 0; s < n; ++s) sum += exp(z[s] - zmax);
            const double lse = zmax + log(sum);
            for (int64_t s = 0; s < n; ++s) p[s] += exp(z[s] - lse) / (double)H;
        }
        const double* I = scores + (int64_t)r * Lk;
        double imax = -INFINITY;
        for (int64_t s = 0; s < n; ++s) if (I[s] > imax) imax = I[s];
        double isum = 0.0;
        for (int64_t s = 0; s < n; ++s) isum += exp(I[s] - imax);
        const double lse_i = imax + log(isum);
        double acc = 0.0;
        for (int64_t s = 0; s < n; ++s)
            if (p[s] > 0.0) acc += p[s] * (log(p[s]) - (I[s] - lse_i));
        kl[r] = acc;
        free(z);
        free(p);
    }
    return bad ? -1 : 0;
}

/*
 * Backward of the sparse attention (the sparse training stage of "DeepseekV3.2
 * 拆解", section 预训练策略, trains the main model through the selected sets):
 * for each row r and head h, over the selected entries i (s_i = idx[r][i]
 * valid, counted once per occurrence),
 *   z_i  = scale * q[r][h] . kv[s_i][0:d_qk],   p = softmax(z)
 *   dp_i = dout[r][h] . kv[s_i][0:d_v],         D = sum_i p_i dp_i
 *   dz_i = p_i (dp_i - D)
 *   dq[r][h]            = scale * sum_i dz_i kv[s_i][0:d_qk]
 *   dkv[s_i][0:d_qk]   += scale * dz_i q[r][h]
 *   dkv[s_i][0:d_v]    += p_i dout[r][h]
 * q [n_rows][H][d_qk], kv [Lk][d_qk], dout [n_rows][H][d_v] (F32 or BF16);
 * dq [n_rows][H][d_qk] and dkv [Lk][d_qk] float64 (dkv overwritten).
 * Rows run in parallel with a private dkv per thread, summed at the end.
 */
int orc_sparse_attn_bwd(const void* q, const void* kv, const void* dout, int dtype, const int32_t* idx,
                        int n_rows, int k, int Lk, int H, int d_qk, int d_v, double scale,
                        double* dq, double* dkv)
{
    if ((dtype != ORC_F32 && dtype != ORC_BF16) || d_v > d_qk)
        return -1;
    memset(dkv, 0, sizeof(double) * (size_t)Lk * (size_t)d_qk);
    int bad = 0;
#pragma omp parallel reduction(|: bad)
    {
        double* my = (double*)calloc((size_t)Lk * (size_t)d_qk, sizeof(double));
        double* z = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        double* dp = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < n_rows; ++r) {
            int n = 0;
            for (int i = 0; i < k; ++i) {
                const int32_t s = idx[(int64_t)r * k + i];
                if (s >= Lk) bad = 1;
                if (s >= 0 && s < Lk) rows[n++] = s;
            }
            for (int h = 0; h < H; ++h) {
                const int64_t qo = ((int64_t)r * H + h) * d_qk, go = ((int64_t)r * H + h) * d_v;
                double* dqh = dq + qo;
                for (int d = 0; d < d_qk; ++d) dqh[d] = 0.0;
                if (n == 0) continue;
                double zmax = -INFINITY;
                for (int i = 0; i < n; ++i) {
                    double a = 0.0, g = 0.0;
                    for (int d = 0; d < d_qk; ++d)
                        a += (double)load_elem(q, dtype, qo + d) * (double)load_elem(kv, dtype, (int64_t)rows[i] * d_qk + d);
                    for (int d = 0; d < d_v; ++d)
                        g += (double)load_elem(dout, dtype, go + d) * (double)load_elem(kv, dtype, (int64_t)rows[i] * d_qk + d);
                    z[i] = scale * a;
                    dp[i] = g;
                    if (z[i] > zmax) zmax = z[i];
                }
                double sum = 0.0;
                for (int i = 0; i < n; ++i) { z[i] = exp(z[i] - zmax); sum += z[i]; }
                double D = 0.0;
                for (int i = 0; i < n; ++i) { z[i] /= sum; D += z[i] * dp[i]; }      /* z now holds p */
                for (int i = 0; i < n; ++i) {
                    const double dz = z[i] * (dp[i] - D);
                    const int64_t ko = (int64_t)rows[i] * d_qk;
                    for (int d = 0; d < d_qk; ++d) {
                        dqh[d] += scale * dz * (double)load_elem(kv, dtype, ko + d);
                        my[ko + d] += scale * dz * (double)load_elem(q, dtype, qo + d);
                    }
                    for (int d = 0; d < d_v; ++d)
                        my[ko + d] += z[i] * (double)load_elem(dout, dtype, go + d);
                }
            }
        }
#pragma omp critical
        for (int64_t e = 0; e < (int64_t)Lk * d_qk; ++e) dkv[e] += my[e];
        free(my);
        free(z);
        free(dp);
        free(rows);
    }
    return bad ? -1 : 0;
}

/* Number of threads OpenMP would use for the loops above. */
int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
