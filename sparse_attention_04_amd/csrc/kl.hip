// Indexer distillation loss of the dense warm-up on gfx950 ("DeepseekV3.2
// 拆解", section 预训练策略: the indexer is trained alone against the dense
// attention with L^I = sum_t KL(p_t || Softmax(I_t))).  p_t is taken as the
// mean over the H heads of the main attention's dense distributions over the
// keys s <= t_pos (the pages leave the head aggregation open):
//
//   z[h,s] = scale * q[t,h,:] . kv[s,0:576]
//   p[s]   = (1/H) sum_h exp(z[h,s] - LSE_h)
//   KL_t   = sum_s p[s] log p[s] - sum_s p[s] I[t,s] + LSE(I[t,:]) * sum_s p[s]
//
// One workgroup per query row, one wave per 32 heads, the query held in
// registers as 36 bf16 MFMA operands (v_mfma_f32_32x32x16_bf16, keys as the A
// operand).  Two sweeps over the row's keys in chunks of 32 rows staged in
// LDS: the first keeps each head's running maximum and sum (LSE_h), the second
// recomputes the scores, turns them into per-head probabilities, sums them
// over the heads through LDS and folds p log p, p I and p into three sums.
// The work is two QK^T products per query row (no value product).
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kKC = 32;                 // keys per chunk
constexpr int kQK = 576;                // latent row width (key)
constexpr int kSteps = kQK / 16;        // MFMA K steps
constexpr int kKPitch = kQK * 2 + 16;   // staged key row pitch in bytes (conflict-free b128 reads)

__device__ __forceinline__ float block_sum(float v, float* red, int nwaves)
{
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = 0.f;
    for (int w = 0; w < nwaves; ++w) s += red[w];
    return s;
}

__device__ __forceinline__ float block_max(float v, float* red, int nwaves)
{
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float m = -INFINITY;
    for (int w = 0; w < nwaves; ++w) m = fmaxf(m, red[w]);
    return m;
}

template <int NW>
__global__ __launch_bounds__(64 * NW)
void indexer_kl_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                       const float* __restrict__ scores, float* __restrict__ kl, int Lq, int Lk, int q_pos0,
                       float scale_log2)
{
    constexpr int H = 32 * NW;
    constexpr int NT = 64 * NW;
    __shared__ __attribute__((aligned(16))) uint8_t krow[kKC * kKPitch];
    __shared__ float E[kKC][H + 1];                  // per key: each head's probability
    __shared__ float red[NW];

    const int t = blockIdx.x, b = blockIdx.y;
    const int tpos = q_pos0 + t, n = tpos + 1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hi = lane >> 5;
    const int h = wave * 32 + col;

    // query fragments: head h, dims 16 c + 8 hi .. +8
    const uint16_t* qrow = q + (((int64_t)b * Lq + t) * H + h) * kQK;
    v8bf qf[kSteps];
#pragma unroll
    for (int c = 0; c < kSteps; ++c) qf[c] = as_bf8(*(const u32x4*)(qrow + c * 16 + hi * 8));

    // log-sum-exp of the indexer scores over s < n
    const float* I = scores + ((int64_t)b * Lq + t) * Lk;
    float mi = -INFINITY;
    for (int s = tid; s < n; s += NT) mi = fmaxf(mi, I[s]);
    mi = block_max(mi, red, NW);
    float si = 0.f;
    for (int s = tid; s < n; s += NT) si += expf(I[s] - mi);
    const float lse_i = mi + logf(block_sum(si, red, NW));

    const uint16_t* kvb = kv + (int64_t)b * Lk * kQK;
    // stage keys c0 .. c0+31 (rows past the row's last key repeat it; masked below)
    auto stage = [&](int c0) {
        __syncthreads();                                       // previous chunk fully consumed
        for (int pc = tid; pc < kKC * (kQK / 8); pc += NT) {
            const int r = pc / (kQK / 8), c = pc - r * (kQK / 8);
            const int s = min(c0 + r, n - 1);
            *(u32x4*)(krow + r * kKPitch + c * 16) = *(const u32x4*)(kvb + (int64_t)s * kQK + c * 8);
        }
        __syncthreads();
    };
    // S^T of the chunk for this wave's heads: element v is key c0 + 8 (v / 4) + 4 hi + v % 4
    auto scores_T = [&]() -> v16f {
        v16f acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
        const uint8_t* kr = krow + col * kKPitch + hi * 16;
#pragma unroll
        for (int c = 0; c < kSteps; ++c)
            acc = mfma_bf16_32x32x16(as_bf8(*(const u32x4*)(kr + c * 32)), qf[c], acc);
        return acc;
    };

    // pass 1: per-head maximum and sum (log2 domain)
    float m = -INFINITY, l = 0.f;
    for (int c0 = 0; c0 < n; c0 += kKC) {
        stage(c0);
        const v16f st = scores_T();
        float z[16], cm = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int s = c0 + 8 * (v >> 2) + 4 * hi + (v & 3);
            z[v] = (s < n) ? st[v] * scale_log2 : -INFINITY;
            cm = fmaxf(cm, z[v]);
        }
        cm = fmaxf(cm, __shfl_xor(cm, 32, kWave));
        const float mn = fmaxf(m, cm);                         // finite: key c0 <= tpos is valid
        float ps = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) ps += exp2f(z[v] - mn);
        ps += __shfl_xor(ps, 32, kWave);
        l = l * exp2f(m - mn) + ps;
        m = mn;
    }
    const float lse2 = m + log2f(l);

    // pass 2: p per key, then the three sums
    float a_plogp = 0.f, a_pI = 0.f, a_p = 0.f;
    constexpr int TPK = NT / kKC;                              // threads per key in the head sum
    for (int c0 = 0; c0 < n; c0 += kKC) {
        stage(c0);
        const v16f st = scores_T();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int kk = 8 * (v >> 2) + 4 * hi + (v & 3);
            E[kk][h] = (c0 + kk < n) ? exp2f(st[v] * scale_log2 - lse2) : 0.f;
        }
        __syncthreads();
        const int kk = tid / TPK, part = tid % TPK;
        float ph = 0.f;
        for (int j = part; j < H; j += TPK) ph += E[kk][j];
#pragma unroll
        for (int o = 1; o < TPK; o <<= 1) ph += __shfl_xor(ph, o, kWave);
        const int s = c0 + kk;
        if (part == 0 && s < n) {
            const float p = ph * (1.f / H);
            if (p > 0.f) a_plogp += p * logf(p);
            a_pI += p * I[s];
            a_p += p;
        }
    }
    a_plogp = block_sum(a_plogp, red, NW);
    a_pI = block_sum(a_pI, red, NW);
    a_p = block_sum(a_p, red, NW);
    if (tid == 0) kl[(int64_t)b * Lq + t] = a_plogp - a_pI + lse_i * a_p;
}

}  // namespace

hipError_t launch_indexer_kl(const KlLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.Lq == 0) return hipSuccess;
    const float scale_log2 = a.scale * 1.4426950408889634f;
    const dim3 grid(a.Lq, a.B);
#define DSA_KLLAUNCH(NW)                                                                              \
    hipLaunchKernelGGL(indexer_kl_kernel<NW>, grid, dim3(64 * NW), 0, s, (const uint16_t*)a.q,       \
                       (const uint16_t*)a.kv, a.scores, a.kl, a.Lq, a.Lk, a.q_pos0, scale_log2)
    switch (a.H) {
    case 32: DSA_KLLAUNCH(1); break;
    case 64: DSA_KLLAUNCH(2); break;
    case 128: DSA_KLLAUNCH(4); break;
    default: return hipErrorInvalidValue;
    }
#undef DSA_KLLAUNCH
    return hipGetLastError();
}

}  // namespace dsa
