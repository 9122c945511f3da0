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
// registers as 36 bf16 MFMA operands (v_mfma_f32_32x32x16_bf16).  Two sweeps
// over the row's keys in chunks of 32 rows:
//  1. S^T (keys as the A operand, so a lane holds 16 keys of one head): each
//     head's running maximum and sum, LSE_h;
//  2. S (the same registers with the operands swapped, so a lane holds 16
//     heads of one key): per key, the wave's sum over its heads of
//     exp(z - LSE_h), 16 values in the lane plus its partner lane; the waves'
//     sums meet in LDS and one wave folds p log p, p I and p into three sums
//     one chunk later, behind the next chunk's barrier.
// The rows stream through a two-slot LDS ring with asynchronous global -> LDS
// copies issued one chunk ahead: each row's first 512 columns at a 1040-byte
// pitch (one copy instruction per row; 16 consecutive rows read at one column
// cover all banks once), its last 64 columns packed 8 rows per 1 KB with piece
// p of row r at position p ^ (r % 8), and the chunk's 32 indexer scores.  At
// 256 registers and under 80 KB of LDS per workgroup, two rows share a CU.
// The work is two QK^T products per query row (no value product).
#include "hw.h"
#include "launch.h"

#include <type_traits>

namespace dsa {

namespace {

constexpr int kKC = 32;                 // keys per chunk
constexpr int kQK = 576;                // latent row width (key)
constexpr int kSteps = kQK / 16;        // MFMA K steps
constexpr int kVPitch = 1040;           // bytes per staged row head (first 512 columns + one skew piece)
constexpr int kVBytes = kKC * kVPitch;
constexpr int kScoreOff = kVBytes + kKC * 128;  // after the 64-column tails: the chunk's 32 indexer scores
constexpr int kSlot = kScoreOff + 256;
constexpr int kRing = 2;

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
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1)   // 128 heads: two workgroups per CU, at most 256 registers
void indexer_kl_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                       const float* __restrict__ scores, float* __restrict__ kl, int Lq, int Lk, int q_pos0,
                       float scale_log2)
{
    constexpr int H = 32 * NW;
    constexpr int NT = 64 * NW;
    __shared__ __attribute__((aligned(16))) uint8_t ring[kRing][kSlot];
    __shared__ float lse_h[H];                       // per head, log2 domain
    __shared__ float pw[2][NW][kKC];                 // per chunk parity, wave, key: the wave's head sum
    __shared__ float red[NW];

    const int t = Lq - 1 - (int)blockIdx.x, b = blockIdx.y;     // longest rows first
    const int tpos = q_pos0 + t, n = tpos + 1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hi = lane >> 5;
    const int h = wave * 32 + col;

    // query fragments: head h, dims 16 c + 8 hi .. +8 (the B operand of S^T
    // and, with the same contents, the A operand of S)
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
    const int nch = (n + kKC - 1) / kKC;
    // copies of keys c0 .. c0+31 into ring slot `slot` (rows past the row's
    // last key repeat it; masked below): row e on wave e % NW, tail group ti
    // (rows 8 ti .. 8 ti + 7) on wave ti % NW, the scores on wave 0 (lanes
    // 32..63 repeat the last)
    auto issue = [&](int c0, int slot) {
        const uint32_t base = lds_byte_address(ring[slot]);
        for (int e = wave; e < kKC; e += NW) {
            const int sr = min(c0 + e, n - 1);
            global_to_lds16_async(kvb + (int64_t)sr * kQK + lane * 8,
                                  __builtin_amdgcn_readfirstlane(base + (uint32_t)e * kVPitch));
        }
        for (int ti = wave; ti < kKC / 8; ti += NW) {
            const int r = 8 * ti + (lane >> 3);
            const int sr = min(c0 + r, n - 1);
            const int pc = (lane & 7) ^ (r & 7);
            global_to_lds16_async(kvb + (int64_t)sr * kQK + 512 + pc * 8,
                                  __builtin_amdgcn_readfirstlane(base + (uint32_t)(kVBytes + ti * 1024)));
        }
        if (wave == 0)
            global_to_lds4_async(I + min(c0 + lane, n - 1), __builtin_amdgcn_readfirstlane(base + (uint32_t)kScoreOff));
    };
    // top of chunk ch: this wave's copies of ch landed, then every wave's
    // (and every wave is done with ch - 1, whose slot takes ch + 1)
    auto next_chunk = [&](int ch) {
        wait_vmcnt0();
        __syncthreads();
        if (ch + 1 < nch) issue((ch + 1) * kKC, (ch + 1) % kRing);
    };
    // the 36 K-step fragments of the lane's key (chunk row col) in slot
    // `slot`, read kPre steps ahead of their MFMA (order pinned: the compiler
    // would otherwise move each read next to its use); ST selects S^T
    // (keys x heads) or S (heads x keys)
    auto product = [&](int slot, auto st_tag) -> v16f {
        constexpr bool ST = decltype(st_tag)::value;
        v16f acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
        const uint8_t* vr = ring[slot] + col * kVPitch + hi * 16;
        const uint8_t* tr = ring[slot] + kVBytes + (col >> 3) * 1024 + (col & 7) * 128;
        auto frag = [&](int c) -> u32x4 {
            return c < 32 ? *(const u32x4*)(vr + 32 * c) : *(const u32x4*)(tr + (((2 * (c - 32) + hi) ^ (col & 7)) << 4));
        };
        constexpr int kPre = 3;
        u32x4 kf[kPre + 1];
#pragma unroll
        for (int i = 0; i < kPre; ++i) kf[i] = frag(i);
#pragma unroll
        for (int c = 0; c < kSteps; ++c) {
            if (c + kPre < kSteps) kf[(c + kPre) % (kPre + 1)] = frag(c + kPre);
            if constexpr (ST) acc = mfma_bf16_32x32x16(as_bf8(kf[c % (kPre + 1)]), qf[c], acc);
            else acc = mfma_bf16_32x32x16(qf[c], as_bf8(kf[c % (kPre + 1)]), acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        return acc;
    };
    using STag = std::integral_constant<bool, true>;
    using SRow = std::integral_constant<bool, false>;

    // pass 1: per-head maximum and sum (log2 domain); S^T element v is key
    // c0 + 8 (v / 4) + 4 hi + v % 4 of head h
    float m = -INFINITY, l = 0.f;
    __syncthreads();
    issue(0, 0);
    for (int ch = 0; ch < nch; ++ch) {
        const int c0 = ch * kKC;
        next_chunk(ch);
        const v16f st = product(ch % kRing, STag{});
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
    if (hi == 0) lse_h[h] = m + log2f(l);
    __syncthreads();                                           // pass 1 done with the ring; lse_h published
    // S element v is head wave*32 + 8 (v / 4) + 4 hi + v % 4 of key c0 + col
    float lsev[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) lsev[v] = lse_h[wave * 32 + 8 * (v >> 2) + 4 * hi + (v & 3)];

    // pass 2: per key, p = mean over heads of exp2(z - lse); wave 0's lanes
    // col < 32 fold chunk ch - 1's keys in after chunk ch's barrier
    float a_plogp = 0.f, a_pI = 0.f, a_p = 0.f;
    float i_prev = 0.f;                                        // indexer score of key (ch - 1) * 32 + col
    auto fold = [&](int ch_done, float iv) {
        const int s = ch_done * kKC + col;
        if (wave == 0 && hi == 0 && s < n) {
            float ph = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) ph += pw[ch_done & 1][w][col];
            const float p = ph * (1.f / H);
            if (p > 0.f) a_plogp += p * logf(p);
            a_pI += p * iv;
            a_p += p;
        }
    };
    issue(0, 0);
    for (int ch = 0; ch < nch; ++ch) {
        next_chunk(ch);
        if (ch > 0) fold(ch - 1, i_prev);
        const uint8_t* slot = ring[ch % kRing];
        const float i_cur = *(const float*)(slot + kScoreOff + 4 * col);
        const v16f sv = product(ch % kRing, SRow{});
        float ph = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) ph += exp2f(fmaf(sv[v], scale_log2, -lsev[v]));
        ph += __shfl_xor(ph, 32, kWave);
        if (hi == 0) pw[ch & 1][wave][col] = ph;
        i_prev = i_cur;
    }
    __syncthreads();
    if (nch > 0) fold(nch - 1, i_prev);
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
