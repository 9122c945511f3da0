// Input side of the DSA path on gfx950: per-token FP8 e4m3 quantisation of
// the indexer vectors ("DeepseekV3.2 拆解", section 核心组件: the indexer runs
// in FP8; "DeepSeek模型架构创新解析" section 4.3: a safety margin on the FP8
// scale), the assembly of latent / query rows from their compressed part and
// their decoupled rotary part (same page, section 1.1), and the FP8 form of
// the latent rows with a scale per 128-column block (same page, section 2.3).
//
// Both kernels are HBM-bound streaming passes: every input byte is read once
// and every output byte written once, with 16- or 32-byte accesses per lane.
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kQThreads = 256;
constexpr float kE4m3Max = 448.f;

// Four fp32 values to e4m3fn codes (bytes 0..3 in order) with the gfx950
// conversion, round to nearest even.
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d)
{
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// One group of 2^tpt_log2 threads per token; each thread holds up to NCH
// chunks of 8 values (chunk c*tpt + st of its token), so the token is read
// from memory once: amax over the group, scale, then codes from registers.
template <bool BF16IN, int NCH>
__global__ __launch_bounds__(kQThreads)
void quantize_e4m3_kernel(const void* __restrict__ x, uint8_t* __restrict__ codes,
                          float* __restrict__ scales, int64_t n_tok, int tok_len, int repeat,
                          float margin, int tpt_log2)
{
    __shared__ float red[kQThreads / kWave];
    const int tpt = 1 << tpt_log2;
    const int tid = threadIdx.x, lane = tid & 63;
    const int st = tid & (tpt - 1);
    const int slot = tid >> tpt_log2;
    const int64_t tok = (int64_t)blockIdx.x * (kQThreads >> tpt_log2) + slot;
    const bool live = tok < n_tok;
    const int nchunk = tok_len >> 3;

    float v[NCH][8];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = c * tpt + st;
        const bool on = live && ch < nchunk;
        if (BF16IN) {
            u32x4 u = {0u, 0u, 0u, 0u};
            if (on) u = *(const u32x4*)((const uint16_t*)x + tok * tok_len + ch * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[c][2 * e] = __uint_as_float(u[e] << 16);
                v[c][2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
            }
        } else {
            v4f a = {0.f, 0.f, 0.f, 0.f}, b = a;
            if (on) {
                const v4f* p = (const v4f*)((const float*)x + tok * tok_len + ch * 8);
                a = p[0];
                b = p[1];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[c][e] = a[e];
                v[c][4 + e] = b[e];
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[c][e]));
    }
    // amax over the token's threads (aligned groups of tpt lanes, or whole waves)
    if (tpt <= kWave) {
        for (int o = 1; o < tpt; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    } else {
        amax = wave_max(amax);
        if (lane == 0) red[tid >> 6] = amax;
        __syncthreads();
        const int w0 = slot * (tpt >> 6);
        for (int w = 0; w < (tpt >> 6); ++w) amax = fmaxf(amax, red[w0 + w]);
    }
    if (!live) return;
    // scale and division in fp32 (IEEE-rounded), the precision the codes are decided in
    const float scale = amax > 0.f ? (amax * margin) / kE4m3Max : 1.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = c * tpt + st;
        if (ch >= nchunk) break;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(v[c][e] / scale, -kE4m3Max), kE4m3Max);
        *(u32x2*)(codes + tok * tok_len + ch * 8) =
            u32x2{cvt_e4m3x4(y[0], y[1], y[2], y[3]), cvt_e4m3x4(y[4], y[5], y[6], y[7])};
    }
    for (int r = st; r < repeat; r += tpt) scales[tok * repeat + r] = scale;
}

// One workgroup per token (b, t).  The d_rope/2 angles (pos0 + t) *
// base^(-2p/d_rope) are evaluated in fp64 and their cosines and sines kept in
// LDS; every head's row then copies its compressed part and rotates its
// rotary pairs in fp32, 8 values (16 bytes) per access.
constexpr int kRThreads = 256;
constexpr int kMaxRopePairs = 64;

__global__ __launch_bounds__(kRThreads)
void rope_assemble_kernel(const uint16_t* __restrict__ nope, const uint16_t* __restrict__ rope,
                          uint16_t* __restrict__ out, int L, int heads, int d_nope, int d_rope,
                          int pos0, double log2_base)
{
    __shared__ float cs[kMaxRopePairs], sn[kMaxRopePairs];
    const int64_t tok = blockIdx.x;                  // b * L + t
    const int t = (int)(tok % L);
    const int tid = threadIdx.x;
    const int np = d_rope >> 1;
    if (tid < np) {
        const double a = (double)(pos0 + t) * exp2(-(2.0 * tid / d_rope) * log2_base);
        double s, c;
        sincos(a, &s, &c);
        cs[tid] = (float)c;
        sn[tid] = (float)s;
    }
    __syncthreads();
    const int w = d_nope + d_rope;
    const int nch = d_nope >> 3, rch = d_rope >> 3;
    const int64_t row0 = tok * heads;
    for (int i = tid; i < heads * nch; i += kRThreads) {
        const int h = i / nch, c = i - h * nch;
        *(u32x4*)(out + (row0 + h) * w + c * 8) = *(const u32x4*)(nope + (row0 + h) * d_nope + c * 8);
    }
    for (int i = tid; i < heads * rch; i += kRThreads) {
        const int h = i / rch, c = i - h * rch;
        const u32x4 u = *(const u32x4*)(rope + (row0 + h) * d_rope + c * 8);
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = 4 * c + e;                 // pair p = values 2p, 2p+1
            const float x0 = __uint_as_float(u[e] << 16);
            const float x1 = __uint_as_float(u[e] & 0xFFFF0000u);
            const float cp = cs[p], sp = sn[p];
            o[e] = pack_bf16x2(x0 * cp - x1 * sp, x0 * sp + x1 * cp);
        }
        *(u32x4*)(out + (row0 + h) * w + d_nope + c * 8) = o;
    }
}

// FP8 latent rows: one wave per token.  Lane l converts dims 8l..8l+7 of the
// 512 latent dims; the 16 lanes of each 128-dim block share its amax, whose
// scale t = amax / 448 (fp32) is rounded up to a power of two, so the codes
// x / scale come from an exact division.  Lanes 0..7 copy the bf16 rotary
// part (dims 512..575).
constexpr int kPackRow = 656;

__global__ __launch_bounds__(256)
void kv_pack_fp8_kernel(const uint16_t* __restrict__ kv, uint8_t* __restrict__ out, int64_t n_tok)
{
    const int lane = threadIdx.x & 63;
    const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tok >= n_tok) return;                         // whole waves leave together
    const uint16_t* row = kv + tok * 576;
    uint8_t* o = out + tok * kPackRow;
    const u32x4 u = *(const u32x4*)(row + 8 * lane);
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(u[e] << 16);
        v[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
        amax = fmaxf(amax, fmaxf(fabsf(v[2 * e]), fabsf(v[2 * e + 1])));
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    float scale = 1.f;
    if (amax > 0.f) {
        int ex;
        const float t = amax / kE4m3Max;
        const float f = frexpf(t, &ex);
        scale = (f == 0.5f) ? t : ldexpf(1.f, ex);
    }
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(v[e] / scale, -kE4m3Max), kE4m3Max);
    *(u32x2*)(o + 8 * lane) = u32x2{cvt_e4m3x4(y[0], y[1], y[2], y[3]), cvt_e4m3x4(y[4], y[5], y[6], y[7])};
    if ((lane & 15) == 0) *(float*)(o + 512 + 4 * (lane >> 4)) = scale;
    if (lane < 8) *(u32x4*)(o + 528 + 16 * lane) = *(const u32x4*)(row + 512 + 8 * lane);
}

}  // namespace

hipError_t launch_kv_pack_fp8(const KvPackLaunch& a, hipStream_t s)
{
    if (a.n_tok == 0) return hipSuccess;
    hipLaunchKernelGGL(kv_pack_fp8_kernel, dim3((unsigned)((a.n_tok + 3) / 4)), dim3(256), 0, s,
                       (const uint16_t*)a.kv, (uint8_t*)a.out, a.n_tok);
    return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const QuantLaunch& a, hipStream_t s)
{
    if (a.n_tok == 0) return hipSuccess;
    const int nchunk = a.tok_len / 8;
    const bool wide = nchunk > kQThreads * 4;        // more than 8192 values per token
    const int per = wide ? 8 : 4;                    // chunks held per thread
    int tpt_log2 = 0;
    while ((1 << tpt_log2) * per < nchunk) ++tpt_log2;
    const int64_t per_block = kQThreads >> tpt_log2;
    const unsigned blocks = (unsigned)((a.n_tok + per_block - 1) / per_block);
#define DSA_QLAUNCH(BF, N)                                                                        \
    hipLaunchKernelGGL((quantize_e4m3_kernel<BF, N>), dim3(blocks), dim3(kQThreads), 0, s, a.x, a.codes, \
                       a.scales, a.n_tok, a.tok_len, a.repeat, a.margin, tpt_log2)
    if (a.bf16) {
        if (wide) DSA_QLAUNCH(true, 8); else DSA_QLAUNCH(true, 4);
    } else {
        if (wide) DSA_QLAUNCH(false, 8); else DSA_QLAUNCH(false, 4);
    }
#undef DSA_QLAUNCH
    return hipGetLastError();
}

hipError_t launch_rope_assemble(const RopeLaunch& a, hipStream_t s)
{
    const int64_t n_tok = (int64_t)a.B * a.L;
    if (n_tok == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_assemble_kernel, dim3((unsigned)n_tok), dim3(kRThreads), 0, s,
                       (const uint16_t*)a.nope, (const uint16_t*)a.rope, (uint16_t*)a.out, a.L, a.heads,
                       a.d_nope, a.d_rope, a.pos0, log2(a.base));
    return hipGetLastError();
}

}  // namespace dsa
