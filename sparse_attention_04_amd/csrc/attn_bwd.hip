// Backward of the sparse MQA/MLA attention on gfx950 (the sparse training
// stage of "DeepseekV3.2 拆解", section 预训练策略, trains the main model
// through the selected sets).  For row t, head h and selected entries i
// (rows s_i of the latent cache, value = first 512 of 576 columns):
//   P_i  = exp(scale q.kv_i - lse),  dP_i = dO . v_i,  D = dO . O
//   dZ_i = P_i (dP_i - D)
//   dq   = scale sum_i dZ_i kv_i;   dkv_i += scale dZ_i q  (576),  dkv_i += P_i dO  (first 512)
//
// Two kernels, both with bf16 MFMAs and fp32 accumulation:
//  1. dq: one workgroup per (row, group of up to 64 heads), one wave per 16
//     heads.  q^T and dO^T stay in registers as 16x16x32 operands; per chunk
//     of 32 selected rows (staged in LDS, plus a transposed copy) it forms
//     S^T and dP^T, then P and dZ, and accumulates dq^T = K^T dZ^T in 36
//     register tiles.  P and dZ are also written (bf16, keys-major) for 2.
//  2. dkv: one workgroup per (row, 8 of the 18 column tiles of 32), one wave
//     per 2 tiles.  A tile of the first 512 columns takes both products,
//     scale dZ q and P dO, into one accumulator (one atomic per element, not
//     two); the last 2 tiles take scale dZ q only.  The B operands (q and dO,
//     heads along K) stay in registers for the whole row; per chunk the 32 x H
//     weights (P and scale dZ) come through LDS and each 32 x 32 tile is added
//     to the selected rows with fp32 atomics (so dkv's summation order varies
//     between runs).
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kBQK = 576;            // latent row width
constexpr int kBV = 512;             // value width
constexpr int kBNC = 32;             // selected rows per chunk
constexpr int kBKP = kBQK + 8;       // staged row pitch (bf16 elements): conflict-free 16-lane b128 reads
constexpr int kBTP = kBNC + 8;       // transposed copy pitch (bf16 elements)

// ---------------------------------------------------------------- 1. dq, P, dZ

template <int NW>
__global__ __launch_bounds__(64 * NW)
void attn_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                        const int32_t* __restrict__ idx, const uint16_t* __restrict__ out,
                        const float* __restrict__ lse, const uint16_t* __restrict__ dout,
                        float* __restrict__ dq, uint16_t* __restrict__ wsP, uint16_t* __restrict__ wsZ,
                        int Lq, int Lk, int H, int k, float scale)
{
    __shared__ __attribute__((aligned(16))) uint16_t Kc[kBNC * kBKP];   // chunk rows, row-major
    __shared__ __attribute__((aligned(16))) uint16_t KT[kBQK * kBTP];   // transposed: KT[d][r]
    __shared__ __attribute__((aligned(16))) uint16_t T[NW][2][kBNC * 16]; // P / dZ, [key][head] per wave
    __shared__ int rows[kBNC];
    __shared__ int wlast[NW];

    const int t = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int hb = blockIdx.z * 16 * NW + wave * 16;                    // this wave's first head
    const int h = hb + col;                                             // this lane's head (S^T column)
    const int64_t qrow = (int64_t)b * Lq + t;

    v8bf qT[kBQK / 32], doT[kBV / 32];
#pragma unroll
    for (int c = 0; c < kBQK / 32; ++c) qT[c] = as_bf8(*(const u32x4*)(q + (qrow * H + h) * kBQK + 32 * c + 8 * g));
#pragma unroll
    for (int c = 0; c < kBV / 32; ++c) doT[c] = as_bf8(*(const u32x4*)(dout + (qrow * H + h) * kBV + 32 * c + 8 * g));
    // D = dO . O for head h: lane group g covers dims {32 c + 8 g + e}
    float Dh = 0.f;
#pragma unroll
    for (int c = 0; c < kBV / 32; ++c) {
        const u32x4 o4 = *(const u32x4*)(out + (qrow * H + h) * kBV + 32 * c + 8 * g);
        const u32x4 d4 = __builtin_bit_cast(u32x4, doT[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Dh = fmaf(bf16_bits_to_f32(o4[e] & 0xFFFFu), bf16_bits_to_f32(d4[e] & 0xFFFFu), Dh);
            Dh = fmaf(bf16_bits_to_f32(o4[e] >> 16), bf16_bits_to_f32(d4[e] >> 16), Dh);
        }
    }
    Dh += __shfl_xor(Dh, 16, kWave);
    Dh += __shfl_xor(Dh, 32, kWave);
    const float lse2 = lse[qrow * H + h] * 1.4426950408889634f;
    const float scale_log2 = scale * 1.4426950408889634f;

    const int32_t* irow = idx + qrow * k;
    // chunks past the last valid entry are not visited
    int last = -1;
    for (int i = tid; i < k; i += 64 * NW) {
        const int s = irow[i];
        if (s >= 0 && s < Lk) last = i;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, kWave));
    if (lane == 0) wlast[wave] = last;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) last = max(last, wlast[w]);
    const int nchunks = (last + kBNC) / kBNC;

    v4f dqa[kBQK / 16];
#pragma unroll
    for (int m = 0; m < kBQK / 16; ++m) dqa[m] = v4f{0.f, 0.f, 0.f, 0.f};
    const uint16_t* kvb = kv + (int64_t)b * Lk * kBQK;

    for (int ch = 0; ch < nchunks; ++ch) {
        const int c0 = ch * kBNC;
        __syncthreads();                                                // previous chunk consumed
        if (tid < kBNC) {
            const int s = (c0 + tid < k) ? irow[c0 + tid] : -1;
            rows[tid] = (s >= 0 && s < Lk) ? s : -1;
        }
        __syncthreads();
        for (int p = tid; p < kBNC * (kBQK / 8); p += 64 * NW) {
            const int r = p / (kBQK / 8), c = p - r * (kBQK / 8);
            const int s = rows[r];
            u32x4 v = {0u, 0u, 0u, 0u};
            if (s >= 0) v = *(const u32x4*)(kvb + (int64_t)s * kBQK + c * 8);
            *(u32x4*)(Kc + r * kBKP + c * 8) = v;
        }
        __syncthreads();
        for (int p = tid; p < (kBNC / 2) * kBQK; p += 64 * NW) {
            const int rp = p % (kBNC / 2), d = p / (kBNC / 2);
            const uint32_t lo = Kc[(2 * rp) * kBKP + d], hi2 = Kc[(2 * rp + 1) * kBKP + d];
            *(uint32_t*)(KT + d * kBTP + 2 * rp) = lo | (hi2 << 16);
        }
        __syncthreads();

        // S^T and dP^T, keys 16 j + 4 g + i of tile j, head h
        v4f st[2], dpt[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint16_t* kr = Kc + (16 * j + col) * kBKP + 8 * g;
            v4f a = {0.f, 0.f, 0.f, 0.f}, bq = a;
#pragma unroll
            for (int c = 0; c < kBQK / 32; ++c) a = mfma_bf16_16x16x32(as_bf8(*(const u32x4*)(kr + 32 * c)), qT[c], a);
#pragma unroll
            for (int c = 0; c < kBV / 32; ++c) bq = mfma_bf16_16x16x32(as_bf8(*(const u32x4*)(kr + 32 * c)), doT[c], bq);
            st[j] = a;
            dpt[j] = bq;
        }
        float pv[8], zv[8];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = rows[16 * j + 4 * g + i] >= 0;
                const float p = ok ? exp2f(fmaf(st[j][i], scale_log2, -lse2)) : 0.f;
                pv[4 * j + i] = p;
                zv[4 * j + i] = p * (dpt[j][i] - Dh) * scale;          // scale dZ, used by dq and dkv
            }
        // dq^T tiles: A = dZ (head col, key slots 8g..8g+7 = keys 4g..4g+3, 16+4g..16+4g+3),
        // B = K^T (same key slots, dim 16 m + col) from the transposed copy
        const v8bf az = as_bf8(u32x4{pack_bf16x2(zv[0], zv[1]), pack_bf16x2(zv[2], zv[3]),
                                     pack_bf16x2(zv[4], zv[5]), pack_bf16x2(zv[6], zv[7])});
#pragma unroll
        for (int m = 0; m < kBQK / 16; ++m) {
            const uint16_t* kt = KT + (16 * m + col) * kBTP + 4 * g;
            const u32x2 lo = *(const u32x2*)kt, hi2 = *(const u32x2*)(kt + 16);
            dqa[m] = mfma_bf16_16x16x32(az, as_bf8(u32x4{lo[0], lo[1], hi2[0], hi2[1]}), dqa[m]);
        }
        // P and dZ (bf16) to the workspace, keys-major: through LDS so that a
        // lane stores 8 heads of one key
        uint16_t* tp = T[wave][0];
        uint16_t* tz = T[wave][1];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 16 * j + 4 * g + i;
                const uint32_t pz = pack_bf16x2(pv[4 * j + i], zv[4 * j + i]);
                tp[kk * 16 + col] = (uint16_t)(pz & 0xFFFFu);
                tz[kk * 16 + col] = (uint16_t)(pz >> 16);
            }
        __syncthreads();
        {
            const int kk = lane & 31, half = lane >> 5;
            if (c0 + kk < k) {
                const int64_t wo = (qrow * k + c0 + kk) * H + hb + 8 * half;
                *(u32x4*)(wsP + wo) = *(const u32x4*)(tp + kk * 16 + 8 * half);
                *(u32x4*)(wsZ + wo) = *(const u32x4*)(tz + kk * 16 + 8 * half);
            }
        }
    }
    // keys never visited (past the last valid entry) get zero weights
    for (int i = nchunks * kBNC + (tid >> 1); i < k; i += 32 * NW) {
        const int64_t wo = (qrow * k + i) * H + blockIdx.z * 16 * NW + 8 * (tid & 1);
        for (int w = 0; w < 2 * NW; w += 2) {
            *(u32x4*)(wsP + wo + 8 * w) = u32x4{0u, 0u, 0u, 0u};
            *(u32x4*)(wsZ + wo + 8 * w) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // dq[h = hb + 4 g + i][16 m + col]
#pragma unroll
    for (int m = 0; m < kBQK / 16; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dq[(qrow * H + hb + 4 * g + i) * kBQK + 16 * m + col] = dqa[m][i];
}

// ---------------------------------------------------------------- 2. dkv

constexpr int kTilesPerWave = 2;
constexpr int kDkvTiles = kBQK / 32;                                    // 18 (16 with a value part)
constexpr int kTilesPerGroup = 4 * kTilesPerWave;                       // 8 per workgroup

template <int KS>                                                       // K steps of 16 heads (H = 16 KS)
__global__ __launch_bounds__(256)
void attn_bwd_dkv_kernel(const uint16_t* __restrict__ q, const int32_t* __restrict__ idx,
                         const uint16_t* __restrict__ dout, const uint16_t* __restrict__ wsP,
                         const uint16_t* __restrict__ wsZ, float* __restrict__ dkv, int Lq, int Lk, int k,
                         float scale)
{
    constexpr int H = 16 * KS;
    __shared__ __attribute__((aligned(16))) uint16_t W[2][kBNC * (H + 8)];   // [P | dZ][key][head]
    __shared__ int rows[kBNC];
    const int t = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hs = lane >> 5;
    const int64_t qrow = (int64_t)b * Lq + t;
    const int tile0 = blockIdx.z * kTilesPerGroup + wave * kTilesPerWave;
    const int ntl = max(0, min(kTilesPerWave, kDkvTiles - tile0));

    // B operands of tile T (dims 32 T + n): q, and for T < 16 also dO; heads
    // 16 st + 8 hs + e along K
    v8bf bq[kTilesPerWave][KS], bo[kTilesPerWave][KS];
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
        const int T = tile0 + j;
        const bool hasv = T < kBV / 32;
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            uint32_t uq[4] = {0u, 0u, 0u, 0u}, uo[4] = {0u, 0u, 0u, 0u};
            if (j < ntl) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const int64_t h0 = qrow * H + 16 * st + 8 * hs + e;
                    uq[e / 2] = (uint32_t)q[h0 * kBQK + 32 * T + n] | ((uint32_t)q[(h0 + 1) * kBQK + 32 * T + n] << 16);
                    if (hasv)
                        uo[e / 2] = (uint32_t)dout[h0 * kBV + 32 * T + n] |
                                    ((uint32_t)dout[(h0 + 1) * kBV + 32 * T + n] << 16);
                }
            }
            bq[j][st] = as_bf8(u32x4{uq[0], uq[1], uq[2], uq[3]});
            bo[j][st] = as_bf8(u32x4{uo[0], uo[1], uo[2], uo[3]});
        }
    }

    const int32_t* irow = idx + qrow * k;
    float* dkvb = dkv + (int64_t)b * Lk * kBQK;
    const int nch = (k + kBNC - 1) / kBNC;
    for (int ch = 0; ch < nch; ++ch) {
        const int c0 = ch * kBNC;
        __syncthreads();
        if (tid < kBNC) {
            const int s = (c0 + tid < k) ? irow[c0 + tid] : -1;
            rows[tid] = (s >= 0 && s < Lk) ? s : -1;
        }
        // the chunk's weights: 32 keys x H heads of P and of dZ
        for (int p = tid; p < 2 * kBNC * (H / 8); p += 256) {
            const int which = p / (kBNC * (H / 8)), rem = p % (kBNC * (H / 8));
            const int kk = rem / (H / 8), c = rem % (H / 8);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (c0 + kk < k) v = *(const u32x4*)((which ? wsZ : wsP) + (qrow * k + c0 + kk) * H + 8 * c);
            *(u32x4*)(&W[which][kk * (H + 8) + 8 * c]) = v;
        }
        __syncthreads();
        bool any = false;
        for (int r = 0; r < kBNC; ++r) any |= rows[r] >= 0;
        if (!any) continue;                                             // workgroup-uniform
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j) {
            if (j >= ntl) break;                                        // wave-uniform
            const int T = tile0 + j;
            const uint16_t* wz = W[1] + n * (H + 8) + 8 * hs;           // scale dZ
            const uint16_t* wp = W[0] + n * (H + 8) + 8 * hs;           // P
            v16f acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
            for (int st = 0; st < KS; ++st)
                acc = mfma_bf16_32x32x16(as_bf8(*(const u32x4*)(wz + 16 * st)), bq[j][st], acc);
            if (T < kBV / 32) {
#pragma unroll
                for (int st = 0; st < KS; ++st)
                    acc = mfma_bf16_32x32x16(as_bf8(*(const u32x4*)(wp + 16 * st)), bo[j][st], acc);
            }
            const int d = 32 * T + n;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int s = rows[8 * (v >> 2) + 4 * hs + (v & 3)];
                if (s >= 0) unsafeAtomicAdd(dkvb + (int64_t)s * kBQK + d, acc[v]);
            }
        }
    }
}

__global__ __launch_bounds__(256)
void fill_zero_kernel(float* __restrict__ p, int64_t n4)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
        *(v4f*)(p + 4 * i) = v4f{0.f, 0.f, 0.f, 0.f};
}

}  // namespace

size_t attn_bwd_workspace_bytes(int B, int Lq, int H, int k)
{
    return 2 * (size_t)B * Lq * k * H * sizeof(uint16_t);
}

hipError_t launch_attn_bwd(const AttnBwdLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.Lq == 0) return hipSuccess;
    uint16_t* wsP = (uint16_t*)a.workspace;
    uint16_t* wsZ = wsP + (size_t)a.B * a.Lq * a.k * a.H;
    // dkv = 0 (a kernel, not a memset, so the sequence can be captured in a graph)
    const int64_t n4 = (int64_t)a.B * a.Lk * kBQK / 4;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<int64_t>((n4 + 255) / 256, 65536)), dim3(256), 0, s,
                       a.dkv, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nw = a.H >= 64 ? 4 : a.H / 16;
    const dim3 g1(a.Lq, a.B, a.H / (16 * nw));
#define DSA_DQ(NW)                                                                                            \
    hipLaunchKernelGGL(attn_bwd_dq_kernel<NW>, g1, dim3(64 * NW), 0, s, (const uint16_t*)a.q, (const uint16_t*)a.kv, \
                       a.idx, (const uint16_t*)a.out, a.lse, (const uint16_t*)a.dout, a.dq, wsP, wsZ, a.Lq, a.Lk, a.H, \
                       a.k, a.scale)
    switch (nw) {
    case 1: DSA_DQ(1); break;
    case 2: DSA_DQ(2); break;
    case 4: DSA_DQ(4); break;
    default: return hipErrorInvalidValue;
    }
#undef DSA_DQ
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2(a.Lq, a.B, (kDkvTiles + kTilesPerGroup - 1) / kTilesPerGroup);
#define DSA_DKV(KS)                                                                                           \
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<KS>, g2, dim3(256), 0, s, (const uint16_t*)a.q, a.idx,             \
                       (const uint16_t*)a.dout, wsP, wsZ, a.dkv, a.Lq, a.Lk, a.k, a.scale)
    switch (a.H / 16) {
    case 1: DSA_DKV(1); break;
    case 2: DSA_DKV(2); break;
    case 4: DSA_DKV(4); break;
    case 8: DSA_DKV(8); break;
    default: return hipErrorInvalidValue;
    }
#undef DSA_DKV
    return hipGetLastError();
}

}  // namespace dsa
