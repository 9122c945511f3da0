// Lightning-indexer scores on gfx950.
//
// I[t,s] = k_scale[s] * sum_j (w[t,j] * q_scale[t,j]) * ReLU(q8[t,j,:] . k8[s,:])
// for s <= t_pos ("DeepseekV3.2 拆解", section 核心组件, indexer equation; the
// FP8 format and the ReLU are the page's choices for throughput).
//
// FP8 kernel layout (H^I = 64 heads, d^I = 128):
//  - one workgroup = 4 waves = one block of 16 query rows;
//  - wave w keeps the e4m3 query fragments of heads 16w..16w+15 for the 16
//    rows in registers (one 16x128 MFMA operand per head, 8 VGPRs each);
//  - keys stream through LDS in groups of 64 (8 KB); every key fragment is
//    reused for the wave's 16 heads;
//  - per head, one v_mfma_f32_16x16x128_f8f6f4 forms the 16-key x 16-query dot
//    products with a fresh fp32 accumulator (K = 128 = d^I, so there is no
//    long FP8 accumulation chain), and the epilogue applies ReLU and the
//    per-(query, head) weight in fp32 registers;
//  - the four waves' partial head sums meet in LDS, are multiplied by the key
//    scale, masked causally and written as fp32.
// The MFMA operand roles are A = keys (M), B = queries (N), so a lane's four
// outputs are four consecutive keys of one query and its head weight is one
// scalar per head.
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kQB = 16;        // query rows per workgroup
constexpr int kKG = 64;        // keys per LDS group (4 MFMA tiles of 16)
constexpr int kD = 128;        // indexer dim (bytes per key / per query head)
constexpr int kH = 64;         // indexer heads
constexpr int kHPW = 16;       // heads per wave
constexpr int kThreads = 256;  // 4 waves

__global__ __launch_bounds__(kThreads)
void indexer_fp8_kernel(const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
                        const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
                        const float* __restrict__ w, float* __restrict__ scores,
                        int Lq, int Lk, int q_pos0, int t_begin, int t_count,
                        int64_t sc_bstride, int64_t sc_rstride, int write_masked, int skip_upto_k)
{
    __shared__ __attribute__((aligned(16))) uint8_t ktile[kKG * kD];
    __shared__ __attribute__((aligned(16))) v4f red[4][4][kWave];   // [wave][tile][lane]

    const int nqb = (t_count + kQB - 1) / kQB;
    const int qb = nqb - 1 - (int)blockIdx.x;          // longest rows first
    const int b = blockIdx.y;
    const int t0 = t_begin + qb * kQB;
    const int rows_here = min(kQB, t_begin + t_count - t0);
    const int tpos_last = q_pos0 + t0 + rows_here - 1;
    if (skip_upto_k > 0 && tpos_last + 1 <= skip_upto_k)
        return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;

    // Query operand (B): row t0 + col, head j, bytes [32*grp, 32*grp + 32).
    const int tq = t0 + min(col, rows_here - 1);
    const int64_t qrow = (int64_t)b * Lq + tq;
    v8i qf[kHPW];
    float wq[kHPW];
#pragma unroll
    for (int h = 0; h < kHPW; ++h) {
        const int j = wave * kHPW + h;
        const u32x4* p = (const u32x4*)(q8 + (qrow * kH + j) * kD + grp * 32);
        qf[h] = as_i8(p[0], p[1]);
        wq[h] = w[qrow * kH + j] * q_scale[qrow * kH + j];
    }

    const int nkeys = tpos_last + 1;
    const int ngroups = (nkeys + kKG - 1) / kKG;
    const int ld_key = tid >> 2, ld_part = tid & 3;     // 64 keys x 4 parts of 32 B
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    for (int g = 0; g < ngroups; ++g) {
        const int s0 = g * kKG;
        // stage keys [s0, s0 + 64) in LDS
        {
            const int s = s0 + ld_key;
            u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
            if (s < Lk) {
                const u32x4* p = (const u32x4*)(k8 + ((int64_t)b * Lk + s) * kD + ld_part * 32);
                lo = p[0];
                hi = p[1];
            }
            __syncthreads();                            // previous group fully consumed
            u32x4* d = (u32x4*)(ktile + ld_key * kD + ld_part * 32);
            d[0] = lo;
            d[1] = hi;
            __syncthreads();
        }
        // key operand (A) fragments of the 4 tiles
        v8i af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4* p = (const u32x4*)(ktile + (i * 16 + col) * kD + grp * 32);
            af[i] = as_i8(p[0], p[1]);
        }
        v4f acc[4] = {zero, zero, zero, zero};
#pragma unroll
        for (int h = 0; h < kHPW; ++h) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v4f d = mfma_fp8_16x16x128(af[i], qf[h], zero);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[i][r] = fmaf(wq[h], fmaxf(d[r], 0.f), acc[i][r]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
        __syncthreads();
        // thread (wave = tile i, lane): sum the four waves' head partials
        v4f sum = red[0][wave][lane];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            const v4f x = red[ww][wave][lane];
            sum[0] += x[0]; sum[1] += x[1]; sum[2] += x[2]; sum[3] += x[3];
        }
        if (col < rows_here) {
            const int t = t0 + col;
            const int tpos = q_pos0 + t;
            const int sb = s0 + wave * 16 + grp * 4;
            float* dst = scores + (int64_t)b * sc_bstride + (int64_t)(t - t_begin) * sc_rstride + sb;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = sb + r;
                v[r] = (s <= tpos) ? sum[r] * k_scale[(int64_t)b * Lk + min(s, Lk - 1)] : -INFINITY;
            }
            const bool vec_ok = ((uintptr_t)dst & 15u) == 0;
            if (vec_ok && sb + 3 < Lk && (write_masked || sb + 3 <= tpos)) {
                *(v4f*)dst = v4f{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = sb + r;
                    if (s < Lk && (write_masked || s <= tpos)) dst[r] = v[r];
                }
            }
        }
    }

    if (write_masked) {
        // -inf beyond the last computed group for every row of the block
        const int s_from = ngroups * kKG;
        for (int r = 0; r < rows_here; ++r) {
            float* dst = scores + (int64_t)b * sc_bstride + (int64_t)(t0 + r - t_begin) * sc_rstride;
            for (int s = s_from + tid; s < Lk; s += kThreads) dst[s] = -INFINITY;
        }
    }
}

// fp32 indexer for small problems: one workgroup per query row, one thread per
// key.  The query row lives in LDS; dot products are plain fp32 FMAs.
constexpr int kF32Threads = 256;

__global__ __launch_bounds__(kF32Threads)
void indexer_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                        const float* __restrict__ w, float* __restrict__ scores,
                        int Lq, int Lk, int q_pos0, int t_begin, int H, int D,
                        int64_t sc_bstride, int64_t sc_rstride, int write_masked, int skip_upto_k)
{
    extern __shared__ float qsh[];                  // [H*D] + [H]
    const int t = t_begin + blockIdx.x;
    const int b = blockIdx.y;
    const int tpos = q_pos0 + t;
    if (skip_upto_k > 0 && tpos + 1 <= skip_upto_k)
        return;
    const int64_t qrow = (int64_t)b * Lq + t;
    for (int i = threadIdx.x; i < H * D; i += kF32Threads) qsh[i] = q[qrow * H * D + i];
    for (int i = threadIdx.x; i < H; i += kF32Threads) qsh[H * D + i] = w[qrow * H + i];
    __syncthreads();
    float* dst = scores + (int64_t)b * sc_bstride + (int64_t)blockIdx.x * sc_rstride;
    for (int s = threadIdx.x; s < Lk; s += kF32Threads) {
        if (s > tpos) {
            if (write_masked) dst[s] = -INFINITY;
            continue;
        }
        const float* kr = k + ((int64_t)b * Lk + s) * D;
        float I = 0.f;
        for (int j = 0; j < H; ++j) {
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(qsh[j * D + d], kr[d], dot);
            I = fmaf(qsh[H * D + j], fmaxf(dot, 0.f), I);
        }
        dst[s] = I;
    }
}

}  // namespace

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.t_count == 0) return hipSuccess;
    if (a.fp8) {
        const int nqb = (a.t_count + kQB - 1) / kQB;
        hipLaunchKernelGGL(indexer_fp8_kernel, dim3(nqb, a.B), dim3(kThreads), 0, s,
                           (const uint8_t*)a.q, a.q_scale, (const uint8_t*)a.k, a.k_scale, a.w,
                           a.scores, a.Lq, a.Lk, a.q_pos0, a.t_begin, a.t_count,
                           a.sc_bstride, a.sc_rstride, (int)a.write_masked, a.skip_upto_k);
    } else {
        const size_t shm = sizeof(float) * ((size_t)a.H * a.D + a.H);
        hipLaunchKernelGGL(indexer_f32_kernel, dim3(a.t_count, a.B), dim3(kF32Threads), shm, s,
                           (const float*)a.q, (const float*)a.k, a.w, a.scores, a.Lq, a.Lk,
                           a.q_pos0, a.t_begin, a.H, a.D, a.sc_bstride, a.sc_rstride,
                           (int)a.write_masked, a.skip_upto_k);
    }
    return hipGetLastError();
}

}  // namespace dsa
