// Sparse MQA attention over the selected latent rows on gfx950
// ("DeepseekV3.2 拆解", section 核心组件: u_t = Attn(h_t, {c_s : s in top-k});
// the latent row serves as key (first d_qk columns) and value (first d_v
// columns) because the key up-projection is absorbed into the query,
// "DeepSeek模型架构创新解析" section 1.1).
//
// bf16 kernel: one workgroup per query row, one wave per 16 query heads.
// Every head of the row shares the same selected set, so the workgroup gathers
// each selected latent row once into LDS (chunks of 32 rows) and all waves
// reuse it:
//   S^T[row, head] = K_chunk (32 x d_qk, LDS) . Q^T (d_qk x 16, registers)
//   online softmax in fp32 (exp2 domain), per head
//   O^T[dim, head] += V_chunk^T (d_v x 32, LDS, transposed copy) . P^T
// both with v_mfma_f32_16x16x32_bf16.  The S^T accumulator layout (lane l:
// rows 4*(l/16)+i of a 16-row tile, head l%16) is exactly the B-operand
// layout P^T needs once the 32 rows of a chunk are assigned to K slots as
// {4g..4g+3, 16+4g..16+4g+3} for lane group g; the transposed V copy is read
// with the same slot order.  Output is rounded to bf16 (nearest even); the
// log-sum-exp is written in fp32.
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kNC = 32;                   // selected rows per chunk

template <int DQK, int DV>
struct AttnShape {
    static constexpr int KP = DQK + 8;    // K chunk pitch (bf16 elements), breaks bank aliasing
    static constexpr int VP = kNC + 8;    // V^T pitch (bf16 elements)
    static constexpr int QC = DQK / 32;   // MFMA K steps for Q.K
    static constexpr int DT = DV / 16;    // 16-wide value tiles
    static constexpr size_t lds_bytes = sizeof(uint16_t) * ((size_t)kNC * KP + (size_t)DV * VP) + sizeof(int) * kNC;
};

template <int DQK, int DV>
__global__ __launch_bounds__(512)
void sparse_attn_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                             const int32_t* __restrict__ idx, uint16_t* __restrict__ out,
                             float* __restrict__ lse, int Lq, int Lk, int t_begin, int H, int k,
                             int64_t idx_bstride, float scale_log2)
{
    using S = AttnShape<DQK, DV>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint16_t* Kc = (uint16_t*)smem;                         // [kNC][KP]
    uint16_t* VT = Kc + kNC * S::KP;                        // [DV][VP]
    int* rows = (int*)(VT + DV * S::VP);                    // [kNC]

    const int row = blockIdx.x, b = blockIdx.y;
    const int t = t_begin + row;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int h = wave * 16 + col;                          // this lane's head

    // Q^T operand: head h, dims c*32 + 8*grp .. +8
    const uint16_t* qrow = q + (((int64_t)b * Lq + t) * H + h) * DQK;
    v8bf qf[S::QC];
#pragma unroll
    for (int c = 0; c < S::QC; ++c) qf[c] = as_bf8(*(const u32x4*)(qrow + c * 32 + grp * 8));

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    v4f o[S::DT];
#pragma unroll
    for (int i = 0; i < S::DT; ++i) o[i] = zero;
    float m = -INFINITY, l = 0.f;

    const int32_t* irow = idx + (int64_t)b * idx_bstride + (int64_t)row * k;
    const uint16_t* kvb = kv + (int64_t)b * Lk * DQK;
    constexpr int PPR = DQK / 8;                            // 16-byte pieces per row

    for (int c0 = 0; c0 < k; c0 += kNC) {
        if (tid < kNC) {
            const int s = (c0 + tid < k) ? irow[c0 + tid] : -1;
            rows[tid] = (s >= 0 && s < Lk) ? s : -1;
        }
        __syncthreads();
        // gather the chunk's latent rows (row-major, padded pitch)
        for (int p = tid; p < kNC * PPR; p += nthr) {
            const int r = p / PPR, c = p - r * PPR;
            const int s = rows[r];
            u32x4 v = {0u, 0u, 0u, 0u};
            if (s >= 0) v = *(const u32x4*)(kvb + (int64_t)s * DQK + c * 8);
            *(u32x4*)(Kc + r * S::KP + c * 8) = v;
        }
        __syncthreads();
        // transposed copy of the value columns: VT[d][r] = Kc[r][d]
        for (int p = tid; p < (kNC / 2) * DV; p += nthr) {
            const int rp = p % (kNC / 2), d = p / (kNC / 2);
            const uint32_t lo = Kc[(2 * rp) * S::KP + d];
            const uint32_t hi = Kc[(2 * rp + 1) * S::KP + d];
            *(uint32_t*)(VT + d * S::VP + 2 * rp) = lo | (hi << 16);
        }
        __syncthreads();

        // S^T for the two 16-row tiles
        v4f st[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            v4f acc = zero;
            const uint16_t* kr = Kc + (i * 16 + col) * S::KP + grp * 8;
#pragma unroll
            for (int c = 0; c < S::QC; ++c)
                acc = mfma_bf16_16x16x32(as_bf8(*(const u32x4*)(kr + c * 32)), qf[c], acc);
            st[i] = acc;
        }
        // online softmax (log2 domain) for head h over rows {16i + 4grp + r}
        float z[8];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool valid = rows[i * 16 + grp * 4 + r] >= 0;
                const float v = valid ? st[i][r] * scale_log2 : -INFINITY;
                z[i * 4 + r] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float m_new = fmaxf(m, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m - m_new);
        float psum = 0.f;
        uint32_t pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // K slot pair (2i, 2i+1): slots 0..3 -> tile 0 rows, 4..7 -> tile 1 rows
            const int a0 = 2 * i, a1 = 2 * i + 1;
            const float p0 = (z[a0] == -INFINITY) ? 0.f : exp2f(z[a0] - m_new);
            const float p1 = (z[a1] == -INFINITY) ? 0.f : exp2f(z[a1] - m_new);
            psum += p0 + p1;
            pb[i] = f32_to_bf16_bits(p0) | (f32_to_bf16_bits(p1) << 16);
        }
        psum += __shfl_xor(psum, 16, kWave);
        psum += __shfl_xor(psum, 32, kWave);
        l = l * alpha + psum;
        m = m_new;
        const v8bf pfrag = as_bf8(u32x4{pb[0], pb[1], pb[2], pb[3]});
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) {
            const uint16_t* vr = VT + (dt * 16 + col) * S::VP + grp * 4;
            const u32x2 lo = *(const u32x2*)vr;             // rows 4g .. 4g+3
            const u32x2 hi = *(const u32x2*)(vr + 16);      // rows 16+4g .. 16+4g+3
            const v8bf vfrag = as_bf8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            v4f acc = o[dt];
            acc[0] *= alpha; acc[1] *= alpha; acc[2] *= alpha; acc[3] *= alpha;
            o[dt] = mfma_bf16_16x16x32(vfrag, pfrag, acc);
        }
        __syncthreads();                                     // chunk buffers reused
    }

    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    uint16_t* orow = out + (((int64_t)b * Lq + t) * H + h) * DV;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
        const uint32_t w0 = f32_to_bf16_bits(o[dt][0] * inv) | (f32_to_bf16_bits(o[dt][1] * inv) << 16);
        const uint32_t w1 = f32_to_bf16_bits(o[dt][2] * inv) | (f32_to_bf16_bits(o[dt][3] * inv) << 16);
        *(u32x2*)(orow + dt * 16 + grp * 4) = u32x2{w0, w1};
    }
    if (lse != nullptr && grp == 0)
        lse[((int64_t)b * Lq + t) * H + h] = (l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// fp32 kernel for small problems: one workgroup per query row; heads in turn.
constexpr int kF32T = 256;

__global__ __launch_bounds__(kF32T)
void sparse_attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kv,
                            const int32_t* __restrict__ idx, float* __restrict__ out,
                            float* __restrict__ lse, int Lq, int Lk, int t_begin, int H, int Dqk,
                            int Dv, int k, int64_t idx_bstride, float scale)
{
    extern __shared__ float sh[];                 // z[k] | rows[k] | red[kF32T/64]
    float* z = sh;
    int* rows = (int*)(z + k);
    float* red = (float*)(rows + k);
    const int row = blockIdx.x, b = blockIdx.y;
    const int t = t_begin + row;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t* irow = idx + (int64_t)b * idx_bstride + (int64_t)row * k;
    for (int i = tid; i < k; i += kF32T) {
        const int s = irow[i];
        rows[i] = (s >= 0 && s < Lk) ? s : -1;
    }
    __syncthreads();
    const float* kvb = kv + (int64_t)b * Lk * Dqk;
    for (int h = 0; h < H; ++h) {
        const float* qh = q + (((int64_t)b * Lq + t) * H + h) * Dqk;
        float mloc = -INFINITY;
        for (int i = tid; i < k; i += kF32T) {
            float v = -INFINITY;
            if (rows[i] >= 0) {
                const float* kr = kvb + (int64_t)rows[i] * Dqk;
                float dot = 0.f;
                for (int d = 0; d < Dqk; ++d) dot = fmaf(qh[d], kr[d], dot);
                v = dot * scale;
            }
            z[i] = v;
            mloc = fmaxf(mloc, v);
        }
        mloc = wave_max(mloc);
        if (lane == 0) red[wave] = mloc;
        __syncthreads();
        float mx = red[0];
        for (int w2 = 1; w2 < kF32T / 64; ++w2) mx = fmaxf(mx, red[w2]);
        __syncthreads();
        float sloc = 0.f;
        for (int i = tid; i < k; i += kF32T) {
            const float p = (z[i] == -INFINITY) ? 0.f : expf(z[i] - mx);
            z[i] = p;
            sloc += p;
        }
        sloc = wave_sum(sloc);
        if (lane == 0) red[wave] = sloc;
        __syncthreads();
        float den = 0.f;
        for (int w2 = 0; w2 < kF32T / 64; ++w2) den += red[w2];
        const float inv = den > 0.f ? 1.f / den : 0.f;
        float* oh = out + (((int64_t)b * Lq + t) * H + h) * Dv;
        for (int d = tid; d < Dv; d += kF32T) {
            float acc = 0.f;
            for (int i = 0; i < k; ++i)
                if (rows[i] >= 0) acc = fmaf(z[i], kvb[(int64_t)rows[i] * Dqk + d], acc);
            oh[d] = acc * inv;
        }
        if (lse != nullptr && tid == 0)
            lse[((int64_t)b * Lq + t) * H + h] = den > 0.f ? mx + logf(den) : -INFINITY;
        __syncthreads();
    }
}

template <int DQK, int DV>
hipError_t launch_bf16(const AttnLaunch& a, hipStream_t s)
{
    using S = AttnShape<DQK, DV>;
    const int threads = (a.H / 16) * kWave;
    auto kern = sparse_attn_bf16_kernel<DQK, DV>;
    // more than 64 KB of dynamic LDS must be requested explicitly
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)S::lds_bytes);
    if (e != hipSuccess) return e;
    const float scale_log2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL(kern, dim3(a.t_count, a.B), dim3(threads), S::lds_bytes, s,
                       (const uint16_t*)a.q, (const uint16_t*)a.kv, a.idx, (uint16_t*)a.out, a.lse,
                       a.Lq, a.Lk, a.t_begin, a.H, a.k, a.idx_bstride, scale_log2);
    return hipGetLastError();
}

}  // namespace

bool sparse_attn_bf16_supported(int Dqk, int Dv)
{
    return (Dqk == 576 && Dv == 512) || (Dqk == 128 && Dv == 128) || (Dqk == 64 && Dv == 64);
}

hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.t_count == 0) return hipSuccess;
    if (a.bf16) {
        if (a.Dqk == 576 && a.Dv == 512) return launch_bf16<576, 512>(a, s);
        if (a.Dqk == 128 && a.Dv == 128) return launch_bf16<128, 128>(a, s);
        if (a.Dqk == 64 && a.Dv == 64) return launch_bf16<64, 64>(a, s);
        return hipErrorInvalidValue;
    }
    const size_t shm = sizeof(float) * (size_t)a.k + sizeof(int) * (size_t)a.k + sizeof(float) * (kF32T / 64);
    hipLaunchKernelGGL(sparse_attn_f32_kernel, dim3(a.t_count, a.B), dim3(kF32T), shm, s,
                       (const float*)a.q, (const float*)a.kv, a.idx, (float*)a.out, a.lse,
                       a.Lq, a.Lk, a.t_begin, a.H, a.Dqk, a.Dv, a.k, a.idx_bstride, a.scale);
    return hipGetLastError();
}

}  // namespace dsa
