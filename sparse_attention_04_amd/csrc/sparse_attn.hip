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
#include "attn_layout.h"
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
            pb[i] = pack_bf16x2(p0, p1);
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
        const uint32_t w0 = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
        const uint32_t w1 = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
        *(u32x2*)(orow + dt * 16 + grp * 4) = u32x2{w0, w1};
    }
    if (lse != nullptr && grp == 0)
        lse[((int64_t)b * Lq + t) * H + h] = (l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// bf16 kernel for n_heads % 32 == 0 (the MLA workload): one workgroup per
// query row, one wave per 32 heads, v_mfma_f32_32x32x16_bf16 throughout.
//  - The selected latent rows stream through a two-slot LDS ring, 32 rows
//    per chunk, copied with asynchronous global->LDS loads issued one chunk
//    ahead, so the copy of chunk c+1 overlaps the MFMA work on chunk c.  A row is stored as its value part (the first d_v columns, one
//    copy instruction of 64 x 16 bytes, whose source row is wave-uniform) and
//    its tail (the remaining d_qk - d_v columns, 8 rows per copy
//    instruction), so the copies need no per-lane row lookups.  The query's
//    whole index list (k <= 2048) is staged in LDS once, so the only memory
//    traffic inside the loop is the row copies: s_waitcnt vmcnt(0) plus one
//    workgroup barrier per chunk publishes a chunk and frees the other slot.
//  - Value parts sit at a pitch of 1040 bytes (one 16-byte skew per row) and
//    S^T row slot m = 16t + 8a + 4h + j holds chunk row 16t + 2a + h + 4j.
//    With that order both the key-fragment reads (16 rows per quarter-wave)
//    and the transpose reads (rows 4 apart, 8 bytes per lane) cover all 64
//    LDS banks exactly once, and every fragment address is one per-lane base
//    plus an immediate.  Tails are packed 8 rows per 1 KB with piece c of
//    row r at position c ^ (r % 8).
//  - S^T[32 rows x 32 heads] = K_chunk . Q^T, the query operand (36 steps of
//    32 heads x 16 dims) held in registers for the whole row.
//  - Softmax in fp32 (exp2 domain) against a per-head reference maximum m
//    fixed at the first chunk holding a valid row, so O is never rescaled
//    (no VALU work on the 256 accumulator registers).  Probabilities
//    exp2(z - m) may exceed 1 by up to 2^64, which bf16 and fp32 carry
//    without overflow; the final division by the same-frame sum l makes the
//    result independent of m.  If any logit exceeds m by more than 64 the
//    pass only keeps tracking the true maximum and the query is recomputed
//    once with it (workgroup-uniform decision, at most two passes).
//  - O^T[32 dims x 32 heads] += V^T . P^T, where P^T is the S^T accumulator
//    converted to bf16 in place (its lane layout is the B-operand layout) and
//    V^T fragments come straight from the row-major chunk through LDS
//    transpose reads (no transposed copy of V).
// FP8 latent rows (F8 = true): 656 bytes per token -- e4m3 codes of dims
// 0..511, four fp32 power-of-two scales (one per 128 dims), and dims 512..575
// in bf16.  The copies land in a staging area (codes, scales, rotary part),
// and at the top of each chunk the workgroup writes the chunk into the ring
// in the bf16 layout above: code * scale is exact in bf16 because the scale
// is a power of two, so the MFMA work that follows is unchanged.
constexpr int kF8Row = 656;                 // bytes per packed row
constexpr int kF8Codes = 32 * 512;          // staging: codes of the chunk's 32 rows
constexpr int kF8Scales = 1024;             // staging: 16 bytes of scales per row (one copy instruction)
constexpr int kF8Stage = kF8Codes + kF8Scales + 32 * 128;

template <int DQK, int DV, int NW, bool F8, bool SPLIT>
__global__ __launch_bounds__(64 * NW)
void sparse_attn_bf16_w32_kernel(const uint16_t* __restrict__ q, const void* __restrict__ kv,
                                 const int32_t* __restrict__ idx, uint16_t* __restrict__ out,
                                 float* __restrict__ lse, int Lq, int Lk, int t_begin, int H, int k,
                                 int64_t idx_bstride, float scale_log2, int cps,
                                 float* __restrict__ part_o, float* __restrict__ part_lse)
{
    using S = W32Shape<DQK, DV, NW>;
    constexpr int NC = S::NC;
    __shared__ __attribute__((aligned(16))) uint8_t ring[S::NBUF][S::BUF_BYTES];
    __shared__ __attribute__((aligned(16))) int32_t sel[S::KMAX];   // the query's index list (-1 padded)
    __shared__ int wlast[NW];                                       // per wave: last valid list position
    __shared__ __attribute__((aligned(16))) uint8_t stg[F8 ? 2 : 1][F8 ? kF8Stage : 16];

    const int row = blockIdx.x, b = blockIdx.y;
    const int t = t_begin + row;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int col = lane & 31, hi = lane >> 5;
    const int h = wave * 32 + col;

    const uint16_t* qrow = q + (((int64_t)b * Lq + t) * H + h) * DQK;
    v8bf qf[S::QC];
#pragma unroll
    for (int c = 0; c < S::QC; ++c) qf[c] = as_bf8(*(const u32x4*)(qrow + c * 16 + hi * 8));

    v16f o[S::DT];
#pragma unroll
    for (int i = 0; i < S::DT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int32_t* irow = idx + (int64_t)b * idx_bstride + (int64_t)row * k;
    const uint16_t* kvb = (const uint16_t*)kv + (F8 ? 0 : (int64_t)b * Lk * DQK);
    const uint8_t* kv8b = (const uint8_t*)kv + (F8 ? (int64_t)b * Lk * kF8Row : 0);
    // Stage the index list; entries that cannot be read become -1.  Chunks
    // past the last valid entry (a short row's -1 padding) are not visited.
    // Every load is issued before any is used (one memory round trip);
    // entries past k read entry k - 1 (k >= 1) and are dropped.
    int last = -1;
    {
        constexpr int EPT = S::KMAX / (64 * NW);     // list entries per thread
        static_assert(S::KMAX % (64 * NW) == 0, "whole list entries per thread");
        int32_t ent[EPT];
#pragma unroll
        for (int m = 0; m < EPT; ++m) ent[m] = irow[min(tid + 64 * NW * m, k - 1)];
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int i = tid + 64 * NW * m;
            const bool ok = i < k && ent[m] >= 0 && ent[m] < Lk;
            sel[i] = ok ? ent[m] : -1;
            last = ok ? i : last;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, kWave));
    if (lane == 0) wlast[wave] = last;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) last = max(last, wlast[w]);
    last = __builtin_amdgcn_readfirstlane(last);                   // workgroup-uniform
    // Split over the selected set (gridDim.z > 1): this workgroup takes chunks
    // [c0, c0 + cps) of the list and leaves a normalised partial output and
    // its log-sum-exp for the merge kernel.
    const int c0 = (int)blockIdx.z * cps;
    const int nchunks = max(0, min((last + NC) / NC - c0, cps));   // last = -1: nothing to attend
    // bit r set when entry r of chunk c is a real row
    auto valid_mask = [&](int c) -> uint32_t {
        return (uint32_t)__ballot(lane < NC && sel[c * NC + (lane & 31)] >= 0);
    };
    // this wave's copies of chunk c: RPW value parts, then its share of tails.
    // Padding entries copy row 0; they are masked in the softmax.
    auto issue_chunk = [&](int c) {
        if constexpr (F8) {
            // 21 copy instructions per chunk, instruction i on wave i % NW:
            // 16 of codes (2 rows each), 1 of scales (rows 0..31, the upper
            // half of the wave repeats them), 4 of rotary parts (8 rows each)
            const uint32_t sbase = lds_byte_address(stg[c & 1]);
#pragma unroll 1
            for (int i = wave; i < 21; i += NW) {
                int r, off;
                if (i < 16) {
                    r = 2 * i + (lane >> 5);
                    off = (lane & 31) * 16;
                } else if (i == 16) {
                    r = lane & 31;
                    off = 512;
                } else {
                    r = 8 * (i - 17) + (lane >> 3);
                    off = 528 + (lane & 7) * 16;
                }
                const int sr = max(sel[c * NC + r], 0);
                global_to_lds16_async(kv8b + (int64_t)sr * kF8Row + off,
                                      __builtin_amdgcn_readfirstlane(sbase + (uint32_t)i * 1024));
            }
            return;
        }
        const int32_t* rr_ = &sel[c * NC];
        int vr[S::RPW];
#pragma unroll
        for (int e = 0; e < S::RPW; e += 4) {
            const u32x4 x = *(const u32x4*)(rr_ + wave * S::RPW + e);   // same address on every lane
            vr[e] = (int)x[0]; vr[e + 1] = (int)x[1]; vr[e + 2] = (int)x[2]; vr[e + 3] = (int)x[3];
        }
        int trow[S::TI / NW];
#pragma unroll
        for (int j = 0; j < S::TI / NW; ++j) trow[j] = rr_[8 * (wave * (S::TI / NW) + j) + (lane >> 3)];
        const uint32_t vbase = __builtin_amdgcn_readfirstlane(lds_byte_address(ring[c % S::NBUF]));
#pragma unroll
        for (int e = 0; e < S::RPW; ++e) {
            const int r = wave * S::RPW + e;
            const int sr = max(__builtin_amdgcn_readfirstlane(vr[e]), 0);
            global_to_lds16_async(kvb + (int64_t)sr * DQK + lane * 8,
                                  __builtin_amdgcn_readfirstlane(vbase + (uint32_t)r * S::VPITCH));
        }
#pragma unroll
        for (int j = 0; j < S::TI / NW; ++j) {
            const int ti = wave * (S::TI / NW) + j;          // tail instruction: rows 8*ti .. 8*ti+7
            const int r = 8 * ti + (lane >> 3);
            const int sr = max(trow[j], 0);
            const int piece = (lane & 7) ^ (r & 7);
            global_to_lds16_async(kvb + (int64_t)sr * DQK + DV + piece * 8,
                                  __builtin_amdgcn_readfirstlane(vbase + (uint32_t)(S::VBYTES + ti * 1024)));
        }
    };

    const int js = (lane & 15) >> 2, qs = lane & 3, g2 = (lane >> 4) & 1;
    constexpr float kHeadroom = 64.f;                        // log2 units
    float m_seen = -INFINITY;                                // running true maximum (log2 domain)
    for (int pass = 0; pass < 2; ++pass) {
        bool overflow = false;
        // Iteration `it` computes chunk `it` and, once every wave is past
        // chunk it-1, issues chunk it+1 into the freed slot.
        for (int it = -1; it < nchunks; ++it) {
            wait_vmcnt0();                                   // this wave's copies of chunk it landed
            __syncthreads();                                 // all of chunk it visible; chunk it-1 consumed
            const int c = c0 + (it < 0 ? 0 : it);
            const uint32_t vmask = valid_mask(c);
            const uint8_t* cur = ring[c % S::NBUF];
            if constexpr (F8) {
                if (it >= 0) {
                    // staging -> ring: 8 codes per unit (dims 8j..8j+7 of row r)
                    const uint8_t* sg = stg[c & 1];
                    uint8_t* rg = ring[c % S::NBUF];
#pragma unroll 1
                    for (int u = tid; u < 32 * 64; u += 64 * NW) {
                        const int r = u >> 6, j = u & 63;
                        const u32x2 cw = *(const u32x2*)(sg + r * 512 + 8 * j);
                        const float sc = *(const float*)(sg + kF8Codes + r * 16 + 4 * (j >> 4));
                        u32x4 o4;
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[e], false);
                            const f32x2_t hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[e], true);
                            // code * scale is exact with few significant bits: keep the top half
                            o4[2 * e] = (__float_as_uint(lo[0] * sc) >> 16) | (__float_as_uint(lo[1] * sc) & 0xFFFF0000u);
                            o4[2 * e + 1] = (__float_as_uint(hi2[0] * sc) >> 16) |
                                            (__float_as_uint(hi2[1] * sc) & 0xFFFF0000u);
                        }
                        *(u32x4*)(rg + r * S::VPITCH + 16 * j) = o4;
                    }
                    // rotary parts: piece p of row r to its swizzled tail position
#pragma unroll 1
                    for (int u = tid; u < 32 * 8; u += 64 * NW) {
                        const int r = u >> 3, pc = u & 7;
                        const u32x4 x = *(const u32x4*)(sg + kF8Codes + kF8Scales + r * 128 + pc * 16);
                        *(u32x4*)(rg + S::VBYTES + (r >> 3) * 1024 + ((r & 7) * 8 + (pc ^ (r & 7))) * 16) = x;
                    }
                    __syncthreads();
                }
            }

            // S^T (32 rows x 32 heads); key fragments read kPre steps ahead.
            // Step c2 < DV/16 reads value-part piece 2*c2 + hi of row
            // slot_row(col); later steps read the tail.
            v16f sacc;
#pragma unroll
            for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
            if (it >= 0) {
                const int krow_i = slot_row(col);
                const uint8_t* vrow = cur + krow_i * S::VPITCH + hi * 16;
                const uint8_t* trow = cur + S::VBYTES + krow_i * (S::TP * 16);
                const int tsw = krow_i & 7;
                auto kfrag = [&](int c2) -> u32x4 {
                    if (c2 < DV / 16) return *(const u32x4*)(vrow + 32 * c2);
                    return *(const u32x4*)(trow + (((2 * (c2 - DV / 16) + hi) ^ tsw) << 4));
                };
                constexpr int kPre = 7;
                u32x4 kf[kPre + 1];
#pragma unroll
                for (int i = 0; i < kPre; ++i) kf[i] = kfrag(i);
#pragma unroll
                for (int c2 = 0; c2 < S::QC; ++c2) {
                    if (c2 + kPre < S::QC) kf[(c2 + kPre) % (kPre + 1)] = kfrag(c2 + kPre);
                    sacc = mfma_bf16_32x32x16(as_bf8(kf[c2 % (kPre + 1)]), qf[c2], sacc);
                    // keep the reads kPre steps ahead: no instruction crosses this point
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // queue the next chunk (while the last QK MFMAs drain)
            if (it + 1 < nchunks) issue_chunk(c0 + it + 1);
            if (it < 0) continue;

            // Softmax of head h over the chunk's rows.  Probabilities only
            // need the reference m (fixed at the first chunk with a valid row),
            // so they feed the PV product right away; the chunk maximum (for
            // the overflow check) is taken afterwards, off the critical path.
            if (vmask == 0u) continue;                       // nothing selected here (uniform)
            if (vmask != 0xFFFFFFFFu) {
                // element v holds chunk row slot_row(8 (v/4) + 4 hi + v%4) = hi + rv(v)
                const uint32_t vmh = vmask >> hi;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int rv = slot_row(8 * (v >> 2) + (v & 3));
                    sacc[v] = ((vmh >> rv) & 1u) ? sacc[v] : -INFINITY;
                }
            }
            if (__any(m == -INFINITY)) {                     // first chunk holding a valid row
                float cmax0 = -INFINITY;
#pragma unroll
                for (int v = 0; v < 16; ++v) cmax0 = fmaxf(cmax0, sacc[v]);
                m = fmaxf(cmax0, __shfl_xor(cmax0, 32, kWave)) * scale_log2;
            }
            if (__any(overflow)) {                           // only the maximum is still tracked
                float cm = -INFINITY;
#pragma unroll
                for (int v = 0; v < 16; ++v) cm = fmaxf(cm, sacc[v]);
                m_seen = fmaxf(m_seen, fmaxf(cm, __shfl_xor(cm, 32, kWave)) * scale_log2);
                continue;
            }
            const float negm = -m;
            uint32_t pw[8];
            float psum = 0.f, cmax = -INFINITY;
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                // masked entries are -inf: exp2(-inf) = 0
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[v], scale_log2, negm));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[v + 1], scale_log2, negm));
                psum += p0 + p1;
                cmax = fmaxf(cmax, fmaxf(sacc[v], sacc[v + 1]));
                pw[v >> 1] = pack_bf16x2(p0, p1);
            }

            // O^T += V^T . P^T, two 16-row K steps.  K slot (a, j) of lane group
            // hi is S^T row slot 16*tt + 8a + 4*hi + j, i.e. chunk row
            // 16*tt + 2a + hi + 4j; the lane reads dims dt*32 + 16*g2 + 4*qs ..
            // +3 of its source row (8 bytes at 64*dt + 32*g2 + 8*qs).
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const v8bf pfrag = as_bf8(u32x4{pw[4 * tt], pw[4 * tt + 1], pw[4 * tt + 2], pw[4 * tt + 3]});
                const int r0 = 16 * tt + hi + 4 * js, r1 = r0 + 2;
                const uint8_t* v0 = cur + r0 * S::VPITCH + 32 * g2 + 8 * qs;
                const uint8_t* v1 = cur + r1 * S::VPITCH + 32 * g2 + 8 * qs;
#pragma unroll
                for (int dt = 0; dt < S::DT; ++dt) {
                    const v4s lo4 = lds_read_tr16(v0 + 64 * dt);
                    const v4s hi4 = lds_read_tr16(v1 + 64 * dt);
                    const u32x2 a = __builtin_bit_cast(u32x2, lo4);
                    const u32x2 bq = __builtin_bit_cast(u32x2, hi4);
                    o[dt] = mfma_bf16_32x32x16(as_bf8(u32x4{a[0], a[1], bq[0], bq[1]}), pfrag, o[dt]);
                }
            }
            // bookkeeping that overlaps the PV MFMAs: sum and maximum
            psum += __shfl_xor(psum, 32, kWave);
            l += psum;
            cmax = fmaxf(cmax, __shfl_xor(cmax, 32, kWave)) * scale_log2;
            m_seen = fmaxf(m_seen, cmax);
            overflow = overflow || (cmax > m + kHeadroom);
        }
        // every wave must agree before the ring is reused by a second pass
        if (!__syncthreads_or(overflow ? 1 : 0)) break;
        // recompute with the true maximum as the reference
        m = m_seen;
        l = 0.f;
#pragma unroll
        for (int i = 0; i < S::DT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
    }

    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    const float lse_row = (l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
    if constexpr (SPLIT) {
        // partial (b, row, split z, head h): fp32, normalised by its own sum
        const int64_t pr = ((int64_t)b * gridDim.x + row) * gridDim.z + blockIdx.z;
        float* prow = part_o + (pr * H + h) * DV;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = dt * 32 + 8 * g + 4 * hi;
                *(v4f*)(prow + d0) = v4f{o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                                         o[dt][4 * g + 3] * inv};
            }
        if (hi == 0) part_lse[pr * H + h] = lse_row;
    } else {
        uint16_t* orow = out + (((int64_t)b * Lq + t) * H + h) * DV;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = dt * 32 + 8 * g + 4 * hi;
                const uint32_t w0 = pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv);
                const uint32_t w1 = pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
                *(u32x2*)(orow + d0) = u32x2{w0, w1};
            }
        if (lse != nullptr && hi == 0)
            lse[((int64_t)b * Lq + t) * H + h] = lse_row;
    }
}

// bf16 kernel for rows of D = d_qk = d_v in {64, 128} (the MQA shapes) with
// the head counts attn_mqa.hip does not take (H / 16 waves not 1, 2, 4 or 8,
// or not dividing D / 16): one workgroup per query row, one wave per 16
// heads, v_mfma_f32_16x16x32_bf16.
//  - The query's index list (k <= 2048) is staged in LDS once; the selected
//    rows stream through a two-slot LDS ring of 32 rows, copied
//    asynchronously one chunk ahead, 1 KB (1024 / 2D rows) per copy
//    instruction.  At 24 KB of LDS six rows share a CU, which hides the
//    copies' latency better than a deeper ring (four slots measured 1.7x
//    slower).  Piece p (16 bytes) of row r sits at position
//    p ^ (r % (D / 8)), so the 16 rows a key-fragment read gathers at one
//    piece, and the rows of a transpose read, hit distinct banks.
//  - S^T = K_chunk . Q^T per 16-key tile; element i of lane group g holds
//    chunk row 16 j + g + 4 i (the key-tile rows are read permuted).
//  - Online softmax in fp32 (exp2 domain) with the usual rescaling of the
//    16 x D output accumulators when the running maximum grows.
//  - O^T += V^T . P^T with K = 32 keys: P^T is the two S^T tiles converted to
//    bf16 in place, and V^T comes from the row-major chunk through LDS
//    transpose reads over the same key slots (rows g + 4 q, and 16 more).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW)
void sparse_attn_bf16_w16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                 const int32_t* __restrict__ idx, uint16_t* __restrict__ out,
                                 float* __restrict__ lse, int Lq, int Lk, int t_begin, int H, int k,
                                 int64_t idx_bstride, float scale_log2)
{
    constexpr int NC = 32;                       // rows per chunk
    constexpr int PPR = D / 8;                   // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;                // rows per copy instruction
    constexpr int SLOT = NC * D * 2;             // ring bytes per chunk
    constexpr int NBUF = 2;                      // ring slots: copies run one chunk ahead
    constexpr int KMAX = 2048;
    static_assert(D == 64 || D == 128, "64- or 128-wide rows");
    __shared__ __attribute__((aligned(16))) uint8_t ring[NBUF][SLOT];
    __shared__ __attribute__((aligned(16))) int32_t sel[KMAX];
    __shared__ int wlast[NW];

    const int row = blockIdx.x, b = blockIdx.y;
    const int t = t_begin + row;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4, i16 = lane & 15;
    const int h = wave * 16 + col;

    // Q^T operand: head h, dims 32 c + 8 g .. +8
    const uint16_t* qrow = q + (((int64_t)b * Lq + t) * H + h) * D;
    v8bf qf[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[c] = as_bf8(*(const u32x4*)(qrow + 32 * c + 8 * g));

    const int32_t* irow = idx + (int64_t)b * idx_bstride + (int64_t)row * k;
    // Every load is issued before any is used (one memory round trip);
    // entries past k read entry k - 1 (k >= 1) and are dropped.
    int last = -1;
    {
        constexpr int EPT = (KMAX + 64 * NW - 1) / (64 * NW);   // list entries per thread
        int32_t ent[EPT];
#pragma unroll
        for (int m = 0; m < EPT; ++m) ent[m] = irow[min(tid + 64 * NW * m, k - 1)];
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int i = tid + 64 * NW * m;
            if (i < KMAX) {
                const bool ok = i < k && ent[m] >= 0 && ent[m] < Lk;
                sel[i] = ok ? ent[m] : -1;
                last = ok ? i : last;
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, kWave));
    if (lane == 0) wlast[wave] = last;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) last = max(last, wlast[w]);
    const int nch = __builtin_amdgcn_readfirstlane((last + NC) / NC);

    const uint16_t* kvb = kv + (int64_t)b * Lk * D;
    // copies of chunk c: instruction i covers rows RPI i .. RPI i + RPI - 1,
    // lane l row RPI i + l / PPR, position l % PPR, piece (l % PPR) ^ (row % PPR)
    auto issue = [&](int c) {
        const uint32_t base = lds_byte_address(ring[c % NBUF]);
        for (int i = wave; i < NC / RPI; i += NW) {
            const int r = RPI * i + lane / PPR;
            const int sr = max(sel[c * NC + r], 0);
            const int piece = (lane % PPR) ^ (r % PPR);
            global_to_lds16_async(kvb + (int64_t)sr * D + 8 * piece,
                                  __builtin_amdgcn_readfirstlane(base + (uint32_t)(i * 1024)));
        }
    };
    // byte offset of 16-bit column d (multiple of 4) of chunk row r
    auto off = [](int r, int d) -> uint32_t {
        return (uint32_t)(r * D * 2 + ((((d >> 3) ^ (r % PPR))) << 4) + 2 * (d & 7));
    };

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    v4f o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = zero;
    float m = -INFINITY, l = 0.f;

    if (nch > 0) issue(0);
    for (int ch = 0; ch < nch; ++ch) {
        const int c0 = ch * NC;
        wait_vmcnt0();
        __syncthreads();                                           // chunk ch landed; chunk ch - 1 consumed
        if (ch + 1 < nch) issue(ch + 1);                           // into chunk ch - 1's slot
        const uint8_t* cur = ring[ch % NBUF];

        // S^T tiles
        v4f st[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 16 * j + 4 * (col & 3) + (col >> 2);
            v4f a = zero;
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
                a = mfma_bf16_16x16x32(as_bf8(*(const u32x4*)(cur + off(r, 32 * c + 8 * g))), qf[c], a);
            st[j] = a;
        }
        // online softmax of head h over the chunk's rows 16 j + g + 4 i
        float z[8], mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = sel[c0 + 16 * j + g + 4 * i] >= 0;
                const float v = valid ? st[j][i] * scale_log2 : -INFINITY;
                z[4 * j + i] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float m_new = fmaxf(m, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m - m_new);
        float psum = 0.f;
        uint32_t pb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p0 = (z[2 * e] == -INFINITY) ? 0.f : exp2f(z[2 * e] - m_new);
            const float p1 = (z[2 * e + 1] == -INFINITY) ? 0.f : exp2f(z[2 * e + 1] - m_new);
            psum += p0 + p1;
            pb[e] = pack_bf16x2(p0, p1);
        }
        psum += __shfl_xor(psum, 16, kWave);
        psum += __shfl_xor(psum, 32, kWave);
        l = l * alpha + psum;
        m = m_new;
        const v8bf pfrag = as_bf8(u32x4{pb[0], pb[1], pb[2], pb[3]});
        // O^T tiles: A = V^T over key slots 8 g + q (rows g + 4 q) and
        // 8 g + 4 + q (rows 16 + g + 4 q), dims 16 dt + col
        const int rl = g + 4 * (i16 >> 2);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const int d = 16 * dt + 4 * (i16 & 3);
            const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(cur + off(rl, d)));
            const u32x2 hi2 = __builtin_bit_cast(u32x2, lds_read_tr16(cur + off(rl + 16, d)));
            v4f acc = o[dt];
            acc[0] *= alpha; acc[1] *= alpha; acc[2] *= alpha; acc[3] *= alpha;
            o[dt] = mfma_bf16_16x16x32(as_bf8(u32x4{lo[0], lo[1], hi2[0], hi2[1]}), pfrag, acc);
        }
    }

    // O^T tile dt: lane (head col, group g) holds dims 16 dt + 4 g .. +3
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    uint16_t* orow = out + (((int64_t)b * Lq + t) * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        const uint32_t w0 = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
        const uint32_t w1 = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
        *(u32x2*)(orow + 16 * dt + 4 * g) = u32x2{w0, w1};
    }
    if (lse != nullptr && g == 0)
        lse[((int64_t)b * Lq + t) * H + h] = (l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// Merge of the split partials: per (b, row, head), the log-sum-exp of the
// parts and the parts' outputs weighted by exp(lse_z - lse), in fp32, then
// rounded to bf16.  One thread per 4 output values; the parts are summed in
// split order, so the result is deterministic.
constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads)
void attn_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                       uint16_t* __restrict__ out, float* __restrict__ lse, int64_t n_items, int rows, int Lq,
                       int t_begin, int nsplit, int H, int DV)
{
    const int64_t i = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    if (i >= n_items) return;
    const int q4 = DV / 4;
    const int d4 = (int)(i % q4);
    int64_t rest = i / q4;
    const int h = (int)(rest % H);
    rest /= H;
    const int row = (int)(rest % rows);
    const int b = (int)(rest / rows);
    const int64_t pr0 = ((int64_t)b * rows + row) * nsplit;
    float mx = -INFINITY;
    for (int z = 0; z < nsplit; ++z) mx = fmaxf(mx, part_lse[(pr0 + z) * H + h]);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    if (mx != -INFINITY) {
        for (int z = 0; z < nsplit; ++z) {
            const float wz = expf(part_lse[(pr0 + z) * H + h] - mx);
            const v4f x = *(const v4f*)(part_o + ((pr0 + z) * H + h) * DV + 4 * d4);
            den += wz;
            acc[0] = fmaf(wz, x[0], acc[0]);
            acc[1] = fmaf(wz, x[1], acc[1]);
            acc[2] = fmaf(wz, x[2], acc[2]);
            acc[3] = fmaf(wz, x[3], acc[3]);
        }
        const float inv = 1.f / den;
        acc[0] *= inv; acc[1] *= inv; acc[2] *= inv; acc[3] *= inv;
    }
    const int64_t orow = ((int64_t)b * Lq + t_begin + row) * H + h;
    *(u32x2*)(out + orow * DV + 4 * d4) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    if (lse != nullptr && d4 == 0) lse[orow] = (mx != -INFINITY) ? mx + logf(den) : -INFINITY;
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

int sparse_attn_split(int64_t rows, int H, int Dqk, int Dv, int k, bool bf16)
{
    // the 32-head kernel over few query rows: split each row's selected set
    // so that about 256 workgroups run, at least 4 chunks of 32 rows each
    if (!bf16 || (H != 32 && H != 64 && H != 128) || Dqk != 576 || Dv != 512 || k > 2048 || rows <= 0 ||
        rows >= 128)
        return 1;
    const int nch = (k + 31) / 32;
    int ns = (int)((256 + rows - 1) / rows);
    ns = ns < 8 ? ns : 8;
    ns = ns < nch / 4 ? ns : nch / 4;
    return ns > 1 ? ns : 1;
}

size_t sparse_attn_counter_bytes(int64_t rows, int H, int Dqk, int Dv, int k, bool bf16)
{
    if (!bf16 || (H != 32 && H != 64 && H != 128) || Dqk != 576 || Dv != 512 || k > 2048 || rows <= 0) return 0;
    return sparse_attn_split(rows, H, Dqk, Dv, k, bf16) == 1 ? 256 : 0;
}

size_t sparse_attn_split_bytes(int64_t rows, int H, int Dv, int nsplit)
{
    if (nsplit <= 1) return 0;
    return (size_t)rows * nsplit * H * (Dv + 1) * sizeof(float);
}

bool sparse_attn_bf16_supported(int Dqk, int Dv)
{
    return (Dqk == 576 && Dv == 512) || (Dqk == 128 && Dv == 128) || (Dqk == 64 && Dv == 64);
}

template <int DQK, int DV, int NW, bool F8>
hipError_t launch_bf16_w32(const AttnLaunch& a, hipStream_t s)
{
    const float scale_log2 = a.scale * 1.4426950408889634f;
    const int ns = (a.nsplit > 1 && a.part != nullptr) ? a.nsplit : 1;
    const int nch = (a.k + 31) / 32;
    const int cps = (nch + ns - 1) / ns;
    float* part_o = a.part;
    float* part_lse = ns > 1 ? a.part + (size_t)a.B * a.t_count * ns * a.H * DV : nullptr;
    if (!F8 && DQK == 576 && DV == 512) {
        // bf16 latent rows: the scheduled kernel of attn_mla.hip
        hipError_t e = launch_sparse_attn_mla(a, s, ns, cps, part_o, part_lse);
        if (e != hipSuccess || ns == 1) return e;
    } else if (ns == 1) {
        hipLaunchKernelGGL((sparse_attn_bf16_w32_kernel<DQK, DV, NW, F8, false>), dim3(a.t_count, a.B, 1),
                           dim3(64 * NW), 0, s, (const uint16_t*)a.q, a.kv, a.idx, (uint16_t*)a.out, a.lse,
                           a.Lq, a.Lk, a.t_begin, a.H, a.k, a.idx_bstride, scale_log2, cps, part_o, part_lse);
        return hipGetLastError();
    } else {
        hipLaunchKernelGGL((sparse_attn_bf16_w32_kernel<DQK, DV, NW, F8, true>), dim3(a.t_count, a.B, ns),
                           dim3(64 * NW), 0, s, (const uint16_t*)a.q, a.kv, a.idx, (uint16_t*)a.out, a.lse,
                           a.Lq, a.Lk, a.t_begin, a.H, a.k, a.idx_bstride, scale_log2, cps, part_o, part_lse);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t n_items = (int64_t)a.B * a.t_count * a.H * (DV / 4);
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((n_items + kMergeThreads - 1) / kMergeThreads)),
                       dim3(kMergeThreads), 0, s, part_o, part_lse, (uint16_t*)a.out, a.lse, n_items, a.t_count,
                       a.Lq, a.t_begin, ns, a.H, DV);
    return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_bf16_w32_any(const AttnLaunch& a, hipStream_t s, bool* handled)
{
    *handled = true;
    if (a.kv_fp8) {
        switch (a.H / 32) {
        case 1: return launch_bf16_w32<DQK, DV, 1, true>(a, s);
        case 2: return launch_bf16_w32<DQK, DV, 2, true>(a, s);
        case 4: return launch_bf16_w32<DQK, DV, 4, true>(a, s);
        }
    } else {
        switch (a.H / 32) {
        case 1: return launch_bf16_w32<DQK, DV, 1, false>(a, s);
        case 2: return launch_bf16_w32<DQK, DV, 2, false>(a, s);
        case 4: return launch_bf16_w32<DQK, DV, 4, false>(a, s);
        }
    }
    *handled = false;
    return hipSuccess;
}

hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.t_count == 0) return hipSuccess;
    if (a.kv_fp8) {
        // FP8 latent rows: the 32-head kernel only (checked by the caller)
        bool handled = false;
        hipError_t e = hipErrorInvalidValue;
        if (a.bf16 && a.H % 32 == 0 && a.k <= 2048 && a.Dqk == 576 && a.Dv == 512)
            e = launch_bf16_w32_any<576, 512>(a, s, &handled);
        return handled ? e : hipErrorInvalidValue;
    }
    if (a.bf16 && a.H % 32 == 0 && a.k <= 2048) {
        bool handled = false;
        hipError_t e = hipSuccess;
        if (a.Dqk == 576 && a.Dv == 512) e = launch_bf16_w32_any<576, 512>(a, s, &handled);
        if (handled) return e;
    }
    if (a.bf16 && a.Dqk == a.Dv && sparse_attn_mqa_supported(a.H, a.Dqk, a.k, a.Lk))
        return launch_sparse_attn_mqa(a, s);
    if (a.bf16 && a.k <= 2048 && a.Dqk == a.Dv && (a.Dqk == 128 || a.Dqk == 64)) {
        const float scale_log2 = a.scale * 1.4426950408889634f;
#define DSA_W16(D, NW)                                                                                          \
        hipLaunchKernelGGL((sparse_attn_bf16_w16_kernel<D, NW>), dim3(a.t_count, a.B), dim3(64 * NW), 0, s,    \
                           (const uint16_t*)a.q, (const uint16_t*)a.kv, a.idx, (uint16_t*)a.out, a.lse, a.Lq,  \
                           a.Lk, a.t_begin, a.H, a.k, a.idx_bstride, scale_log2)
#define DSA_W16_NW(D)                                                                                           \
        switch (a.H / 16) {                                                                                     \
        case 1: DSA_W16(D, 1); break;                                                                           \
        case 2: DSA_W16(D, 2); break;                                                                           \
        case 3: DSA_W16(D, 3); break;                                                                           \
        case 4: DSA_W16(D, 4); break;                                                                           \
        case 5: DSA_W16(D, 5); break;                                                                           \
        case 6: DSA_W16(D, 6); break;                                                                           \
        case 7: DSA_W16(D, 7); break;                                                                           \
        case 8: DSA_W16(D, 8); break;                                                                           \
        default: return hipErrorInvalidValue;                                                                   \
        }
        if (a.Dqk == 128) { DSA_W16_NW(128) } else { DSA_W16_NW(64) }
#undef DSA_W16_NW
#undef DSA_W16
        return hipGetLastError();
    }
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
