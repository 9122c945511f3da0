// Lightning-indexer scores on gfx950.
//
// I[t,s] = k_scale[s] * sum_j (w[t,j] * q_scale[t,j]) * ReLU(q8[t,j,:] . k8[s,:])
// for s <= t_pos ("DeepseekV3.2 拆解", section 核心组件, indexer equation; the
// FP8 format and the ReLU are the page's choices for throughput).
//
// FP8 kernel.  With ReLU(x) = (x + |x|) / 2 the score splits into a linear part
// and an absolute part:
//   I[t,s] = k_scale[s] * ( c[t,:] . k8[s,:]  +  sum_j v[t,j] * |q8[t,j,:] . k8[s,:]| )
//   v[t,j] = w[t,j] * q_scale[t,j] / 2,   c[t,d] = sum_j v[t,j] * q8[t,j,d].
// The absolute part costs one fused multiply-add per (query, key, head) (the
// |.| is a free source modifier), half the vector work of max + fma; the
// linear part is one 128-long dot product per (query, key), done on the bf16
// matrix cores with c split into three bf16 parts (keys are exact in bf16).
//
// Layout (H^I = 64 heads, d^I = 128):
//  - one workgroup = 4 waves = one block of 16 query rows;
//  - wave w keeps the e4m3 query fragments of heads 16w..16w+15 for the 16
//    rows in registers (one 16x128 MFMA operand per head, 8 VGPRs each) and
//    the bf16 parts of c for dims {32g + 8w + e : g < 4, e < 8};
//  - keys stream through a two-slot LDS tile in groups of 64 (8 KB), copied
//    global -> LDS asynchronously one group ahead;
//  - per 16-key tile a wave runs 3 bf16 MFMAs (its slice of the linear part)
//    and 16 v_mfma_f32_16x16x128_f8f6f4 (one per head, fresh fp32 accumulator:
//    K = 128 = d^I, so there is no long FP8 accumulation chain), each followed
//    by four |.|-fmas into the tile's accumulator;
//  - the four waves' partial sums meet in LDS, are multiplied by the key
//    scale, masked causally and written as fp32.
// The MFMA operand roles are A = keys (M), B = queries (N), so a lane's four
// outputs are four consecutive keys of one query and its head weight is one
// scalar per head.
#include "hw.h"
#include "launch.h"

#include <algorithm>

namespace dsa {

namespace {

constexpr int kQB = 16;        // query rows per workgroup
constexpr int kKG = 64;        // keys per LDS group (4 MFMA tiles of 16)
constexpr int kD = 128;        // indexer dim (bytes per key / per query head)
constexpr int kH = 64;         // indexer heads
constexpr int kHPW = 16;       // heads per wave
constexpr int kThreads = 256;  // 4 waves

// Byte offset of 16-byte chunk `c` (0..7) of row `r` of the LDS key tile.  The
// chunks of a row are permuted by (r >> 1) & 7, so 16 consecutive rows read at
// one logical chunk cover all 64 banks exactly once.
__device__ __forceinline__ int ktile_off(int r, int c) { return r * kD + ((c ^ ((r >> 1) & 7)) << 4); }

// Round to bf16 (nearest even) and return the rounded value as fp32.
__device__ __forceinline__ float round_bf16(float x) { return bf16_bits_to_f32(pack_bf16x2(x, 0.f) & 0xFFFFu); }

// The block kernel's other modes (rows indexed b * Lq + t):
//  - kshift > 0: the sample pass.  Key j of the launch is key s = j << kshift
//    of the sequence, row t takes j <= t_pos >> kshift, and the score of key
//    j goes to column j;
//  - flag non-null: the block runs only if one of its rows has flag != 0;
//  - CAND: no scores are stored.  The keys of a row whose score is >= tau[row]
//    are appended to the row's list in ascending s, as (score bits, s) pairs,
//    the first cap of them stored, and cand_cnt[row] gets their number.  A
//    row's keys must all be in one workgroup (no split over blockIdx.z): the
//    position of a group's entries is the row's running count, kept by every
//    thread of the row, plus the count of the group's lower keys.
struct IdxExt {
    int kshift;
    const int32_t* flag;
    const float* tau;
    uint32_t* cand;
    int32_t* cand_cnt;
    int cap;
    int* blk_ctr;
};

template <bool CAND>
__global__ __launch_bounds__(kThreads)
void indexer_fp8_kernel(const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
                        const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
                        const float* __restrict__ w, float* __restrict__ scores,
                        int Lq, int Lk, int q_pos0, int t_begin, int t_count,
                        int64_t sc_bstride, int64_t sc_rstride, int write_masked, int skip_upto_k, int gps,
                        IdxExt x)
{
    __shared__ __attribute__((aligned(16))) uint8_t ktile[2][kKG * kD];
    // [buffer][wave][row r * 16 + (quad e ^ r)]: wave w's partial sums of block
    // row r at keys 4e .. 4e+3 of the group; the XOR makes both the writes (16
    // rows at one quad) and the reads (one row, 16 quads) hit 16 distinct
    // 16-byte bank groups
    __shared__ __attribute__((aligned(16))) v4f red[2][4][16 * kQB];
    __shared__ __attribute__((aligned(16))) uint32_t cpart[3][kQB][kD / 2]; // bf16 pairs: hi, mid, lo

    const int nqb = (t_count + kQB - 1) / kQB;
    // Longest rows first.  With a block counter (keys not split), each
    // workgroup takes the next (sequence, row block) from it, so the GPU's
    // dies share the blocks by speed; the grid has about 1/8 more workgroups
    // than blocks and the late ones leave.  Which workgroup scores a block
    // does not change a score.
    int qb = nqb - 1 - (int)blockIdx.x, b = blockIdx.y;
    if (x.blk_ctr != nullptr) {
        __shared__ int s_blk;
        if (threadIdx.x == 0) s_blk = atomicAdd(x.blk_ctr, 1);
        __syncthreads();
        const int item = s_blk;
        if (item >= (int)gridDim.y * nqb) return;           // uniform over the workgroup
        const int b_ = item % (int)gridDim.y;               // the sequences' blocks interleaved
        b = __builtin_amdgcn_readfirstlane(b_);
        qb = __builtin_amdgcn_readfirstlane(nqb - 1 - item / (int)gridDim.y);
    }
    const int t0 = t_begin + qb * kQB;
    const int rows_here = min(kQB, t_begin + t_count - t0);
    const int tpos_last = q_pos0 + t0 + rows_here - 1;
    if (!write_masked && skip_upto_k > 0 && tpos_last + 1 <= skip_upto_k)
        return;
    if (x.flag) {
        int any = 0;
        for (int r = 0; r < rows_here; ++r) any |= x.flag[(int64_t)b * Lq + t0 + r];
        if (!any) return;
    }
    const int kshift = x.kshift;
    const int Lks = ((Lk - 1) >> kshift) + 1;          // keys of the launch (all of them when kshift = 0)
    // Key groups of this block: [g0, g1) of the ngroups its rows need (split
    // over blockIdx.z when there are few row blocks); a split past the
    // block's keys has nothing to do.
    const int ngroups = ((tpos_last >> kshift) + 1 + kKG - 1) / kKG;
    const int g0 = (int)blockIdx.z * gps;
    const int g1 = min(g0 + gps, ngroups);
    if (g0 >= g1)
        return;

    // The -inf upper triangle.  Block qb writes the masked tail of its mirror
    // block nqb-1-qb: columns [mfrom, Lk) of the mirror's rows, where mfrom
    // is the end of the groups the mirror computes itself.  The mirror's tail
    // is about as long as this block's row range, so the longest-computing
    // blocks (issued first) carry the longest tails, one 16-byte store per
    // thread per key group, while the MFMA work runs; the short blocks at the
    // end of the launch carry short tails.
    const int t0_m = t_begin + (nqb - 1 - qb) * kQB;
    const int rows_m = min(kQB, t_begin + t_count - t0_m);
    const int mfrom = ((q_pos0 + t0_m + rows_m - 1) / kKG + 1) * kKG;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;

    // Absolute part, operand B: row t0 + col, head j, bytes [32*grp, 32*grp + 32).
    const int tq = t0 + min(col, rows_here - 1);
    const int64_t qrow = (int64_t)b * Lq + tq;
    v8i qf[kHPW];
    float wv[kHPW];
#pragma unroll
    for (int h = 0; h < kHPW; ++h) {
        const int j = wave * kHPW + h;
        const u32x4* p = (const u32x4*)(q8 + (qrow * kH + j) * kD + grp * 32);
        qf[h] = as_i8(p[0], p[1]);
        wv[h] = 0.5f * w[qrow * kH + j] * q_scale[qrow * kH + j];
    }

    // Linear part: thread (row r, dims d0..d0+7) forms c[r, d] from all heads
    // (four interleaved partial sums, then a pairwise combine) and stores its
    // three-way bf16 split.
    {
        const int r = tid >> 4, d0 = (tid & 15) * 8;
        const int64_t row = (int64_t)b * Lq + t0 + min(r, rows_here - 1);
        float part[4][8];
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int e = 0; e < 8; ++e) part[p][e] = 0.f;
#pragma unroll 4
        for (int j = 0; j < kH; ++j) {
            const float v = 0.5f * w[row * kH + j] * q_scale[row * kH + j];
            const u32x2 u = *(const u32x2*)(q8 + (row * kH + j) * kD + d0);
            float x[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[h], false);
                const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[h], true);
                x[4 * h] = lo[0]; x[4 * h + 1] = lo[1]; x[4 * h + 2] = hi[0]; x[4 * h + 3] = hi[1];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) part[j & 3][e] = fmaf(v, x[e], part[j & 3][e]);
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            float hv[2], mv[2], lv[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float c = (part[0][e + k] + part[1][e + k]) + (part[2][e + k] + part[3][e + k]);
                hv[k] = round_bf16(c);
                const float r1 = c - hv[k];
                mv[k] = round_bf16(r1);
                lv[k] = r1 - mv[k];
            }
            cpart[0][r][(d0 + e) / 2] = pack_bf16x2(hv[0], hv[1]);
            cpart[1][r][(d0 + e) / 2] = pack_bf16x2(mv[0], mv[1]);
            cpart[2][r][(d0 + e) / 2] = pack_bf16x2(lv[0], lv[1]);
        }
    }

    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    // Keys of group g go global -> LDS by direct copies: chunk p (16 B) of the
    // swizzled tile is row p / 8, physical chunk p % 8, so each lane fetches the
    // logical chunk that belongs there.  Rows past Lk repeat key Lk - 1; their
    // outputs are never stored.
    const uint32_t ktile_lds = lds_byte_address(&ktile[0][0]);
    auto issue_keys = [&](int g, int slot) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int p = n * kThreads + tid;
            const int r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
            const int s = min(g * kKG + r, Lks - 1);
            const uint8_t* src = k8 + ((int64_t)b * Lk + ((int64_t)s << kshift)) * kD + c * 16;
            const uint32_t dst = ktile_lds + slot * (kKG * kD) + (n * kThreads + wave * kWave) * 16;
            global_to_lds16_async(src, __builtin_amdgcn_readfirstlane(dst));
        }
    };
    issue_keys(g0, g0 & 1);
    wait_vmcnt0();
    __syncthreads();

    // Linear part, operand B: query col, dims 32*grp + 8*wave + (0..7).
    v8bf cb[3];
#pragma unroll
    for (int p = 0; p < 3; ++p)
        cb[p] = as_bf8(*(const u32x4*)&cpart[p][col][(32 * grp + 8 * wave) / 2]);
    const int lin_chunk = 2 * grp + (wave >> 1), lin_byte = 8 * (wave & 1);

    // After each group's barrier, thread (wave, lane) finishes row
    // er = 4 wave + lane / 16 of the block at keys s0 + 4 eq .. + 3, eq =
    // lane % 16: a row's 64 keys lie in one 16-lane row of one wave, in
    // ascending s, so its scores leave as one 256-byte run and its
    // candidates are counted by a scan within the 16 lanes.
    const int er = 4 * wave + (lane >> 4), eq = lane & 15;
    // CAND: this thread's row, its threshold and its entries so far (the same
    // count in all 16 threads of the row).
    const int64_t crow = (int64_t)b * Lq + t0 + er;
    const bool cact = CAND && er < rows_here && q_pos0 + t0 + er + 1 > skip_upto_k;
    const float ctau = cact ? x.tau[crow] : INFINITY;
    uint32_t crun = 0;

    // Per group: the copy of group g+1 into the other tile slot runs while g
    // is computed; one wait + barrier publishes both the next key tile and
    // this group's partial sums (the reduction buffer is double-buffered too).
    for (int g = g0; g < g1; ++g) {
        const int s0 = g * kKG;
        const int kb = g & 1;
        const uint8_t* kt = ktile[kb];
        if (g + 1 < g1) issue_keys(g + 1, kb ^ 1);
        // key scales of the four keys this thread finishes after the barrier,
        // fetched now so the epilogue does not wait on memory
        const int sb = s0 + 4 * eq;
        float ksc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ksc[r] = k_scale[(int64_t)b * Lk + ((int64_t)min(sb + r, Lks - 1) << kshift)];
        // key fragments of tile i: the linear part's 8 bytes and the 32-byte
        // MFMA operand; those of tile i + 1 are read while tile i computes
        auto load_frag = [&](int i, u32x2& kk_, v8i& af_) {
            const int kr = i * 16 + col;
            kk_ = *(const u32x2*)(kt + ktile_off(kr, lin_chunk) + lin_byte);
            af_ = as_i8(*(const u32x4*)(kt + ktile_off(kr, 2 * grp)),
                        *(const u32x4*)(kt + ktile_off(kr, 2 * grp + 1)));
        };
        u32x2 kk;
        v8i af;
        load_frag(0, kk, af);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x2 kk_next;
            v8i af_next;
            if (i + 1 < 4) load_frag(i + 1, kk_next, af_next);
            // linear part: this wave's 32 dims of c[col] . k[kr]
            u32x4 kbf;
            kbf[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kk[0], 1.0f, false));
            kbf[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kk[0], 1.0f, true));
            kbf[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kk[1], 1.0f, false));
            kbf[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kk[1], 1.0f, true));
            const v8bf ka = as_bf8(kbf);
            v4f acc = mfma_bf16_16x16x32(ka, cb[2], zero);
            acc = mfma_bf16_16x16x32(ka, cb[1], acc);
            acc = mfma_bf16_16x16x32(ka, cb[0], acc);
            // absolute part over the wave's 16 heads
            // software-pipelined: the MFMAs of heads h + 1 and h + 2 are in
            // flight while the result of head h is folded in
            v4f d = mfma_fp8_16x16x128(af, qf[0], zero);
            v4f d1 = mfma_fp8_16x16x128(af, qf[1], zero);
#pragma unroll
            for (int h = 0; h < kHPW; ++h) {
                const v4f d2 = (h + 2 < kHPW) ? mfma_fp8_16x16x128(af, qf[(h + 2) % kHPW], zero) : d1;
                __builtin_amdgcn_sched_barrier(0);           // keep the issue order written here
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf(wv[h], fabsf(d[r]), acc[r]);
                __builtin_amdgcn_sched_barrier(0);
                d = d1;
                d1 = d2;
            }
            red[kb][wave][col * 16 + ((4 * i + grp) ^ col)] = acc;
            if (i + 1 < 4) {
                kk = kk_next;
                af = af_next;
            }
        }
        wait_vmcnt0();
        __syncthreads();
        // sum the four waves' partials of row er, keys sb .. sb + 3
        const int rs = er * 16 + (eq ^ er);
        v4f sum = red[kb][0][rs];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            const v4f x = red[kb][ww][rs];
            sum[0] += x[0]; sum[1] += x[1]; sum[2] += x[2]; sum[3] += x[3];
        }
        if (write_masked) {
            // mirror tail: row tid / 16 of the mirror block, 4 columns per thread
            const int r = tid >> 4, s = mfrom + s0 + 4 * (tid & 15);
            if (r < rows_m && s < Lk) {
                float* dst = scores + (int64_t)b * sc_bstride + (int64_t)(t0_m + r - t_begin) * sc_rstride + s;
                if (s + 3 < Lk && ((uintptr_t)dst & 15u) == 0) {
                    *(v4f*)dst = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                } else {
                    for (int e = 0; e < 4 && s + e < Lk; ++e) dst[e] = -INFINITY;
                }
            }
        }
        if constexpr (CAND) {
            const int tpos = q_pos0 + t0 + er;
            float v[4];
            uint32_t m = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v[r] = sum[r] * ksc[r];
                m |= (cact && sb + r <= tpos && v[r] >= ctau) ? (1u << r) : 0u;
            }
            const uint32_t c = (uint32_t)__builtin_popcount(m);
            const uint32_t incl = row16_incl_scan(c);
            // the row's count: lane 15 of the 16-lane row, broadcast (DPP row_newbcast)
            const uint32_t total = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x15F, 0xF, 0xF, false);
            // entry positions past cap are clamped to the last slot: such a
            // row overflows, its list is never read
            const uint32_t pos = crun + incl - c;
            uint32_t* dst = x.cand + (size_t)crow * (size_t)x.cap * 2;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t pr = min(pos + (uint32_t)__builtin_popcount(m & ((1u << r) - 1u)), (uint32_t)x.cap - 1u);
                if (m & (1u << r)) *(u32x2*)(dst + 2 * (size_t)pr) = u32x2{__float_as_uint(v[r]), (uint32_t)(sb + r)};
            }
            crun += total;
        } else if (er < rows_here) {
            const int t = t0 + er;
            const int tpos = (q_pos0 + t) >> kshift;
            float* dst = scores + (int64_t)b * sc_bstride + (int64_t)(t - t_begin) * sc_rstride + sb;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = sb + r;
                v[r] = (s <= tpos) ? sum[r] * ksc[r] : -INFINITY;
            }
            const bool vec_ok = ((uintptr_t)dst & 15u) == 0;
            if (vec_ok && sb + 3 < Lks && (write_masked || sb + 3 <= tpos)) {
                *(v4f*)dst = v4f{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = sb + r;
                    if (s < Lks && (write_masked || s <= tpos)) dst[r] = v[r];
                }
            }
        }
    }

    if constexpr (CAND) {
        if (eq == 0 && er < rows_here) x.cand_cnt[crow] = cact ? (int32_t)crun : 0;
        return;
    }

    if (write_masked && g1 == ngroups) {
        // what is left of the mirror tail after one 64-column slice per group
        // (16-byte stores where the row allows, the ragged end one by one;
        // the split holding the last group writes it)
        const int s_from = mfrom + ngroups * kKG;
        const v4f ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        for (int r = 0; r < rows_m; ++r) {
            float* dst = scores + (int64_t)b * sc_bstride + (int64_t)(t0_m + r - t_begin) * sc_rstride;
            int s_vec = s_from, s_end = Lk;
            if (s_from < Lk && (((uintptr_t)(dst + s_from)) & 15u) == 0) {
                const int nvec = (Lk - s_from) >> 2;
                for (int i = tid; i < nvec; i += kThreads) *(v4f*)(dst + s_from + 4 * i) = ninf;
                s_vec = s_from + 4 * nvec;
            }
            for (int s = s_vec + tid; s < s_end; s += kThreads) dst[s] = -INFINITY;
        }
    }
}

// FP8 kernel for few query rows per sequence (decode): one workgroup per
// (query row, range of row_keys keys).  The MFMA's N dimension carries 16
// heads instead of 16 queries, so no work is spent on absent query rows:
// per 16-key tile a wave runs four v_mfma_f32_16x16x128_f8f6f4 (64 heads),
// folds ReLU and the head weights into four fp32 partial sums per lane, and
// sums them over the 16 lanes that hold the 16 heads of a key.  Keys are read
// straight from memory into the A operand, kTileAhead tiles ahead; the four
// waves take alternate tiles and need no workgroup synchronisation.
constexpr int kRowKeysMax = 8192;  // keys per workgroup at most (the LDS score row)
constexpr int kRowKeysMin = 2048;
constexpr int kTileAhead = 8;      // key tiles in flight per wave

// Sum over each 16-lane row of the wave (every lane of the row gets it): DPP
// row rotations by 8, 4, 2 and 1.
__device__ __forceinline__ float row16_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
    return x;
}

__global__ __launch_bounds__(kThreads)
void indexer_fp8_row_kernel(const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
                            const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
                            const float* __restrict__ w, float* __restrict__ scores,
                            int Lq, int Lk, int q_pos0, int t_begin,
                            int64_t sc_bstride, int64_t sc_rstride, int write_masked, int skip_upto_k,
                            int row_keys)
{
    const int t = t_begin + blockIdx.x;
    const int b = blockIdx.y;
    const int tpos = q_pos0 + t;
    if (skip_upto_k > 0 && tpos + 1 <= skip_upto_k)
        return;
    const int s_begin = blockIdx.z * row_keys;
    const int s_stop = min(s_begin + row_keys, Lk);           // this workgroup's key range
    const int s_end = min(s_stop, tpos + 1);                  // keys that get a score
    float* dst = scores + (int64_t)b * sc_bstride + (int64_t)(t - t_begin) * sc_rstride;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (write_masked)
        for (int s = max(s_end, s_begin) + tid; s < s_stop; s += kThreads) dst[s] = -INFINITY;
    if (s_end <= s_begin)
        return;

    // B operand: head 16 h + (lane % 16), bytes [32 (lane / 16), +32) of the query row
    const int hcol = lane & 15, grp = lane >> 4;
    const int64_t qrow = (int64_t)b * Lq + t;
    v8i qf[4];
    float wq[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int j = 16 * h + hcol;
        const u32x4* p = (const u32x4*)(q8 + (qrow * kH + j) * kD + grp * 32);
        qf[h] = as_i8(p[0], p[1]);
        wq[h] = w[qrow * kH + j] * q_scale[qrow * kH + j];
    }
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const int ntiles = (s_end - s_begin + 15) >> 4;
    // Tile i: A operand = key s_begin + 16 i + (lane % 16), 32-byte slice
    // lane / 16; and the key scales of keys s_begin + 16 i + 4 (lane / 16) + r,
    // which this lane's row of sums will hold.  Both are fetched together so
    // no load is waited on inside the MFMA step.  Every step loads a tile
    // (past the last one: the last one again) and the scores go to LDS, so
    // the number of memory instructions per step is fixed and the compiler's
    // waits keep kTileAhead tiles in flight; the row is stored at the end.
    __shared__ __attribute__((aligned(16))) float sc_lds[kRowKeysMax];
    struct Tile {
        v8i a;
        float ks[4];
    };
    auto load_tile = [&](int i) -> Tile {
        Tile tl;
        i = min(i, ntiles - 1);
        const int key = min(s_begin + 16 * i + hcol, Lk - 1);
        const u32x4* p = (const u32x4*)(k8 + ((int64_t)b * Lk + key) * kD + grp * 32);
        tl.a = as_i8(p[0], p[1]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            tl.ks[r] = k_scale[(int64_t)b * Lk + min(s_begin + 16 * i + 4 * grp + r, Lk - 1)];
        return tl;
    };
    Tile tf[kTileAhead];
#pragma unroll
    for (int a = 0; a < kTileAhead; ++a) tf[a] = load_tile(wave + 4 * a);
    for (int i0 = wave; i0 < ntiles; i0 += 4 * kTileAhead) {
#pragma unroll
        for (int a = 0; a < kTileAhead; ++a) {
            const int i = i0 + 4 * a;
            const Tile cur = tf[a];
            tf[a] = load_tile(i + 4 * kTileAhead);
            v4f acc = zero;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const v4f d = mfma_fp8_16x16x128(cur.a, qf[h], zero);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r] = fmaf(wq[h], __int_as_float(max(__float_as_int(d[r]), 0)), acc[r]);
            }
            // sum over the 16 lanes (heads) that share keys 4 (lane / 16) + r
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = row16_sum(acc[r]);
            if (hcol == 0 && i < ntiles)
                *(v4f*)&sc_lds[16 * i + 4 * grp] =
                    v4f{acc[0] * cur.ks[0], acc[1] * cur.ks[1], acc[2] * cur.ks[2], acc[3] * cur.ks[3]};
        }
    }
    __syncthreads();
    // keys s_begin .. s_end - 1: 16-byte stores where the row allows
    const int nk = s_end - s_begin;
    if (((uintptr_t)(dst + s_begin) & 15u) == 0) {
        for (int e = tid; e < nk / 4; e += kThreads) *(v4f*)(dst + s_begin + 4 * e) = *(const v4f*)&sc_lds[4 * e];
        for (int e = (nk & ~3) + tid; e < nk; e += kThreads) dst[s_begin + e] = sc_lds[e];
    } else {
        for (int e = tid; e < nk; e += kThreads) dst[s_begin + e] = sc_lds[e];
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

__global__ void zero_block_counter_kernel(int* __restrict__ p)
{
    if (threadIdx.x == 0) *p = 0;
}

constexpr int64_t kMinBlocks = 1024;    // below this many row blocks the keys are split too

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.t_count == 0) return hipSuccess;
    // The kernel is chosen by the whole problem's rows per sequence (a.Lq),
    // never by the tile's: both kernels round a row's sum differently, and a
    // forward in query-row tiles must give every row the scores the
    // whole-problem call gives it, whatever the size of its tile.
    if (a.fp8 && a.Lq < kQB / 2) {
        // few query rows per sequence: split the keys instead of blocking queries
        // Longer key ranges per workgroup while at least 512 workgroups (two
        // per CU) remain: each wave's prefetch ramp and drain are paid once
        // per range, and the launch fits in one round (64 x 65536 keys: 8192
        // keys per workgroup, 14% faster than 2048).  The partition does not
        // change any score.
        const int last = a.write_masked ? a.Lk : min(a.Lk, a.q_pos0 + a.t_begin + a.t_count);
        int rk = kRowKeysMax;
        while (rk > kRowKeysMin && (int64_t)a.t_count * a.B * ((last + rk - 1) / rk) < 512) rk /= 2;
        const int nz = (last + rk - 1) / rk;
        hipLaunchKernelGGL(indexer_fp8_row_kernel, dim3(a.t_count, a.B, nz), dim3(kThreads), 0, s,
                           (const uint8_t*)a.q, a.q_scale, (const uint8_t*)a.k, a.k_scale, a.w,
                           a.scores, a.Lq, a.Lk, a.q_pos0, a.t_begin,
                           a.sc_bstride, a.sc_rstride, (int)a.write_masked, a.skip_upto_k, rk);
    } else if (a.fp8) {
        // With fewer than 1024 row blocks the keys are split as well, so that
        // about 1024 workgroups run and the longest block's chain of key
        // groups is cut (splits past a block's keys return at once).
        const int nqb = (a.t_count + kQB - 1) / kQB;
        const int64_t tpos_end = (int64_t)a.q_pos0 + a.t_begin + a.t_count;   // largest t_pos + 1
        const int gmax = (int)((((tpos_end - 1) >> a.kshift) + kKG) / kKG);
        const int64_t blocks = (int64_t)nqb * a.B;
        const bool cand = a.tau != nullptr;
        int nz = (blocks >= kMinBlocks || cand) ? 1
                 : (int)std::min<int64_t>((kMinBlocks + blocks - 1) / blocks, gmax);
        const int gps = (gmax + nz - 1) / nz;
        nz = (gmax + gps - 1) / gps;
        const IdxExt x{a.kshift, a.flag, a.tau, a.cand, a.cand_cnt, a.cap, nz == 1 ? a.blk_ctr : nullptr};
        unsigned gx = (unsigned)nqb;
        if (x.blk_ctr != nullptr) {
            // the counter is cleared by a kernel (not a memset): the pair can be captured in a graph
            hipLaunchKernelGGL(zero_block_counter_kernel, dim3(1), dim3(64), 0, s, x.blk_ctr);
            const int64_t items = (int64_t)nqb * a.B;
            const int64_t g = (items + items / 8 + 64 + a.B - 1) / a.B;   // workgroups per sequence row of the grid
            gx = (unsigned)g;
        }
        hipLaunchKernelGGL(cand ? indexer_fp8_kernel<true> : indexer_fp8_kernel<false>, dim3(gx, a.B, nz),
                           dim3(kThreads), 0, s,
                           (const uint8_t*)a.q, a.q_scale, (const uint8_t*)a.k, a.k_scale, a.w,
                           a.scores, a.Lq, a.Lk, a.q_pos0, a.t_begin, a.t_count,
                           a.sc_bstride, a.sc_rstride, (int)a.write_masked, a.skip_upto_k, gps, x);
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
