// Sparse MQA attention over the selected latent rows for the MLA shape
// (576-wide bf16 rows, value = the first 512 columns, 32/64/128 heads, k <=
// 2048) on gfx950 ("DeepseekV3.2 拆解", section 核心组件: u_t = Attn(h_t,
// {c_s : s in top-k}); the latent row is key and value because the key
// up-projection is absorbed into the query, "DeepSeek模型架构创新解析"
// section 1.1).
//
// One workgroup per query row (per split of its selected set for few rows),
// one wave per 32 heads, v_mfma_f32_32x32x16_bf16 throughout, in the LDS
// layout of attn_layout.h (value parts at a 1040-byte pitch, tails packed 8
// rows per 1 KB, S^T row slot m holding chunk row slot_row(m)):
//  - S^T[32 rows x 32 heads] = K_chunk . Q^T with the query operand (36 steps
//    of 32 heads x 16 dims) in registers for the whole row, accumulated in
//    VGPRs (inline MFMAs) while O^T fills the 256 AGPRs;
//  - softmax in fp32 (exp2 domain) against a per-head reference maximum m
//    fixed at the first chunk holding a valid row, so O is never rescaled; a
//    logit more than 64 (log2 units) above m makes the workgroup recompute
//    the row once with the true maximum;
//  - O^T[32 dims x 32 heads] += V^T . P^T with P^T the S^T accumulator in
//    bf16 in place and V^T from LDS transpose reads.
// The schedule is what differs from the 32-head kernel in sparse_attn.hip,
// which measured (cycle stamps per chunk and wave) about 680 cycles issuing
// its row copies in one burst after Q.K and 920 cycles of softmax between
// Q.K and P.V, of about 4700:
//  - the ring holds three chunks, and the copies of chunk i+2 are issued one
//    at a time between the Q.K MFMAs of chunk i, so the CU's memory path
//    moves them while the matrix units work and they have two iterations to
//    land;
//  - the softmax needs no cross-lane step per chunk: each half-wave keeps
//    its own partial sum and running maximum (combined once per row), and
//    checks its own logits against m;
//  - the second half of the softmax (rows of the second 16-key step) runs
//    between the MFMAs of the first P.V step.
#include <type_traits>

#include "attn_layout.h"
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

template <int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW)
void sparse_attn_mla_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                            const int32_t* __restrict__ idx, uint16_t* __restrict__ out,
                            float* __restrict__ lse, int Lq, int Lk, int t_begin, int H, int k,
                            int64_t idx_bstride, float scale_log2, int cps,
                            float* __restrict__ part_o, float* __restrict__ part_lse,
                            int* __restrict__ row_ctr, int t_count, int n_seq)
{
    using S = W32Shape<576, 512, NW>;
    constexpr int NC = S::NC;
    // ring slots: three for many rows; four when each row's set is split
    // over workgroups (few rows: the gathers come from HBM, and a deeper ring
    // keeps more of them in flight; the wait counter, 6 bits, must hold two
    // chunks' copies)
    constexpr int NBUF = (SPLIT && 2 * S::SPW < 64) ? 4 : 3;
    constexpr int AHEAD = NBUF - 1;                           // chunks copied ahead
    constexpr int SPW = S::SPW;                               // copy instructions per wave per chunk
    constexpr int TPW = S::TI / NW;                           // of which tails
    __shared__ __attribute__((aligned(16))) uint8_t ring[NBUF][S::BUF_BYTES];
    __shared__ __attribute__((aligned(16))) int32_t sel[S::KMAX];   // the query's index list (-1 padded)
    __shared__ int wlast[NW];                                       // per wave: last valid list position

    // Unsplit with a row counter: each workgroup takes the next of the
    // n_seq * t_count rows from the counter (the grid has about 1/8 more
    // workgroups than rows; the late ones find none and leave), so dies that
    // run faster take more rows.  Which workgroup computes a row does not
    // change its result.  Otherwise: one workgroup per row, fixed.
    int row = blockIdx.x, b = blockIdx.y;
    if (!SPLIT && row_ctr != nullptr) {
        __shared__ int s_item;
        if (threadIdx.x == 0) s_item = atomicAdd(row_ctr, 1);
        __syncthreads();
        const int item = s_item;
        if (item >= n_seq * t_count) return;                 // uniform over the workgroup
        b = item / t_count;
        row = item - b * t_count;
        b = __builtin_amdgcn_readfirstlane(b);
        row = __builtin_amdgcn_readfirstlane(row);
    }
    const int t = t_begin + row;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int col = lane & 31, hi = lane >> 5;
    const int h = wave * 32 + col;

    // The query's loads, then every load of the index list before any of
    // them is used (one memory round trip instead of one per entry); the
    // list's staging then waits on both.  Entries past k read entry k - 1
    // (k >= 1) and are dropped.
    const uint16_t* qrow = q + (((int64_t)b * Lq + t) * H + h) * 576;
    v8bf qf[S::QC];
#pragma unroll
    for (int c = 0; c < S::QC; ++c) qf[c] = as_bf8(*(const u32x4*)(qrow + c * 16 + hi * 8));
    __builtin_amdgcn_sched_barrier(0);

    const int32_t* irow = idx + (int64_t)b * idx_bstride + (int64_t)row * k;
    constexpr int SPL = S::KMAX / (64 * NW);                 // list entries per lane
    int sv[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) sv[j] = irow[min(tid + j * 64 * NW, k - 1)];
    __builtin_amdgcn_sched_barrier(0);

    v16f o[S::DT];
#pragma unroll
    for (int i = 0; i < S::DT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] = 0.f;

    const uint16_t* kvb = kv + (int64_t)b * Lk * 576;
    // Stage the index list; entries that cannot be read become -1.  Chunks
    // past the last valid entry (a short row's -1 padding) are not visited.
    int last = -1;
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const int i = tid + j * 64 * NW;
        const int sidx = (i < k) ? sv[j] : -1;
        const bool ok = sidx >= 0 && sidx < Lk;
        sel[i] = ok ? sidx : -1;
        last = ok ? i : last;
    }
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) last = max(last, __shfl_xor(last, o2, kWave));
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

    // bit r set when entry r of (absolute) chunk c is a real row
    auto valid_mask = [&](int c) -> uint32_t {
        return (uint32_t)__ballot(lane < NC && sel[c * NC + (lane & 31)] >= 0);
    };
    // Copy sources of this wave's SPW copies of chunk c: RPW value rows (lane
    // i < RPW holds value row i; a copy takes its row with one lane read) and
    // TPW tail rows (8 rows per copy, one per group of 8 lanes).  Padding
    // entries copy row 0; they are masked.
    struct CopySrc {
        int vrl;
        int tr[TPW];
    };
    auto copy_src = [&](int c) -> CopySrc {
        CopySrc cs;
        const int32_t* rr_ = &sel[c * NC];
        cs.vrl = max(rr_[wave * S::RPW + (lane % S::RPW)], 0);
#pragma unroll
        for (int j = 0; j < TPW; ++j) cs.tr[j] = max(rr_[8 * (wave * TPW + j) + (lane >> 3)], 0);
        return cs;
    };
    // copy number j (< SPW) of chunk c into its ring slot
    auto issue_copy = [&](const CopySrc& cs, int c, int j) {
        const uint32_t base = lds_byte_address(ring[c % NBUF]);
        if (j < S::RPW) {
            const int r = wave * S::RPW + j;
            const int sr = __builtin_amdgcn_readlane(cs.vrl, j);
            // the row's address as a wave-uniform (scalar) 64-bit base
            global_to_lds16_saddr(wave_uniform_ptr(kvb + (int64_t)sr * 576), (uint32_t)lane * 16u,
                                  __builtin_amdgcn_readfirstlane(base + (uint32_t)r * S::VPITCH));
        } else {
            const int jj = j - S::RPW;
            const int ti = wave * TPW + jj;                  // tail instruction: rows 8*ti .. 8*ti+7
            const int r = 8 * ti + (lane >> 3);
            const int piece = (lane & 7) ^ (r & 7);
            global_to_lds16_async(kvb + (int64_t)cs.tr[jj] * 576 + 512 + piece * 8,
                                  __builtin_amdgcn_readfirstlane(base + (uint32_t)(S::VBYTES + ti * 1024)));
        }
    };
    auto issue_chunk = [&](int c) {
        const CopySrc cs = copy_src(c);
#pragma unroll
        for (int j = 0; j < SPW; ++j) issue_copy(cs, c, j);
    };

    const int krow_i = slot_row(col);
    const int tsw = krow_i & 7;
    const int js = (lane & 15) >> 2, qs = lane & 3, g2 = (lane >> 4) & 1;
    constexpr float kHeadroom = 64.f;                        // log2 units
    constexpr int kPre = 6;                                  // key fragments read ahead of their MFMA
    constexpr int kPvPre = 2;                                // V^T fragments read ahead of their MFMA
    float m = -INFINITY;                                     // reference maximum (log2 domain), per head
    float l = 0.f;                                           // this half-wave's sum of p
    float m_seen = -INFINITY;                                // this half-wave's largest logit (log2 domain)
    for (int pass = 0; pass < 2; ++pass) {
        bool overflow = false;
#pragma unroll
        for (int i = 0; i < AHEAD; ++i)
            if (nchunks > i) issue_chunk(c0 + i);
        for (int it = 0; it < nchunks; ++it) {
            // chunk it landed; the up to AHEAD - 1 chunks after it may be in flight
            const int later = min(AHEAD - 1, nchunks - 1 - it);
            if constexpr (AHEAD >= 3) {
                if (later >= 2) wait_vmcnt<2 * SPW>();
                else if (later == 1) wait_vmcnt<SPW>();
                else wait_vmcnt0();
            } else {
                if (later == 1) wait_vmcnt<SPW>();
                else wait_vmcnt0();
            }
            __syncthreads();                                 // ... for every wave; chunk it-1 consumed
            const int c = c0 + it;
            const uint8_t* cur = ring[c % NBUF];
            const bool copies = it + AHEAD < nchunks;        // chunk it+AHEAD goes into chunk it-1's slot
            CopySrc cs;
            uint32_t vmask;

            // S^T (32 rows x 32 heads).  Step c2 < 32 reads value-part piece
            // 2*c2 + hi of row slot_row(col); later steps read the tail.  Copy
            // j of chunk it+AHEAD is issued after MFMA min(36 j / SPW + 2, 35)
            // (two MFMAs in, so the LDS reads of its sources have landed).
            v16f sacc;
            // kMode 1: this chunk issues copies, 0: it does not, 2: as copies says
            auto qk = [&](auto mode_tag) {
                constexpr int kMode = decltype(mode_tag)::value;
                const uint8_t* vrow = cur + krow_i * S::VPITCH + hi * 16;
                const uint8_t* trw = cur + S::VBYTES + krow_i * (S::TP * 16);
                auto kfrag = [&](int c2) -> u32x4 {
                    if (c2 < 32) return *(const u32x4*)(vrow + 32 * c2);
                    return *(const u32x4*)(trw + (((2 * (c2 - 32) + hi) ^ tsw) << 4));
                };
                u32x4 kf[kPre + 1];
#pragma unroll
                for (int i = 0; i < kPre; ++i) kf[i] = kfrag(i);
                // the copy sources and the valid-row mask after the first key
                // fragments (the first MFMA waits on those), ahead of the
                // copies and of the softmax that use them
                if (copies) cs = copy_src(c + AHEAD);
                vmask = valid_mask(c);
                // fully unrolled for every wave count: with one wave (36 copies
                // per chunk) the default heuristic kept the loop, and the query
                // fragments, indexed at run time, went to scratch memory
#pragma clang loop unroll(full)
                for (int c2 = 0; c2 < S::QC; ++c2) {
                    if (c2 + kPre < S::QC) kf[(c2 + kPre) % (kPre + 1)] = kfrag(c2 + kPre);
                    // S^T accumulates in VGPRs: the 256 AGPRs hold O^T, and
                    // the compiler (one MFMA register form per function) would
                    // otherwise move an O^T tile out and back every chunk.  The
                    // chain accumulates in place (no wait states needed); its
                    // operands come from LDS and global loads only, which the
                    // compiler's waits cover; the wait states before the
                    // first VALU read of S^T follow the chain.
                    if (c2 == 0)
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                                     : "=&v"(sacc) : "v"(as_bf8(kf[0])), "v"(qf[0]));
                    else
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                                     : "+v"(sacc) : "v"(as_bf8(kf[c2 % (kPre + 1)])), "v"(qf[c2]));
#pragma unroll
                    for (int j = 0; j < SPW; ++j)
                        if ((kMode == 1 || (kMode == 2 && copies)) && c2 == min((j * S::QC) / SPW + 2, S::QC - 1))
                            issue_copy(cs, c + AHEAD, j);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            // Two copies of the loop, with and without the chunk's copies, take
            // the branch around each copy out of the MFMA sequence (2.7% at
            // 128 heads); the instances for 32 heads or split sets keep one
            // loop, which needs no scratch memory.
            if constexpr (!SPLIT && NW > 1) {
                if (copies) qk(std::integral_constant<int, 1>{});
                else qk(std::integral_constant<int, 0>{});
            } else {
                qk(std::integral_constant<int, 2>{});
            }

            // The first V^T fragments of P.V, read before the softmax so that
            // their LDS latency runs under it.  K slot (a, j) of lane group hi
            // is S^T row slot 16*tt + 8a + 4*hi + j, i.e. chunk row
            // 16*tt + 2a + hi + 4j; the lane reads dims dt*32 + 16*g2 + 4*qs ..
            // +3 of its source row.
            const uint8_t* vb = cur + 32 * g2 + 8 * qs;
            auto vfrag = [&](int s) -> u32x4 {
                const int tt = s >> 4, dt = s & 15;
                const int r0 = 16 * tt + hi + 4 * js;
                const u32x2 a = __builtin_bit_cast(u32x2, lds_read_tr16(vb + r0 * S::VPITCH + 64 * dt));
                const u32x2 bq = __builtin_bit_cast(u32x2, lds_read_tr16(vb + (r0 + 2) * S::VPITCH + 64 * dt));
                return u32x4{a[0], a[1], bq[0], bq[1]};
            };
            u32x4 vf[kPvPre + 1];
#pragma unroll
            for (int i = 0; i < kPvPre; ++i) vf[i] = vfrag(i);
            __builtin_amdgcn_sched_barrier(0);

            if (vmask == 0u) continue;                       // nothing selected here (uniform)
            // 20 wait states between the last S^T MFMA (8 passes) and any
            // VALU access to its result registers, more than the hardware's
            // required count for an 8-pass MFMA result
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(sacc));
            // S^T pinned in plain registers for the mask, the maximum and the
            // softmax (with S^T in AGPRs the compiler had read them afresh for
            // each, about 47 more moves per chunk)
            float z[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                z[v] = sacc[v];
                asm volatile("" : "+v"(z[v]));
            }
            if (vmask != 0xFFFFFFFFu) {
                // element v holds chunk row slot_row(8 (v/4) + 4 hi + v%4) = hi + rv(v)
                const uint32_t vmh = vmask >> hi;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int rv = slot_row(8 * (v >> 2) + (v & 3));
                    z[v] = ((vmh >> rv) & 1u) ? z[v] : -INFINITY;
                }
            }
            if (__any(m == -INFINITY)) {                     // first chunk holding a valid row
                float cmax0 = -INFINITY;
#pragma unroll
                for (int v = 0; v < 16; ++v) cmax0 = fmaxf(cmax0, z[v]);
                m = fmaxf(cmax0, __shfl_xor(cmax0, 32, kWave)) * scale_log2;   // both halves share m
            }
            const float negm = -m;
            // p = exp2(z - m) (masked entries are -inf: exp2 gives 0), packed
            // into bf16 pairs in place: P^T's lane layout is the B operand's
            uint32_t pw[8];
            float pz[16];
            float psum = 0.f, cmax = -INFINITY, peven = 0.f;
            auto soft = [&](int v) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(z[v], scale_log2, negm));
                if (v & 1) pw[v >> 1] = pack_bf16x2(peven, pv);
                else peven = pv;
                pz[v] = pv;
            };
#pragma unroll
            for (int v = 0; v < 8; ++v) soft(v);

            // O^T += V^T . P^T, two 16-row K steps (step s = 16 tt + dt), the
            // first V^T fragments read above.  The softmax of elements 8..15
            // runs between the first eight MFMAs.
#pragma unroll
            for (int s = 0; s < 2 * S::DT; ++s) {
                if (s + kPvPre < 2 * S::DT) vf[(s + kPvPre) % (kPvPre + 1)] = vfrag(s + kPvPre);
                const int tt = s >> 4, dt = s & 15;
                const v8bf pfrag = as_bf8(tt == 0 ? u32x4{pw[0], pw[1], pw[2], pw[3]}
                                                  : u32x4{pw[4], pw[5], pw[6], pw[7]});
                o[dt] = mfma_bf16_32x32x16(as_bf8(vf[s % (kPvPre + 1)]), pfrag, o[dt]);
                if (s < 8) soft(8 + s);
                // the sum of p, in the same order, off the path into P.V
                if (s >= 8 && s < 16) { psum += pz[2 * (s - 8)]; psum += pz[2 * (s - 8) + 1]; }
                if (s == 10) {
                    // the chunk's largest logit (overflow check, second-pass
                    // reference), taken between MFMAs, off the path into P.V
#pragma unroll
                    for (int v = 0; v < 16; ++v) cmax = fmaxf(cmax, z[v]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            l += psum;
            cmax *= scale_log2;
            m_seen = fmaxf(m_seen, cmax);
            overflow = overflow || (cmax > m + kHeadroom);
        }
        // every wave must agree before the ring is reused by a second pass
        if (!__syncthreads_or(overflow ? 1 : 0)) break;
        // recompute with the true maximum (both halves') as the reference
        m = fmaxf(m_seen, __shfl_xor(m_seen, 32, kWave));
        l = 0.f;
#pragma unroll
        for (int i = 0; i < S::DT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
    }

    l += __shfl_xor(l, 32, kWave);
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    const float lse_row = (l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
    if constexpr (SPLIT) {
        // partial (b, row, split z, head h): fp32, normalised by its own sum
        const int64_t pr = ((int64_t)b * gridDim.x + row) * gridDim.z + blockIdx.z;
        float* prow = part_o + (pr * H + h) * 512;
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
        // Element 4g + e of o[dt] is dim dt*32 + 8g + 4hi + e of head h.  One
        // swap of the half-waves gives lane hi = 0 all eight dims of group
        // 2p and lane hi = 1 those of group 2p + 1 (16 bytes each).  The
        // wave's 32 rows then go through LDS (the ring is free: every wave
        // has passed the last barrier) in two halves of the value dims, so
        // each store instruction writes two heads' 512-byte runs.  Piece j
        // of staged row r sits at slot j ^ r (conflict-free row reads).
        static_assert(NBUF * S::BUF_BYTES >= NW * 16384, "staging fits the ring");
        // the lane's position, computed afresh (kept from the start of the
        // kernel it would hold a register through the chunk loop)
        const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int col_e = lane_e & 31, hi_e = lane_e >> 5;
        uint8_t* stage = &ring[0][0] + wave * 16384;
        uint16_t* owave = (uint16_t*)wave_uniform_ptr(out + (((int64_t)b * Lq + t) * H + wave * 32) * 512);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int d8 = 0; d8 < 8; ++d8) {
                const int dt = 8 * hh + d8;
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int ga = 2 * p, gb = 2 * p + 1;
                    const uint32_t a0 = pack_bf16x2(o[dt][4 * ga] * inv, o[dt][4 * ga + 1] * inv);
                    const uint32_t a1 = pack_bf16x2(o[dt][4 * ga + 2] * inv, o[dt][4 * ga + 3] * inv);
                    const uint32_t b0 = pack_bf16x2(o[dt][4 * gb] * inv, o[dt][4 * gb + 1] * inv);
                    const uint32_t b1 = pack_bf16x2(o[dt][4 * gb + 2] * inv, o[dt][4 * gb + 3] * inv);
                    const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
                    const int piece = 4 * d8 + 2 * p + hi_e;
                    *(u32x4*)(stage + col_e * 512 + ((piece ^ col_e) << 4)) = u32x4{s0[0], s1[0], s0[1], s1[1]};
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 2 * i + hi_e;
                const u32x4 v = *(const u32x4*)(stage + r * 512 + ((col_e ^ r) << 4));
                *(u32x4*)(owave + (int64_t)r * 512 + hh * 256 + col_e * 8) = v;
            }
        }
        if (lse != nullptr && hi_e == 0)
            ((float*)wave_uniform_ptr(lse + ((int64_t)b * Lq + t) * H + wave * 32))[col_e] = lse_row;
    }
}


__global__ void zero_counter_kernel(int* __restrict__ p)
{
    if (threadIdx.x == 0) *p = 0;
}

template <int NW>
hipError_t launch_mla(const AttnLaunch& a, hipStream_t s, int ns, int cps, float* part_o, float* part_lse)
{
    const float scale_log2 = a.scale * 1.4426950408889634f;
    if (ns == 1 && a.row_ctr != nullptr) {
        // the counter is cleared by a kernel (not a memset), so the pair can
        // be captured in a graph; a one-dimensional grid takes rows (b, t)
        // numbered b * t_count + t
        hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(64), 0, s, a.row_ctr);
        const int64_t items = (int64_t)a.B * a.t_count;
        const int64_t grid = items + items / 8 + 64;
        if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL((sparse_attn_mla_kernel<NW, false>), dim3((unsigned)grid, 1, 1), dim3(64 * NW), 0, s,
                           (const uint16_t*)a.q, (const uint16_t*)a.kv, a.idx, (uint16_t*)a.out, a.lse, a.Lq,
                           a.Lk, a.t_begin, a.H, a.k, a.idx_bstride, scale_log2, cps, part_o, part_lse, a.row_ctr,
                           a.t_count, a.B);
    } else if (ns == 1) {
        hipLaunchKernelGGL((sparse_attn_mla_kernel<NW, false>), dim3(a.t_count, a.B, 1), dim3(64 * NW), 0, s,
                           (const uint16_t*)a.q, (const uint16_t*)a.kv, a.idx, (uint16_t*)a.out, a.lse, a.Lq,
                           a.Lk, a.t_begin, a.H, a.k, a.idx_bstride, scale_log2, cps, part_o, part_lse, nullptr,
                           a.t_count, a.B);
    } else {
        hipLaunchKernelGGL((sparse_attn_mla_kernel<NW, true>), dim3(a.t_count, a.B, ns), dim3(64 * NW), 0, s,
                           (const uint16_t*)a.q, (const uint16_t*)a.kv, a.idx, (uint16_t*)a.out, a.lse, a.Lq,
                           a.Lk, a.t_begin, a.H, a.k, a.idx_bstride, scale_log2, cps, part_o, part_lse, nullptr,
                           a.t_count, a.B);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn_mla(const AttnLaunch& a, hipStream_t s, int ns, int cps, float* part_o,
                                  float* part_lse)
{
    switch (a.H) {
    case 32: return launch_mla<1>(a, s, ns, cps, part_o, part_lse);
    case 64: return launch_mla<2>(a, s, ns, cps, part_o, part_lse);
    case 128: return launch_mla<4>(a, s, ns, cps, part_o, part_lse);
    }
    return hipErrorInvalidValue;
}

}  // namespace dsa
