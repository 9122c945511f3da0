// Sparse MQA attention over selected rows for the square shapes (d_qk = d_v =
// D in {64, 128}, 16 to 128 heads in multiples of 16, k <= 2048) on gfx950
// ("DeepseekV3.2 拆解", section 核心组件: u_t = Attn(h_t, {c_s : s in
// top-k}), every head of query t attending to the same selected rows).
//
// One workgroup per query row, one wave per 16 heads,
// v_mfma_f32_16x16x32_bf16 throughout.  Rows of D bf16 values are short, so
// a row's work per 32-row chunk is small (16 MFMAs per wave) and its chunks
// are bound by their instruction chains and by the CU's LDS traffic (the row
// copies written, the key fragments and the transpose reads of V: 3 x 32 x
// 2D bytes per chunk), not by the matrix units; the wait for a chunk's
// copies measures ~2% of a chunk.  The design keeps every per-chunk
// dependency chain short and LDS small, so that six rows share a CU:
//  - the query's index list is staged in LDS once, with all of a thread's
//    loads in flight together (one memory latency per row);
//  - the selected rows stream through two LDS chunk slots, the copies of
//    chunk i + 1 issued one per S MFMA of chunk i (global_load_lds_dwordx4,
//    1 KB per instruction, a wave-uniform base and 32-bit row offsets);
//  - ring slot s of a chunk holds list entry NI (s % RPI) + s / RPI, so the
//    entries one lane copies are consecutive in the list and come from LDS in
//    one vector read (RPI rows per copy instruction, NI instructions per
//    chunk);
//  - 16-byte piece p of slot s sits at position p ^ (s % (D / 8)), so the
//    key-fragment reads and the transpose reads of V hit distinct banks;
//  - the softmax runs against a per-head reference maximum fixed at the first
//    chunk holding a valid row, so there is no cross-lane step and no rescale
//    per chunk; each lane keeps its own partial sum, and a logit more than 64
//    (log2 units) above the reference makes the workgroup recompute the row
//    with the true maximum;
//  - S^T = K_chunk . Q^T per 16-key tile (element i of lane group g holds
//    slot 16 j + g + 4 i), P^T is the S^T tiles in bf16 in place, and
//    O^T += V^T . P^T with V^T from LDS transpose reads of the same slots.
// Measured alternatives: three or four ring slots (fewer rows per CU) were
// 22% and 45% slower; a four-slot window of list entries fetched per chunk
// instead of the staged list (9 rows per CU) was 13% slower, the CU's chunk
// throughput unchanged.
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

template <int D, int NW>
__global__ __launch_bounds__(64 * NW)
void sparse_attn_mqa_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                            const int32_t* __restrict__ idx, uint16_t* __restrict__ out,
                            float* __restrict__ lse, int Lq, int Lk, int t_begin, int H, int k,
                            int64_t idx_bstride, float scale_log2)
{
    constexpr int NC = 32;                       // rows per chunk
    constexpr int PPR = D / 8;                   // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;                // rows per copy instruction
    constexpr int NI = NC / RPI;                 // copy instructions per chunk
    constexpr int CPW = NI / NW;                 // of which each wave issues
    constexpr int SLOT = NC * D * 2;             // ring bytes per chunk
    constexpr int KMAX = 2048;
    constexpr int EPT = KMAX / (64 * NW);        // list entries staged per thread
    static_assert(D == 64 || D == 128, "64- or 128-wide rows");
    static_assert(NI % NW == 0 && CPW >= 1, "every wave issues the same number of copies");
    __shared__ __attribute__((aligned(16))) uint8_t ring[2][SLOT];
    __shared__ __attribute__((aligned(16))) int32_t sel[KMAX];
    __shared__ int wlast[NW];

    const int row = blockIdx.x, b = blockIdx.y;
    const int t = t_begin + row;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int h = wave * 16 + col;

    // Q^T operand: head h, dims 32 c + 8 g .. +8
    const uint16_t* qrow = q + (((int64_t)b * Lq + t) * H + h) * D;
    v8bf qf[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[c] = as_bf8(*(const u32x4*)(qrow + 32 * c + 8 * g));

    // Stage the index list; entries that cannot be read become -1.  Chunks
    // past the last valid entry (a short row's -1 padding) are not visited.
    const int32_t* irow = idx + (int64_t)b * idx_bstride + (int64_t)row * k;
    int last = -1;
    {
        int32_t ent[EPT];
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int i = tid + 64 * NW * m;
            ent[m] = (i < k) ? irow[i] : -1;
        }
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int i = tid + 64 * NW * m;
            const bool ok = ent[m] >= 0 && ent[m] < Lk;
            sel[i] = ok ? ent[m] : -1;
            last = ok ? i : last;
        }
    }
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) last = max(last, __shfl_xor(last, o2, kWave));
    if (lane == 0) wlast[wave] = last;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) last = max(last, wlast[w]);
    const int nch = __builtin_amdgcn_readfirstlane((last + NC) / NC);

    // the sequence's rows as a wave-uniform base; a row's byte offset fits 32 bits
    const void* kvs = wave_uniform_ptr(kv + (int64_t)b * Lk * D);
    const int cj = lane / PPR;                   // row of a copy instruction this lane fills
    // list entries (relative to the chunk) of this lane's CPW copies
    const int ebase = NI * cj + wave * CPW;
    auto copy_rows = [&](int c, int32_t (&sr)[CPW]) {
        const int32_t* src = &sel[c * NC + ebase];
        if constexpr (CPW % 4 == 0) {
#pragma unroll
            for (int x = 0; x < CPW; x += 4) {
                const u32x4 v = *(const u32x4*)(src + x);
                sr[x] = (int32_t)v[0]; sr[x + 1] = (int32_t)v[1]; sr[x + 2] = (int32_t)v[2]; sr[x + 3] = (int32_t)v[3];
            }
        } else if constexpr (CPW == 2) {
            const u32x2 v = *(const u32x2*)src;
            sr[0] = (int32_t)v[0]; sr[1] = (int32_t)v[1];
        } else {
            sr[0] = src[0];
        }
    };
    // copy x (< CPW) of chunk c: instruction i = wave * CPW + x fills slots
    // RPI i .. RPI i + RPI - 1; this lane takes slot RPI i + cj, list entry
    // NI cj + i, at position lane % PPR (global piece position ^ (slot % PPR));
    // padding entries copy row 0 (masked)
    auto issue_copy = [&](int c, const int32_t (&sr)[CPW], int x) {
        const int i = wave * CPW + x;
        const int s = RPI * i + cj;
        const uint32_t piece = (uint32_t)((lane % PPR) ^ (s % PPR));
        const uint32_t base = lds_byte_address(ring[c % 2]);
        global_to_lds16_saddr(kvs, (uint32_t)max(sr[x], 0) * (uint32_t)(D * 2) + 16u * piece,
                              __builtin_amdgcn_readfirstlane(base + (uint32_t)(i * 1024)));
    };
    // byte offset of 16-bit column d (multiple of 4) of chunk slot r
    auto off = [](int r, int d) -> uint32_t {
        return (uint32_t)(r * D * 2 + ((((d >> 3) ^ (r % PPR))) << 4) + 2 * (d & 7));
    };
    // list entry (relative to the chunk) held by slot lane % 32
    const int my_ent = NI * ((lane & 31) % RPI) + (lane & 31) / RPI;

    constexpr float kHeadroom = 64.f;            // log2 units
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    v4f o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = zero;
    float m = -INFINITY;                         // reference maximum (log2 domain), per head
    float l = 0.f;                               // this lane's sum of p
    float m_seen = -INFINITY;                    // this lane's largest logit (log2 domain)
    bool have_ref = false;                       // m is set (the same for every lane)
    for (int pass = 0; pass < 2; ++pass) {
        bool overflow = false;
        if (nch > 0) {
            int32_t sr[CPW];
            copy_rows(0, sr);
#pragma unroll
            for (int x = 0; x < CPW; ++x) issue_copy(0, sr, x);
        }
        for (int ch = 0; ch < nch; ++ch) {
            wait_vmcnt0();                       // chunk ch landed
            __syncthreads();                     // ... for every wave; chunk ch - 1 consumed
            const bool copies = ch + 1 < nch;    // into chunk ch - 1's ring slot
            int32_t sr[CPW];
            if (copies) copy_rows(ch + 1, sr);
            const int32_t vent = sel[ch * NC + my_ent];
            const uint8_t* cur = ring[ch % 2];

            // S^T tiles: every key fragment read first, then the MFMAs with the
            // copies of chunk ch + 1 between them
            u32x4 kf[D / 16];
#pragma unroll
            for (int s2 = 0; s2 < D / 16; ++s2) {
                const int j = s2 & 1, c = s2 >> 1;
                const int r = 16 * j + 4 * (col & 3) + (col >> 2);
                kf[s2] = *(const u32x4*)(cur + off(r, 32 * c + 8 * g));
            }
            v4f st[2] = {zero, zero};
#pragma unroll
            for (int s2 = 0; s2 < D / 16; ++s2) {
                st[s2 & 1] = mfma_bf16_16x16x32(as_bf8(kf[s2]), qf[s2 >> 1], st[s2 & 1]);
#pragma unroll
                for (int x = 0; x < CPW; ++x)
                    if (s2 == (x * (D / 16)) / CPW && copies) issue_copy(ch + 1, sr, x);
                __builtin_amdgcn_sched_barrier(0);
            }
            // bit s: slot s holds a real row; element i of lane group g of
            // tile j is slot 16 j + g + 4 i
            const uint32_t vmask = (uint32_t)__ballot(lane < 32 && vent >= 0);
            float z[8];
            float cmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool valid = (vmask >> (16 * j + g + 4 * i)) & 1u;
                    const float v = valid ? st[j][i] * scale_log2 : -INFINITY;
                    z[4 * j + i] = v;
                    cmax = fmaxf(cmax, v);
                }
            if (!have_ref && vmask != 0u) {      // first chunk holding a valid row: every head's reference
                const float mx = fmaxf(cmax, __shfl_xor(cmax, 16, kWave));
                m = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                have_ref = true;
            }
            // p = exp2(z - m); masked entries (-inf) give 0, also before the
            // reference is set
            const float negm = have_ref ? -m : 0.f;
            uint32_t pb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(z[2 * e] + negm);
                const float p1 = __builtin_amdgcn_exp2f(z[2 * e + 1] + negm);
                l += p0 + p1;
                pb[e] = pack_bf16x2(p0, p1);
            }
            m_seen = fmaxf(m_seen, cmax);
            overflow = overflow || (cmax > m + kHeadroom);
            const v8bf pfrag = as_bf8(u32x4{pb[0], pb[1], pb[2], pb[3]});
            // O^T tiles: A = V^T over key slots 8 g + q (slots g + 4 q) and
            // 8 g + 4 + q (slots 16 + g + 4 q), dims 16 dt + col
            const int rl = g + 4 * (col >> 2);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const int d = 16 * dt + 4 * (col & 3);
                const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(cur + off(rl, d)));
                const u32x2 hi2 = __builtin_bit_cast(u32x2, lds_read_tr16(cur + off(rl + 16, d)));
                o[dt] = mfma_bf16_16x16x32(as_bf8(u32x4{lo[0], lo[1], hi2[0], hi2[1]}), pfrag, o[dt]);
            }
        }
        // every wave must agree before the ring is reused by a second pass
        if (!__syncthreads_or(overflow ? 1 : 0)) break;
        // recompute with the true maximum (all four lane groups') as the reference
        const float mx = fmaxf(m_seen, __shfl_xor(m_seen, 16, kWave));
        m = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        l = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = zero;
    }

    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
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

template <int D, int NW>
hipError_t launch_mqa(const AttnLaunch& a, hipStream_t s)
{
    const float scale_log2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((sparse_attn_mqa_kernel<D, NW>), dim3(a.t_count, a.B), dim3(64 * NW), 0, s,
                       (const uint16_t*)a.q, (const uint16_t*)a.kv, a.idx, (uint16_t*)a.out, a.lse, a.Lq, a.Lk,
                       a.t_begin, a.H, a.k, a.idx_bstride, scale_log2);
    return hipGetLastError();
}

}  // namespace

bool sparse_attn_mqa_supported(int H, int D, int k, int Lk)
{
    // rows are addressed by 32-bit byte offsets from the sequence's first row
    if (k > 2048 || (D != 64 && D != 128) || H % 16 != 0 || (int64_t)Lk * D * 2 > (int64_t)UINT32_MAX) return false;
    const int nw = H / 16, ni = D == 128 ? 8 : 4;
    return (nw == 1 || nw == 2 || nw == 4 || nw == 8) && ni % nw == 0;
}

hipError_t launch_sparse_attn_mqa(const AttnLaunch& a, hipStream_t s)
{
    if (!sparse_attn_mqa_supported(a.H, a.Dqk, a.k, a.Lk) || a.Dv != a.Dqk || !a.bf16) return hipErrorInvalidValue;
    const int nw = a.H / 16;
    if (a.Dqk == 128) {
        switch (nw) {
        case 1: return launch_mqa<128, 1>(a, s);
        case 2: return launch_mqa<128, 2>(a, s);
        case 4: return launch_mqa<128, 4>(a, s);
        case 8: return launch_mqa<128, 8>(a, s);
        }
    } else {
        switch (nw) {
        case 1: return launch_mqa<64, 1>(a, s);
        case 2: return launch_mqa<64, 2>(a, s);
        case 4: return launch_mqa<64, 4>(a, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace dsa
