// Top-k selection over candidate lists on gfx950 ("DeepseekV3.2 拆解", section
// 核心组件: keep the k largest indexer scores of each query; k = 2048 in the
// section 创新点 table).
//
// The forward's candidate route keeps the full score rows out of memory:
//  1. the indexer scores every 2^kshift-th key of each row (the sample);
//  2. select_threshold_kernel: per row, tau = the need-th largest sample score,
//     chosen so that about 1.5 k of the row's keys score >= tau;
//  3. the indexer scores every key and appends those scoring >= tau to the
//     row's list, in ascending s (cand, at most cap = 2 k stored);
//  4. select_candidates_kernel: when the list holds at least k and at most cap
//     entries it holds every key scoring at least the row's k-th largest score
//     (all of them score >= tau, and at least k do), so the k largest of the
//     list, lowest s first among equal scores, are exactly the row's top k;
//     otherwise the row is flagged and the forward recomputes it from its full
//     score row.
// The sample only decides how long the lists are, never what is selected.
//
// Both kernels give each row one wave (four rows per workgroup, no barriers):
// the row's values sit in registers, entry e = 64 j + lane in element j of
// lane `lane`, mapped to order-preserving uint32 keys; the k-th largest key is
// found by 256-bin LDS histograms over a shrinking key range (wave_kth), and
// the selection is compacted in list order with ballots.  The selection is
// integer work only, so it is exact and deterministic.
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kRowsPerBlock = 4;       // one wave per row
constexpr int kBins = 256;

// Float of an order-preserving key (the inverse of score_key, +0 for the key of
// zero).
__device__ __forceinline__ float key_float(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The need-th largest of the nonzero keys key[j] of one wave (need <= their
// number; zero marks an entry past the row, below the key of every score).
// The search keeps a key range [lo, hi] holding it, starting at the smallest
// and largest key, and splits the range into at most kBins bins
// of 2^sft keys per step: an LDS histogram of (key - lo) >> sft over the keys
// in range (the wave's own 256 words, zero on entry and left zero), scanned
// from the top (lane l owns bins 4 (63 - l) .. +3), gives the bin holding the
// need-th largest and the count above it.  It stops when that bin holds exactly
// the keys still needed (then the top set is key >= the bin's low end: `all`)
// or when the bins are single keys (T is that key, and `need` of the keys
// equal to it belong to the top set, the lowest positions first).
template <int VPT>
__device__ __forceinline__ uint32_t wave_kth(uint32_t* hist, const uint32_t (&key)[VPT], uint32_t& need, bool& all)
{
    const int lane = threadIdx.x & 63;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        lo = min(lo, key[j] ? key[j] : 0xFFFFFFFFu);
        hi = max(hi, key[j]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, kWave));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, kWave));
    }
    while (true) {
        int sft = 0;
        while (((hi - lo) >> sft) >= (uint32_t)kBins) ++sft;
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            if (key[j] >= lo && key[j] <= hi) atomicAdd(&hist[(key[j] - lo) >> sft], 1u);
        // bins 4 (63 - lane) .. +3, largest first
        const int b0 = 4 * (63 - lane);
        const u32x4 c = *(const u32x4*)&hist[b0];
        *(u32x4*)&hist[b0] = u32x4{0u, 0u, 0u, 0u};
        const uint32_t local = c[0] + c[1] + c[2] + c[3];
        const uint32_t incl = wave_incl_scan(local, lane);
        uint32_t a = incl - local;                 // keys in the bins above this lane's
        const bool mine = a < need && need <= a + local;
        uint32_t bin = 0, above = 0, cnt = 0;
        if (mine) {
#pragma unroll
            for (int e = 3; e >= 0; --e) {
                if (a < need && need <= a + c[e]) {
                    bin = b0 + e;
                    above = a;
                    cnt = c[e];
                }
                a += c[e];
            }
        }
        const int src = __builtin_ctzll(__ballot(mine));
        bin = __builtin_amdgcn_readlane(bin, src);
        above = __builtin_amdgcn_readlane(above, src);
        cnt = __builtin_amdgcn_readlane(cnt, src);
        need -= above;
        const uint32_t blo = lo + (bin << sft);
        if (cnt == need) {
            all = true;
            return blo;
        }
        if (sft == 0) {
            all = false;
            return blo;
        }
        lo = blo;
        hi = (uint32_t)min((uint64_t)hi, (uint64_t)blo + ((1ull << sft) - 1u));
    }
}

template <int VPT>
__global__ __launch_bounds__(64 * kRowsPerBlock)
void select_threshold_kernel(SelectLaunch a)
{
    __shared__ __attribute__((aligned(16))) uint32_t hist[kRowsPerBlock][kBins];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRowsPerBlock + wave, b = blockIdx.y;
    uint32_t* h = hist[wave];
    *(u32x4*)&h[4 * lane] = u32x4{0u, 0u, 0u, 0u};
    if (t >= a.Lq) return;                          // whole waves leave
    const int64_t row = (int64_t)b * a.Lq + t;
    const int tpos = a.q_pos0 + t;
    if (tpos + 1 <= a.cap) {                        // every key of the row is a candidate
        if (lane == 0) a.tau[row] = -INFINITY;
        return;
    }
    const int ns = (tpos >> a.kshift) + 1;          // sample keys j << kshift <= t_pos
    const float* src = a.sample + row * a.s_rstride;
    uint32_t key[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int e = 64 * j + lane;
        key[j] = e < ns ? score_key(src[e]) : 0u;
    }
    uint32_t need = (uint32_t)min(a.need, ns);
    bool all = false;
    const uint32_t T = wave_kth<VPT>(h, key, need, all);
    if (lane == 0) a.tau[row] = key_float(T);
}

template <int VPT>
__global__ __launch_bounds__(64 * kRowsPerBlock)
void select_candidates_kernel(SelectLaunch a)
{
    __shared__ __attribute__((aligned(16))) uint32_t hist[kRowsPerBlock][kBins];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRowsPerBlock + wave, b = blockIdx.y;
    uint32_t* h = hist[wave];
    *(u32x4*)&h[4 * lane] = u32x4{0u, 0u, 0u, 0u};
    if (t >= a.Lq) return;                          // whole waves leave
    const int64_t row = (int64_t)b * a.Lq + t;
    const int tpos = a.q_pos0 + t;
    const int k = a.k;
    int32_t* out = a.idx + (int64_t)b * a.idx_bstride + (int64_t)t * k;
    if (tpos + 1 <= k) {                            // every preceding token, -1 padded
        for (int i = lane; i < k; i += 64) out[i] = i <= tpos ? i : -1;
        if (lane == 0) a.flag[row] = 0;
        return;
    }
    const int n = a.cand_cnt[row];
    if (n < k || n > a.cap) {                       // the list may miss part of the top k
        if (lane == 0) a.flag[row] = 1;
        return;
    }
    if (lane == 0) a.flag[row] = 0;
    const u32x2* src = (const u32x2*)(a.cand + row * (int64_t)a.cap * 2);
    uint32_t key[VPT], pos[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int e = 64 * j + lane;
        const u32x2 p = e < n ? src[e] : u32x2{0u, 0u};
        key[j] = e < n ? score_key(__uint_as_float(p[0])) : 0u;
        pos[j] = p[1];
    }
    uint32_t need = (uint32_t)k;
    bool all = false;
    const uint32_t T = wave_kth<VPT>(h, key, need, all);
    // in list order (= ascending s): every key > T, and the first `need` keys
    // equal to T (every key >= T when `all`)
    uint32_t base = 0, eq_seen = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const bool ok = key[j] != 0u;
        bool take;
        if (all) {
            take = ok && key[j] >= T;
        } else {
            const bool eq = ok && key[j] == T;
            const uint64_t ue = __ballot(eq);
            take = (ok && key[j] > T) || (eq && eq_seen + lanes_below(ue) < need);
            eq_seen += (uint32_t)__builtin_popcountll(ue);
        }
        const uint64_t ut = __ballot(take);
        if (take) out[base + lanes_below(ut)] = (int32_t)pos[j];
        base += (uint32_t)__builtin_popcountll(ut);
    }
}

}  // namespace

hipError_t launch_select_threshold(const SelectLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.Lq == 0) return hipSuccess;
    const int64_t smax = ((int64_t)(a.q_pos0 + a.Lq - 1) >> a.kshift) + 1;   // longest sample row
    const dim3 grid((a.Lq + kRowsPerBlock - 1) / kRowsPerBlock, a.B), block(64 * kRowsPerBlock);
    if (smax <= 32 * 64)
        hipLaunchKernelGGL(select_threshold_kernel<32>, grid, block, 0, s, a);
    else if (smax <= 64 * 64)
        hipLaunchKernelGGL(select_threshold_kernel<64>, grid, block, 0, s, a);
    else if (smax <= 128 * 64)
        hipLaunchKernelGGL(select_threshold_kernel<128>, grid, block, 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_select_candidates(const SelectLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.Lq == 0) return hipSuccess;
    const dim3 grid((a.Lq + kRowsPerBlock - 1) / kRowsPerBlock, a.B), block(64 * kRowsPerBlock);
    if (a.cap <= 16 * 64)
        hipLaunchKernelGGL(select_candidates_kernel<16>, grid, block, 0, s, a);
    else if (a.cap <= 32 * 64)
        hipLaunchKernelGGL(select_candidates_kernel<32>, grid, block, 0, s, a);
    else if (a.cap <= 64 * 64)
        hipLaunchKernelGGL(select_candidates_kernel<64>, grid, block, 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace dsa
