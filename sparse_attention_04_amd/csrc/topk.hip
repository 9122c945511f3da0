// Per-query top-k selection on gfx950 ("DeepseekV3.2 拆解", section 核心组件:
// keep the k largest indexer scores of each query; k = 2048 in the section
// 创新点 table).
//
// One workgroup of 1024 threads owns one query row.  The fp32 scores are
// mapped to order-preserving uint32 keys and the k-th largest key T is found
// by a most-significant-digit radix select (digits of 11, 11 and 10 bits; an
// LDS histogram per digit, restricted to the keys that share the digits chosen
// so far).  A final pass compacts, in ascending s, every key > T plus the
// first (lowest-index) keys == T until k entries are written, using a
// workgroup prefix sum per tile of 4096 scores.  The selection is integer work
// only, so it is exact and deterministic.
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kT = 1024;           // threads per row
constexpr int kWaves = kT / kWave;

__global__ __launch_bounds__(kT)
void topk_radix_kernel(const float* __restrict__ scores, int32_t* __restrict__ idx,
                       int q_pos0, int t_begin, int64_t sc_bstride, int64_t sc_rstride,
                       int64_t idx_bstride, int k)
{
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wtot[kWaves];
    __shared__ uint32_t sh_bin, sh_above;

    const int row = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = t_begin + row;
    const int n = q_pos0 + t + 1;                  // candidates s = 0 .. t_pos
    int32_t* out = idx + (int64_t)b * idx_bstride + (int64_t)row * k;
    if (n <= k) {
        for (int i = tid; i < k; i += kT) out[i] = i < n ? i : -1;
        return;
    }
    const float* src = scores + (int64_t)b * sc_bstride + (int64_t)row * sc_rstride;

    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)k;                   // keys still to take at/below the prefix
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int p = 0; p < 3; ++p) {
        const int shift = shifts[p];
        const uint32_t nb = 1u << widths[p];
        for (uint32_t i = tid; i < nb; i += kT) hist[i] = 0;
        __syncthreads();
        for (int s = tid; s < n; s += kT) {
            const uint32_t key = score_key(src[s]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane L owns bins [nb - (L+1)*per, nb - L*per): lane 0 the largest
            const uint32_t per = nb / kWave;
            const uint32_t hi = nb - (uint32_t)lane * per;
            uint32_t local = 0;
            for (uint32_t i = hi - per; i < hi; ++i) local += hist[i];
            const uint32_t incl = wave_incl_scan(local, lane);
            const uint32_t excl = incl - local;
            if (excl < need && need <= incl) {
                uint32_t c = excl;
                for (uint32_t i = hi; i-- > hi - per;) {
                    if (c + hist[i] >= need) {
                        sh_bin = i;
                        sh_above = c;
                        break;
                    }
                    c += hist[i];
                }
            }
        }
        __syncthreads();
        need -= sh_above;
        prefix |= sh_bin << shift;
        pmask |= (nb - 1) << shift;
        __syncthreads();
    }
    const uint32_t T = prefix;                     // the k-th largest key
    // Compaction in ascending s: position = (#keys > T before s) + min(#keys == T before s, need)
    uint32_t base_gt = 0, base_eq = 0;
    for (int s0 = 0; s0 < n; s0 += kT * 4) {
        uint32_t keys[4];
        uint32_t cg = 0, ce = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = s0 + tid * 4 + e;
            keys[e] = (s < n) ? score_key(src[s]) : 0u;
            const bool valid = s < n;
            cg += (valid && keys[e] > T);
            ce += (valid && keys[e] == T);
        }
        const uint32_t packed = (cg << 16) | ce;
        const uint32_t incl = wave_incl_scan(packed, lane);
        if (lane == 63) wtot[wave] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
        for (int ww = 0; ww < kWaves; ++ww) {
            const uint32_t x = wtot[ww];
            before += (ww < wave) ? x : 0u;
            total += x;
        }
        __syncthreads();                           // wtot reused next tile
        const uint32_t pre = before + incl - packed;
        uint32_t gt = base_gt + (pre >> 16);
        uint32_t eq = base_eq + (pre & 0xFFFFu);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = s0 + tid * 4 + e;
            if (s >= n) break;
            // positions stay below k by construction (#keys > T == k - need);
            // the guard only keeps a corrupted input from writing past the row
            if (keys[e] > T) {
                const uint32_t pos = gt + min(eq, need);
                if (pos < (uint32_t)k) out[pos] = s;
                ++gt;
            } else if (keys[e] == T) {
                if (eq < need && gt + eq < (uint32_t)k) out[gt + eq] = s;
                ++eq;
            }
        }
        base_gt += total >> 16;
        base_eq += total & 0xFFFFu;
    }
}

}  // namespace

hipError_t launch_topk(const TopkLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.t_count == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_radix_kernel, dim3(a.t_count, a.B), dim3(kT), 0, s,
                       a.scores, a.idx, a.q_pos0, a.t_begin, a.sc_bstride, a.sc_rstride,
                       a.idx_bstride, a.k);
    return hipGetLastError();
}

}  // namespace dsa
