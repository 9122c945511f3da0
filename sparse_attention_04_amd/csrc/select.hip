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
// Both kernels run one workgroup of 256 threads per row, with the row's values
// in registers (VPT consecutive entries per thread, in list order), mapped to
// order-preserving uint32 keys, and find the k-th largest key by histogram
// steps over a shrinking key range (select_kth).  The selection is integer
// work only, so it is exact and deterministic.
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kST = 256;               // threads per row
constexpr int kSWaves = kST / kWave;
constexpr int kSBins = 2048;
constexpr int kSOut = kSelectMaxCap / 2;   // largest k (cap = 2k)

struct SelHist {
    uint32_t hist[kSBins];
    uint32_t wsum[kSWaves];
    uint32_t wmin[kSWaves], wmax[kSWaves];
    uint32_t bin, above, bincnt;
};

struct SelShared : SelHist {
    int32_t out[kSOut];
};

// Float of an order-preserving key (the inverse of score_key, +0 for the key of
// zero).
__device__ __forceinline__ float key_float(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Exclusive prefix of v over the workgroup's threads, and the total.  The
// callers' LDS writes it depends on need no barrier before, and it may be
// called again right after.
__device__ __forceinline__ uint32_t block_excl_scan(SelHist& sh, uint32_t v, uint32_t& total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t incl = wave_incl_scan(v, lane);
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int ww = 0; ww < kSWaves; ++ww) {
        const uint32_t x = sh.wsum[ww];
        base += (ww < wave) ? x : 0u;
        tot += x;
    }
    __syncthreads();                               // wsum is rewritten by the next scan
    total = tot;
    return base + incl - v;
}

// The need-th largest of the first nv keys of every thread (need <= their
// number).  The search keeps a key range [lo, hi] that holds it, starting at
// the smallest and largest key, and splits the range into at most kSBins bins
// of 2^sft keys per step: one LDS histogram of (key - lo) >> sft over the keys
// in range, scanned from the top, gives the bin holding the need-th largest
// and the count above it.  It stops when that bin holds exactly the keys still
// needed (then the top set is key >= the bin's low end: `all`) or when the
// bins are single keys (then T is that key and `need` keys equal to it belong
// to the top set, the lowest positions first).  At most three steps for 32-bit
// keys; lists of candidates usually need one or two.  The histogram is zero on
// entry and left zero.
template <int VPT>
__device__ __forceinline__ uint32_t select_kth(SelHist& sh, const uint32_t (&key)[VPT], int nv, uint32_t& need,
                                               bool& all)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        if (j < nv) {
            lo = min(lo, key[j]);
            hi = max(hi, key[j]);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, kWave));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, kWave));
    }
    if (lane == 0) {
        sh.wmin[wave] = lo;
        sh.wmax[wave] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int ww = 0; ww < kSWaves; ++ww) {
        lo = min(lo, sh.wmin[ww]);
        hi = max(hi, sh.wmax[ww]);
    }
    constexpr uint32_t per = kSBins / kST;         // bins per thread, scanned from the largest down
    while (true) {
        int sft = 0;
        while (((hi - lo) >> sft) >= (uint32_t)kSBins) ++sft;
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            if (j < nv && key[j] >= lo && key[j] <= hi) atomicAdd(&sh.hist[(key[j] - lo) >> sft], 1u);
        __syncthreads();
        const uint32_t top = kSBins - 1 - per * (uint32_t)tid;
        uint32_t c[per], local = 0;
#pragma unroll
        for (uint32_t j = 0; j < per; ++j) {
            c[j] = sh.hist[top - j];
            sh.hist[top - j] = 0u;
            local += c[j];
        }
        const uint32_t incl = wave_incl_scan(local, lane);
        if (lane == 63) sh.wsum[wave] = incl;
        __syncthreads();
        uint32_t a = incl - local;
#pragma unroll
        for (int ww = 0; ww < kSWaves; ++ww) a += (ww < wave) ? sh.wsum[ww] : 0u;
        if (a < need && need <= a + local) {       // exactly one thread
#pragma unroll
            for (uint32_t j = 0; j < per; ++j) {
                if (a < need && need <= a + c[j]) {
                    sh.bin = top - j;
                    sh.above = a;
                    sh.bincnt = c[j];
                }
                a += c[j];
            }
        }
        __syncthreads();
        need -= sh.above;
        const uint32_t blo = lo + (sh.bin << sft), cnt = sh.bincnt;
        __syncthreads();                           // sh.bin / sh.above / wsum are rewritten next step
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
__global__ __launch_bounds__(kST)
void select_threshold_kernel(SelectLaunch a)
{
    __shared__ SelHist sh;
    const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int64_t row = (int64_t)b * a.Lq + t;
    const int tpos = a.q_pos0 + t;
    if (tpos + 1 <= a.cap) {                       // every key of the row is a candidate
        if (tid == 0) a.tau[row] = -INFINITY;
        return;
    }
    const int ns = (tpos >> a.kshift) + 1;         // sample keys j << kshift <= t_pos
    for (int i = tid; i < kSBins; i += kST) sh.hist[i] = 0u;
    const float* src = a.sample + row * a.s_rstride;
    const int base = tid * VPT;
    const int nv = max(0, min(VPT, ns - base));
    uint32_t key[VPT];
#pragma unroll
    for (int j = 0; j < VPT; j += 4) {
        if (j + 3 < nv) {
            const v4f f = *(const v4f*)(src + base + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) key[j + e] = score_key(f[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) key[j + e] = (j + e < nv) ? score_key(src[base + j + e]) : 0u;
        }
    }
    __syncthreads();
    uint32_t need = (uint32_t)min(a.need, ns);
    bool all = false;
    const uint32_t T = select_kth<VPT>(sh, key, nv, need, all);
    if (tid == 0) a.tau[row] = key_float(T);
}

template <int VPT>
__global__ __launch_bounds__(kST)
void select_candidates_kernel(SelectLaunch a)
{
    static_assert(VPT <= 32, "one mask bit per entry");
    __shared__ SelShared sh;
    const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int64_t row = (int64_t)b * a.Lq + t;
    const int tpos = a.q_pos0 + t;
    const int k = a.k;
    int32_t* out = a.idx + (int64_t)b * a.idx_bstride + (int64_t)t * k;
    if (tpos + 1 <= k) {                           // every preceding token, -1 padded
        for (int i = tid; i < k; i += kST) out[i] = i <= tpos ? i : -1;
        if (tid == 0) a.flag[row] = 0;
        return;
    }
    const int n = a.cand_cnt[row];
    if (n < k || n > a.cap) {                      // the list may miss part of the top k
        if (tid == 0) a.flag[row] = 1;
        return;
    }
    if (tid == 0) a.flag[row] = 0;
    for (int i = tid; i < kSBins; i += kST) sh.hist[i] = 0u;
    const uint32_t* src = a.cand + row * (int64_t)a.cap * 2;
    const int base = tid * VPT;
    const int nv = max(0, min(VPT, n - base));
    uint32_t key[VPT];
#pragma unroll
    for (int j = 0; j < VPT; j += 2) {
        if (j + 1 < nv) {
            const u32x4 p = *(const u32x4*)(src + 2 * (base + j));
            key[j] = score_key(__uint_as_float(p[0]));
            key[j + 1] = score_key(__uint_as_float(p[2]));
        } else {
#pragma unroll
            for (int e = 0; e < 2; ++e)
                key[j + e] = (j + e < nv) ? score_key(__uint_as_float(src[2 * (base + j + e)])) : 0u;
        }
    }
    __syncthreads();
    uint32_t need = (uint32_t)k;
    bool all = false;
    const uint32_t T = select_kth<VPT>(sh, key, nv, need, all);

    // entries taken: every key > T, and keys == T while fewer than `need` of
    // them precede in list order (all of them when `all`)
    uint32_t sel = 0u, eq = 0u;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const bool ok = j < nv;
        sel |= (ok && (all ? key[j] >= T : key[j] > T)) ? (1u << j) : 0u;
        eq |= (ok && !all && key[j] == T) ? (1u << j) : 0u;
    }
    if (!all) {
        uint32_t tot;
        uint32_t r = block_excl_scan(sh, (uint32_t)__builtin_popcount(eq), tot);
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            if (eq & (1u << j)) {
                sel |= (r < need) ? (1u << j) : 0u;
                ++r;
            }
        }
    }
    uint32_t tot;
    uint32_t o = block_excl_scan(sh, (uint32_t)__builtin_popcount(sel), tot);
    // the positions s of the entries taken (read again from the list)
    while (sel) {
        const int j = __builtin_ctz(sel);
        sel &= sel - 1;
        sh.out[o] = (int32_t)src[2 * (base + j) + 1];
        ++o;
    }
    __syncthreads();
    for (int i = tid; i < k; i += kST) out[i] = sh.out[i];
}

}  // namespace

hipError_t launch_select_threshold(const SelectLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.Lq == 0) return hipSuccess;
    const int64_t smax = ((int64_t)(a.q_pos0 + a.Lq - 1) >> a.kshift) + 1;   // longest sample row
    const dim3 grid(a.Lq, a.B), block(kST);
    if (smax <= 16 * kST)
        hipLaunchKernelGGL(select_threshold_kernel<16>, grid, block, 0, s, a);
    else if (smax <= 32 * kST)
        hipLaunchKernelGGL(select_threshold_kernel<32>, grid, block, 0, s, a);
    else if (smax <= 64 * kST)
        hipLaunchKernelGGL(select_threshold_kernel<64>, grid, block, 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_select_candidates(const SelectLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.Lq == 0) return hipSuccess;
    if (a.k > kSOut) return hipErrorInvalidValue;
    const dim3 grid(a.Lq, a.B), block(kST);
    if (a.cap <= 16 * kST)
        hipLaunchKernelGGL(select_candidates_kernel<16>, grid, block, 0, s, a);
    else if (a.cap <= 32 * kST)
        hipLaunchKernelGGL(select_candidates_kernel<32>, grid, block, 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace dsa
