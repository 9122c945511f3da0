// Per-query top-k selection on gfx950 ("DeepseekV3.2 拆解", section 核心组件:
// keep the k largest indexer scores of each query; k = 2048 in the section
// 创新点 table).
//
// One workgroup of 1024 threads owns one query row.  The fp32 scores are
// mapped to order-preserving uint32 keys; the k-th largest key T is found by a
// most-significant-digit radix select (digits of 11, 11 and 10 bits, an LDS
// histogram per digit restricted to the keys that share the digits chosen so
// far), and a final pass compacts, in ascending s, every key > T plus the
// first (lowest-index) keys == T until k entries are written.  The selection
// is integer work only, so it is exact and deterministic.
//
// A first-digit histogram of 1024 evenly spaced sample keys gives a lower bound
// L that about 2k keys of the row exceed; the keys >= L are copied to an LDS
// list, and when that list holds at least k and at most kCand keys the radix
// select runs on the list alone (the k largest keys of the row are all in it);
// otherwise it runs over the whole row.  Rows of up to 32768 scores are read
// from memory once (each thread keeps the keys of positions 4096 v + 4 tid + e
// in registers); longer rows are read again in each pass.  Selected positions are assembled in LDS and
// written out in one coalesced pass.  The histogram is kept in four copies
// (lane % 4 picks one) so that lanes hitting the same bin in one atomic
// instruction mostly hit different LDS words.
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kT = 1024;           // threads per row
constexpr int kWaves = kT / kWave;
constexpr int kNV = 8;             // register-resident steps of 4 keys per thread
constexpr int kTile = kT * 4;      // positions per vector step
constexpr int kRegRow = kTile * kNV;
constexpr int kCopies = 4;
constexpr int kBins = 2048;
constexpr int kCand = 6144;        // LDS list of candidate keys
constexpr int kSelCap = 2048;      // k up to this is assembled in LDS

// Bin totals are stored with one pad word per 32 bins, so lanes reading 32
// consecutive bins each hit distinct banks.
__device__ __forceinline__ uint32_t tot_slot(uint32_t bin) { return bin + (bin >> 5); }

struct TopkShared {
    uint32_t hist[kBins * kCopies];   // [bin][copy]
    uint32_t tot[kBins + kBins / 32];
    uint32_t wtot[kNV][kWaves];
    uint32_t cand[kCand];
    int32_t sel[kSelCap];
    uint32_t bin, above, ncand;
    uint32_t cmax, nsmall, tkey, tgt;
};

// Histogram over nb = 2^kWidth bins of the bins `for_each_bin` yields
// (fn(bin), bin < nb; larger bins ordered higher); leaves in sh.bin the bin
// holding the need-th largest entry and in sh.above the number of entries in
// higher bins.  Requires at least `need` entries.  Every thread calls it; it
// ends with a barrier.
template <int kWidth, typename ForEachBin>
__device__ __forceinline__ void bin_step(TopkShared& sh, uint32_t need, ForEachBin for_each_bin)
{
    constexpr uint32_t nb = 1u << kWidth;
    constexpr uint32_t per = nb / kWave;           // bins per lane in the scan
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (uint32_t i = tid; i < nb * kCopies; i += kT) sh.hist[i] = 0;
    __syncthreads();
    const uint32_t copy = (uint32_t)lane & (kCopies - 1);
    for_each_bin([&](uint32_t bin) { atomicAdd(&sh.hist[bin * kCopies + copy], 1u); });
    __syncthreads();
    for (uint32_t i = tid; i < nb; i += kT) {
        const u32x4 c = *(const u32x4*)&sh.hist[i * kCopies];
        sh.tot[tot_slot(i)] = c[0] + c[1] + c[2] + c[3];
    }
    __syncthreads();
    if (wave == 0) {
        // lane L owns bins [nb - (L+1)*per, nb - L*per): lane 0 the largest
        const uint32_t lo = nb - (uint32_t)(lane + 1) * per;
        uint32_t local = 0;
#pragma unroll 8
        for (uint32_t i = 0; i < per; ++i) local += sh.tot[tot_slot(lo + i)];
        const uint32_t incl = wave_incl_scan(local, lane);
        const uint32_t excl = incl - local;
        // the lane whose range holds the need-th largest key
        const uint64_t hit = __ballot(excl < need && need <= incl);
        const int lt = __ffsll((unsigned long long)hit) - 1;
        const uint32_t base = __builtin_amdgcn_readlane(excl, lt);
        const uint32_t lo_t = nb - (uint32_t)(lt + 1) * per;
        // lanes 0..per-1 take that range's bins from the largest down
        const uint32_t c = (uint32_t)lane < per ? sh.tot[tot_slot(lo_t + per - 1 - lane)] : 0u;
        const uint32_t ci = wave_incl_scan(c, lane);
        const uint64_t hit2 = __ballot((uint32_t)lane < per && base + ci >= need);
        const int it = __ffsll((unsigned long long)hit2) - 1;
        if (lane == it) {
            sh.bin = lo_t + per - 1 - (uint32_t)it;
            sh.above = base + ci - c;
        }
    }
    __syncthreads();
}

// bin_step over the digit at `shift` of the keys matching (prefix, pmask).
template <int kWidth, typename ForEachKey>
__device__ __forceinline__ void radix_step(TopkShared& sh, int shift, uint32_t prefix, uint32_t pmask,
                                           uint32_t need, ForEachKey for_each_key)
{
    constexpr uint32_t mask = (1u << kWidth) - 1;
    bin_step<kWidth>(sh, need, [&](auto&& fn) {
        for_each_key([&](uint32_t key) {
            if ((key & pmask) == prefix) fn((key >> shift) & mask);
        });
    });
}

// Three radix steps (11, 11, 10 bits) over the keys `each` enumerates; returns
// the need-th largest of them (need = k on entry; on return, the number of
// keys equal to the result that belong to the top set).
template <typename ForEachKey>
__device__ __forceinline__ uint32_t radix_select(TopkShared& sh, uint32_t& need, ForEachKey each)
{
    uint32_t prefix = 0, pmask = 0;
    auto take = [&](int shift, int width) {
        need -= sh.above;
        prefix |= sh.bin << shift;
        pmask |= ((1u << width) - 1) << shift;
        __syncthreads();                           // sh.bin / sh.above are rewritten next step
    };
    radix_step<11>(sh, 21, prefix, pmask, need, each);
    take(21, 11);
    radix_step<11>(sh, 10, prefix, pmask, need, each);
    take(10, 11);
    radix_step<10>(sh, 0, prefix, pmask, need, each);
    take(0, 10);
    return prefix;
}

// two rows per CU: 8 waves per SIMD (64 VGPRs) and under 80 KB of LDS each
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(8)))
void topk_radix_kernel(const float* __restrict__ scores, int32_t* __restrict__ idx,
                       int q_pos0, int t_begin, int64_t sc_bstride, int64_t sc_rstride,
                       int64_t idx_bstride, int k)
{
    __shared__ TopkShared sh;

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
    const bool in_regs = n <= kRegRow;
    const bool vec = ((uintptr_t)src & 15u) == 0;
    if (tid == 0) {                                // published by the first barrier below
        sh.ncand = 0;
        sh.cmax = 0;
        sh.nsmall = 0;
    }

    // keys of positions s0..s0+3 (0 past the row)
    auto load4 = [&](int s0, uint32_t (&kk)[4]) {
        if (vec && s0 + 3 < n) {
            const v4f f = *(const v4f*)(src + s0);
#pragma unroll
            for (int e = 0; e < 4; ++e) kk[e] = score_key(f[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) kk[e] = (s0 + e < n) ? score_key(src[s0 + e]) : 0u;
        }
    };
    // Register copy of a row of up to kRegRow: step v holds positions
    // 4096 v + 4 tid + e.  Steps past the row are skipped (workgroup-uniform).
    uint32_t key[kNV][4];
    if (in_regs) {
#pragma unroll
        for (int v = 0; v < kNV; ++v)
            if (v * kTile < n) load4(v * kTile + tid * 4, key[v]);
    }
    // fn(step start s0, keys of s0..s0+3) over the whole row, in ascending steps
    auto for_each_step = [&](auto&& fn) {
        if (in_regs) {
#pragma unroll
            for (int v = 0; v < kNV; ++v)
                if (v * kTile < n) fn(v * kTile + tid * 4, key[v]);
        } else {
            for (int t0 = 0; t0 < n; t0 += kTile) {
                uint32_t kk[4];
                load4(t0 + tid * 4, kk);
                fn(t0 + tid * 4, kk);
            }
        }
    };

    // 1. Lower bound from evenly spaced sample keys: about 2k row keys are
    //    expected at or above the sample's j-th largest key.  A row held in
    //    registers takes that key's first digit (11 bits) from 1024 samples;
    //    a longer row, where one first-digit bin holds too many keys for the
    //    list, takes its first two digits (22 bits) from 2048 samples.
    uint32_t lbound = 0;
    const int64_t target = 2 * (int64_t)k;
    if (target < n) {
        const int ns = in_regs ? kT : 2 * kT;
        const uint32_t j = (uint32_t)((target * ns + n - 1) / n);      // 1 <= j <= ns
        uint32_t sample[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
            sample[e] = (e == 0 || !in_regs) ? score_key(src[(int)(((int64_t)(tid + e * kT) * n) / ns)]) : 0u;
        auto each_sample = [&](auto&& fn) {
            fn(sample[0]);
            if (!in_regs) fn(sample[1]);
        };
        radix_step<11>(sh, 21, 0u, 0u, j, each_sample);
        const uint32_t b1 = sh.bin;
        lbound = b1 << 21;
        if (!in_regs) {
            const uint32_t above = sh.above;
            __syncthreads();                       // sh.bin / sh.above are rewritten below
            radix_step<11>(sh, 10, b1 << 21, 0x7FFu << 21, j - above, each_sample);
            lbound |= sh.bin << 10;
        }
    } else {
        __syncthreads();                           // publishes sh.ncand = 0
    }

    // 2. Copy the keys >= lbound to the LDS list: per step one wave scan and one
    //    atomic per wave.
    uint32_t cmax = 0;                             // largest key in the list (this thread's part)
    for_each_step([&](int s0, const uint32_t (&kk)[4]) {
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) c += (s0 + e < n) && kk[e] >= lbound;
        const uint32_t incl = wave_incl_scan(c, lane);
        uint32_t base = 0;
        if (lane == 63) base = atomicAdd(&sh.ncand, incl);
        base = __builtin_amdgcn_readlane(base, 63) + incl - c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if ((s0 + e < n) && kk[e] >= lbound) {
                if (base < (uint32_t)kCand) sh.cand[base] = kk[e];
                ++base;
                cmax = max(cmax, kk[e]);
            }
        }
    });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cmax = max(cmax, (uint32_t)__shfl_xor((int)cmax, o, kWave));
    if (lane == 0) atomicMax(&sh.cmax, cmax);
    __syncthreads();
    const uint32_t nc = sh.ncand;

    // 3. The k-th largest key T: from the list when it holds the top k (at least
    //    k keys >= lbound) and fits; otherwise from the whole row.
    uint32_t need = (uint32_t)k;
    uint32_t T;
    bool done = false;
    if (nc >= (uint32_t)k && nc <= (uint32_t)kCand) {
        // One histogram of (key - lbound) >> sft, sft chosen so the list's
        // range [lbound, cmax] spans at most 2048 bins; the threshold bin then
        // holds few keys, ranked by brute force.
        const uint32_t lb = lbound, range = sh.cmax - lb;
        const int sft = max(0, (range ? 32 - __clz(range) : 0) - 11);
        bin_step<11>(sh, need, [&](auto&& fn) {
            for (uint32_t i = tid; i < nc; i += kT) fn((sh.cand[i] - lb) >> sft);
        });
        const uint32_t bstar = sh.bin, above = sh.above;
        if (sft == 0) {
            T = lb + bstar;                        // one key value per bin
            need -= above;
            done = true;
        } else {
            // the threshold bin's keys, in the (now free) histogram storage
            uint32_t* small = sh.hist;
            for (uint32_t i = tid; i < nc; i += kT) {
                const uint32_t key = sh.cand[i];
                if (((key - lb) >> sft) == bstar) {
                    const uint32_t pos = atomicAdd(&sh.nsmall, 1u);
                    if (pos < (uint32_t)kT) small[pos] = key;
                }
            }
            __syncthreads();
            const uint32_t cs = sh.nsmall;
            if (cs <= (uint32_t)kT) {
                const uint32_t nb_ = need - above;   // rank wanted inside the bin (1-based)
                if ((uint32_t)tid < cs) {
                    const uint32_t x = small[tid];
                    uint32_t gt = 0, eq = 0;
                    for (uint32_t j = 0; j < cs; ++j) {
                        const uint32_t y = small[j];
                        gt += y > x;
                        eq += y == x;
                    }
                    if (gt < nb_ && nb_ <= gt + eq) {   // every copy of the key writes the same
                        sh.tkey = x;
                        sh.tgt = gt;
                    }
                }
                __syncthreads();
                T = sh.tkey;
                need = nb_ - sh.tgt;
                done = true;
            }
        }
        if (!done) {
            T = radix_select(sh, need, [&](auto&& fn) {
                for (uint32_t i = tid; i < nc; i += kT) fn(sh.cand[i]);
            });
            done = true;
        }
    } else {
        T = radix_select(sh, need, [&](auto&& fn) {
            for (int s0 = tid * 4; s0 < n; s0 += kTile) {
                uint32_t kk[4];
                load4(s0, kk);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (s0 + e < n) fn(kk[e]);
            }
        });
    }

    // 4. Compaction in ascending s: position = (#keys > T before s) + min(#keys == T before s, need).
    //    Counts of (> T, == T) are packed as (gt << 16) | eq (a step of 4096
    //    positions holds at most 4096 of either).  Positions are assembled in
    //    LDS when k fits.
    const bool to_lds = k <= kSelCap;
    int32_t* dst = to_lds ? sh.sel : out;
    auto counts = [&](int s0, const uint32_t (&kk)[4]) {
        uint32_t cg = 0, ce = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool valid = s0 + e < n;
            cg += (valid && kk[e] > T);
            ce += (valid && kk[e] == T);
        }
        return (cg << 16) | ce;
    };
    auto place = [&](int s0, const uint32_t (&kk)[4], uint32_t gt, uint32_t eq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = s0 + e;
            if (s >= n) break;
            // positions stay below k by construction (#keys > T == k - need);
            // the guard only keeps a corrupted input from writing past the row
            if (kk[e] > T) {
                const uint32_t pos = gt + min(eq, need);
                if (pos < (uint32_t)k) dst[pos] = s;
                ++gt;
            } else if (kk[e] == T) {
                if (eq < need && gt + eq < (uint32_t)k) dst[gt + eq] = s;
                ++eq;
            }
        }
    };
    if (in_regs) {
        // All steps at once.  Per-step wave scans give positions within a wave;
        // the (step, wave) totals, in ascending-s order (step-major), get one
        // exclusive scan that every wave evaluates (two totals per lane), and
        // each wave reads its own prefixes with uniform lane reads.  The
        // per-step scans are recomputed after the barrier rather than kept.
        static_assert(kNV * kWaves == 2 * kWave, "two (step, wave) totals per lane");
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
            const uint32_t incl = (v * kTile < n) ? wave_incl_scan(counts(v * kTile + tid * 4, key[v]), lane) : 0u;
            if (lane == 63) sh.wtot[v][wave] = incl;
        }
        __syncthreads();
        const uint32_t* flat = &sh.wtot[0][0];
        const uint32_t x0 = flat[2 * lane], x1 = flat[2 * lane + 1];
        const uint32_t e0 = wave_incl_scan(x0 + x1, lane) - (x0 + x1);   // before entry 2*lane
        const uint32_t ew = (wave & 1) ? e0 + x0 : e0;                   // before entry 2*lane + (wave & 1)
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
            if (v * kTile >= n) break;             // workgroup-uniform
            const uint32_t base = __builtin_amdgcn_readlane(ew, (v * kWaves + wave) >> 1);
            const uint32_t pk = counts(v * kTile + tid * 4, key[v]);
            const uint32_t pre = base + wave_incl_scan(pk, lane) - pk;
            place(v * kTile + tid * 4, key[v], pre >> 16, pre & 0xFFFFu);
        }
    } else {
        uint32_t base_gt = 0, base_eq = 0;
        for (int t0 = 0; t0 < n; t0 += kTile) {
            const int s0 = t0 + tid * 4;
            uint32_t kk[4];
            load4(s0, kk);
            const uint32_t pk = counts(s0, kk);
            const uint32_t incl = wave_incl_scan(pk, lane);
            if (lane == 63) sh.wtot[0][wave] = incl;
            __syncthreads();
            uint32_t before = 0, total = 0;
            for (int ww = 0; ww < kWaves; ++ww) {
                const uint32_t x = sh.wtot[0][ww];
                before += (ww < wave) ? x : 0u;
                total += x;
            }
            __syncthreads();                       // wtot reused next step
            const uint32_t pre = before + incl - pk;
            place(s0, kk, base_gt + (pre >> 16), base_eq + (pre & 0xFFFFu));
            base_gt += total >> 16;
            base_eq += total & 0xFFFFu;
        }
    }
    if (to_lds) {
        __syncthreads();
        for (int i = tid; i < k; i += kT) out[i] = sh.sel[i];
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
