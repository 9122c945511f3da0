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
// list, and when that list holds at least k and at most kCand keys the
// threshold is found on the list alone (the k largest keys of the row are all
// in it): one histogram over the list's range, then a brute-force rank inside
// the threshold bin; otherwise the radix select runs over the whole row.  Rows
// of up to 32768 scores are read from memory once (each thread keeps the keys
// of positions 4096 v + 4 tid + e in registers, in a kernel instance of its
// own), and so are rows of up to 65536 (twice the registers, one row per CU);
// longer rows are read again in each pass.  Selected positions are
// assembled in LDS and written out in one coalesced pass.  The histogram is
// kept in four copies (lane % 4 picks one) so that lanes hitting the same bin
// in one atomic instruction mostly hit different LDS words; its bins are
// scanned by all threads at once.  Stores that only some lanes need go to a
// per-lane trash word instead of being branched around.
#include "hw.h"
#include "launch.h"

#include <algorithm>

namespace dsa {

namespace {

constexpr int kT = 1024;           // threads per row
constexpr int kWaves = kT / kWave;
constexpr int kNV = 8;             // register-resident steps of 4 keys per thread (rows up to kRegRow)
constexpr int kNVLong = 16;        // the same for rows up to 2 kRegRow
constexpr int kTile = kT * 4;      // positions per vector step
constexpr int kRegRow = kTile * kNV;
constexpr int kCopies = 4;
constexpr int kBins = 2048;
constexpr int kCand = 6144;        // LDS list of candidate keys
constexpr int kSelCap = 2048;      // k up to this is assembled in LDS

struct TopkShared {
    uint32_t hist[kBins * kCopies];   // [bin][copy]
    uint32_t wsum[kWaves];            // per-wave totals of a scan
    uint32_t wtot[kNVLong][kWaves];
    uint32_t cand[kCand];
    int32_t sel[kSelCap];
    uint32_t trash[kWave];            // target of the stores of lanes with nothing to store
    uint32_t bin, above, bincnt, ncand;
    uint32_t cmax, nsmall, tkey, tgt, teq;
};

// Histogram over nb = 2^kWidth bins of the bins `for_each_bin` yields
// (fn(bin), bin < nb; larger bins ordered higher); leaves in sh.bin the bin
// holding the need-th largest entry, in sh.above the number of entries in
// higher bins and in sh.bincnt the entries in that bin.  Requires at least
// `need` entries and sh.hist zero on entry (zeroed once at the start of the
// kernel; the copies are cleared again as they are summed).  Every thread
// calls it; the callers' writes it depends on must be published by a barrier
// before; it ends with a barrier.
//
// The bins are scanned from the largest down by all threads at once: thread
// tid owns nb / kT consecutive bins below nb - 1 - (nb / kT) tid, a wave scan
// orders the threads of a wave, and every wave scans the kWaves wave totals.
template <int kWidth, typename ForEachBin>
__device__ __forceinline__ void bin_step(TopkShared& sh, uint32_t need, ForEachBin for_each_bin)
{
    constexpr uint32_t nb = 1u << kWidth;
    constexpr uint32_t per = nb / kT;              // bins per thread
    static_assert(per >= 1 && per * kT == nb, "whole bins per thread");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t copy = (uint32_t)lane & (kCopies - 1);
    for_each_bin([&](uint32_t bin) { atomicAdd(&sh.hist[bin * kCopies + copy], 1u); });
    __syncthreads();
    const uint32_t top = nb - 1 - per * (uint32_t)tid;
    uint32_t c[per], local = 0;
#pragma unroll
    for (uint32_t j = 0; j < per; ++j) {
        u32x4* h = (u32x4*)&sh.hist[(top - j) * kCopies];
        const u32x4 x = *h;
        c[j] = x[0] + x[1] + x[2] + x[3];
        local += c[j];
        *h = u32x4{0u, 0u, 0u, 0u};
    }
    const uint32_t incl = wave_incl_scan(local, lane);
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    const uint32_t wincl = wave_incl_scan((lane < kWaves) ? sh.wsum[lane] : 0u, lane);
    const uint32_t wbase = (wave == 0) ? 0u : (uint32_t)__shfl((int)wincl, wave - 1, kWave);
    uint32_t a = wbase + incl - local;             // entries in the bins above this thread's
    if (a < need && need <= a + local) {           // exactly one thread
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
// keys equal to the result that belong to the top set).  sh.bincnt is left
// holding the number of keys equal to the result.
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

// Two rows per CU (NV = kNV): 8 waves per SIMD (64 VGPRs) and under 80 KB of LDS each.
// IN_REGS: every row of the launch has n <= NV * kTile and either n >= 4 or
// n <= k, starts 16-byte aligned and is held in registers (a separate
// instance, so that the registers of the streaming path do not crowd the
// 4 NV register-resident keys; NV = kNVLong holds rows up to 2 kRegRow at
// one row per CU, 128 VGPRs).  Block x handles row row0 + x.
template <bool IN_REGS, int NV>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(NV > kNV ? 4 : 8)))
void topk_radix_kernel(const float* __restrict__ scores, int32_t* __restrict__ idx,
                       int q_pos0, int t_begin, int row0, int64_t sc_bstride, int64_t sc_rstride,
                       int64_t idx_bstride, int k, const int32_t* __restrict__ flag, int Lq)
{
    __shared__ TopkShared sh;

    // longest rows first: a causal launch would otherwise end on its longest rows
    const int row = row0 + (int)(gridDim.x - 1 - blockIdx.x), b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = t_begin + row;
    if (flag && flag[(int64_t)b * Lq + t] == 0)    // only the flagged rows run
        return;
    const int n = q_pos0 + t + 1;                  // candidates s = 0 .. t_pos
    int32_t* out = idx + (int64_t)b * idx_bstride + (int64_t)row * k;
    if (n <= k) {
        for (int i = tid; i < k; i += kT) out[i] = i < n ? i : -1;
        return;
    }
    const float* src = scores + (int64_t)b * sc_bstride + (int64_t)row * sc_rstride;
    constexpr bool in_regs = IN_REGS;
    static_assert(NV == kNV || (IN_REGS && NV == kNVLong), "register steps");
    // rows longer than kRegRow take a two-digit lower bound from 2048 samples
    constexpr bool two_digits = !IN_REGS || NV > kNV;
    const bool vec = IN_REGS || ((uintptr_t)src & 15u) == 0;
    if (tid == 0) {                                // published by the first barrier below
        sh.ncand = 0;
        sh.cmax = 0;
        sh.nsmall = 0;
    }
    for (int i = tid; i < kBins * kCopies / 4; i += kT) ((u32x4*)sh.hist)[i] = u32x4{0u, 0u, 0u, 0u};

    // 1. Lower bound from evenly spaced sample keys: about 2k row keys are
    //    expected at or above the sample's j-th largest key.  A row held in
    //    registers takes that key's first digit (11 bits) from 1024 samples;
    //    a longer row, where one first-digit bin holds too many keys for the
    //    list, takes its first two digits (22 bits) from 2048 samples.
    const int64_t target = 2 * (int64_t)k;
    const bool sampled = target < n;
    const int ns = two_digits ? 2 * kT : kT;
    uint32_t sraw[2] = {0u, 0u};                   // sample scores, raw bits
    if (sampled) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
            if (e == 0 || two_digits) sraw[e] = __float_as_uint(src[(int)(((int64_t)(tid + e * kT) * n) / ns)]);
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
    // 4096 v + 4 tid + e (0 past the row; steps past the row are skipped,
    // workgroup-uniform).  The row is read in aligned groups of 4 without
    // branches: a group running past the row reads the row's last whole
    // aligned group instead (its keys are set to 0 when converted), and the
    // one partial group (n % 4 != 0) is read with scalar loads and patched in.
    // All loads are issued before the first conversion, so they are in flight
    // together.
    uint32_t key[NV][4];
    if (in_regs) {
        const int last4 = (n - 4) & ~3;            // start of the last whole aligned group
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (v * kTile >= n) break;
            const u32x4 x = *(const u32x4*)(src + min(v * kTile + tid * 4, last4));
#pragma unroll
            for (int e = 0; e < 4; ++e) key[v][e] = x[e];
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (v * kTile >= n) break;
            const uint32_t keep = (v * kTile + tid * 4 <= last4) ? ~0u : 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) key[v][e] = score_key(__uint_as_float(key[v][e])) & keep;
        }
        const int sp = last4 + 4;                  // the partial group, if any (workgroup-uniform)
        if (sp < n) {
            uint32_t px[3];
#pragma unroll
            for (int e = 0; e < 3; ++e) px[e] = (sp + e < n) ? score_key(src[sp + e]) : 0u;
            const bool own = tid == (sp % kTile) / 4;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                if (v == sp / kTile)
#pragma unroll
                    for (int e = 0; e < 3; ++e) key[v][e] = own ? px[e] : key[v][e];
        }
    }
    // A row streamed from memory, in ascending steps: the whole steps of an
    // aligned row are read kPf steps ahead (the loads are always issued,
    // clamped to the last whole step, so the compiler's waits keep them in
    // flight); the partial last step, and every step of an unaligned row,
    // are read as they come.
    constexpr int kPf = 4;
    auto stream_steps = [&](auto&& fn) {
        const int nfull = vec ? n / kTile : 0;
        if (nfull > 0) {
            u32x4 raw[kPf];
#pragma unroll
            for (int j = 0; j < kPf; ++j) raw[j] = *(const u32x4*)(src + min(j, nfull - 1) * kTile + tid * 4);
            for (int st0 = 0; st0 < nfull; st0 += kPf) {
#pragma unroll
                for (int u = 0; u < kPf; ++u) {
                    const int step = st0 + u;
                    if (step >= nfull) break;                      // workgroup-uniform
                    uint32_t kk[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) kk[e] = score_key(__uint_as_float(raw[u][e]));
                    raw[u] = *(const u32x4*)(src + min(step + kPf, nfull - 1) * kTile + tid * 4);
                    fn(step * kTile + tid * 4, kk);
                }
            }
        }
        for (int t0 = nfull * kTile; t0 < n; t0 += kTile) {
            uint32_t kk[4];
            load4(t0 + tid * 4, kk);
            fn(t0 + tid * 4, kk);
        }
    };
    // fn(step start s0, keys of s0..s0+3) over the whole row, in ascending steps
    auto for_each_step = [&](auto&& fn) {
        if (in_regs) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                if (v * kTile < n) fn(v * kTile + tid * 4, key[v]);
        } else {
            stream_steps(fn);
        }
    };
    __syncthreads();                               // zero histogram and counters published

    uint32_t lbound = 0;
    if (sampled) {
        const uint32_t j = (uint32_t)((target * ns + n - 1) / n);      // 1 <= j <= ns
        uint32_t sample[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) sample[e] = score_key(__uint_as_float(sraw[e]));
        // the largest sample: the top of the candidate list's histogram range
        // (published by the barriers below)
        uint32_t smax = two_digits ? max(sample[0], sample[1]) : sample[0];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) smax = max(smax, (uint32_t)__shfl_xor((int)smax, o, kWave));
        if (lane == 0) atomicMax(&sh.cmax, smax);
        auto each_sample = [&](auto&& fn) {
            fn(sample[0]);
            if (two_digits) fn(sample[1]);
        };
        radix_step<11>(sh, 21, 0u, 0u, j, each_sample);
        const uint32_t b1 = sh.bin;
        lbound = b1 << 21;
        if (two_digits) {
            const uint32_t above = sh.above;
            __syncthreads();                       // sh.bin / sh.above are rewritten below
            radix_step<11>(sh, 10, b1 << 21, 0x7FFu << 21, j - above, each_sample);
            lbound |= sh.bin << 10;
        }
    }

    // 2. Copy the keys >= lbound to the LDS list (in any order): one wave scan
    //    of the per-thread counts and one atomic per wave reserve the wave's
    //    range (per step, for a row streamed from memory).
    uint32_t cmax = 0;                             // largest key in the list (this thread's part)
    auto append = [&](auto&& each_key, uint32_t c) {
        const uint32_t incl = wave_incl_scan(c, lane);
        uint32_t base = 0;
        if (lane == 63) base = atomicAdd(&sh.ncand, incl);
        base = __builtin_amdgcn_readlane(base, 63) + incl - c;
        each_key([&](uint32_t key) {
            if (base < (uint32_t)kCand) sh.cand[base] = key;
            ++base;
            cmax = max(cmax, key);
        });
    };
    if (in_regs) {
        // Positions past the row hold key 0, kept out by lb1 = max(lbound, 1).
        // A real key 0 (score bits 0xFFFFFFFF, the smallest key) is then left
        // out too when lbound = 0; it belongs to the top k only if fewer than
        // k keys are >= 1, i.e. the list is short, which sends the row to the
        // radix select over the whole row.  Lanes with nothing to store write
        // to their own trash word, so the stores need no branches.
        const uint32_t lb1 = max(lbound, 1u);
        uint32_t c = 0, rmax = 0;
        if (sampled) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                if (v * kTile < n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) c += key[v][e] >= lb1;
        } else {
            // no samples: the list's range ends at the row's largest key
#pragma unroll
            for (int v = 0; v < NV; ++v)
                if (v * kTile < n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        c += key[v][e] >= lb1;
                        rmax = max(rmax, key[v][e]);
                    }
        }
        const uint32_t incl = wave_incl_scan(c, lane);
        uint32_t base = 0;
        if (lane == 63) base = atomicAdd(&sh.ncand, incl);
        const uint32_t wbase = __builtin_amdgcn_readlane(base, 63);
        base = wbase + incl - c;
        uint32_t* trash = &sh.trash[lane];
        auto store = [&](bool guard) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                if (v * kTile < n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool pass = key[v][e] >= lb1 && (!guard || base < (uint32_t)kCand);
                        *(pass ? &sh.cand[base] : trash) = key[v][e];
                        base += key[v][e] >= lb1;
                    }
        };
        if (wbase + __builtin_amdgcn_readlane(incl, 63) <= (uint32_t)kCand) store(false);   // the wave's range fits
        else store(true);
        cmax = rmax;
    } else {
        for_each_step([&](int s0, const uint32_t (&kk)[4]) {
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) c += (s0 + e < n) && kk[e] >= lbound;
            append([&](auto&& put) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if ((s0 + e < n) && kk[e] >= lbound) put(kk[e]);
            }, c);
        });
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cmax = max(cmax, (uint32_t)__shfl_xor((int)cmax, o, kWave));
    if (lane == 0) atomicMax(&sh.cmax, cmax);
    __syncthreads();
    const uint32_t nc = sh.ncand;

    // 3. The k-th largest key T: from the list when it holds the top k (at least
    //    k keys >= lbound) and fits; otherwise from the whole row.  Also the
    //    number eqT of the row's keys equal to T.
    uint32_t need = (uint32_t)k;
    uint32_t T, eqT;
    bool done = false;
    if (nc >= (uint32_t)k && nc <= (uint32_t)kCand) {
        // One histogram of (key - lbound) >> sft, sft chosen so that
        // [lbound, cmax] spans at most 2048 bins (cmax: the largest sample
        // key, or the row's largest key; keys above cmax share the top bin);
        // the threshold bin then holds few keys, ranked by brute force.
        const uint32_t lb = lbound, range = sh.cmax - lb;
        const int sft = max(0, (range ? 32 - __clz(range) : 0) - 11);
        auto lbin = [&](uint32_t key) { return min((key - lb) >> sft, (uint32_t)kBins - 1u); };
        bin_step<11>(sh, need, [&](auto&& fn) {
            for (uint32_t i = tid; i < nc; i += kT) fn(lbin(sh.cand[i]));
        });
        const uint32_t bstar = sh.bin, above = sh.above;
        if (sft == 0 && bstar + 1 < (uint32_t)kBins) {
            T = lb + bstar;                        // one key value per bin (below the top bin)
            eqT = sh.bincnt;
            need -= above;
            done = true;
        } else {
            // the threshold bin's keys, in the (still unused) output storage
            static_assert(kSelCap >= kT, "room for kT keys");
            uint32_t* small = (uint32_t*)sh.sel;
            for (uint32_t i = tid; i < nc; i += kT) {
                const uint32_t key = sh.cand[i];
                if (lbin(key) == bstar) {
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
                        sh.teq = eq;
                    }
                }
                __syncthreads();
                T = sh.tkey;
                eqT = sh.teq;                      // the bin holds every key equal to T
                need = nb_ - sh.tgt;
                done = true;
            }
        }
        if (!done) {
            T = radix_select(sh, need, [&](auto&& fn) {
                for (uint32_t i = tid; i < nc; i += kT) fn(sh.cand[i]);
            });
            eqT = sh.bincnt;                       // the list's keys == T
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
        eqT = sh.bincnt;                           // the row's keys == T
    }

    // 4. Compaction in ascending s: position = (#keys > T before s) + min(#keys == T before s, need).
    //    In the general case counts of (> T, == T) are packed as
    //    (gt << 16) | eq (a step of 4096 positions holds at most 4096 of
    //    either).  Positions are assembled in LDS when k fits.
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
        // All steps at once.  Usually every key equal to T is taken (eqT ==
        // need) and T >= 1, so the selection is simply key >= T (positions
        // past the row hold key 0).  Per lane, the counts of selected keys of
        // the NV steps (at most 4 each) are packed three to a word in 10-bit
        // fields, so NW3 wave scans give every in-wave prefix (at most 256)
        // and the wave totals; the NV * kWaves (step, wave) totals in
        // ascending-s order (step-major), EPL consecutive ones per lane, get
        // one exclusive scan that every wave evaluates, and each wave reads
        // its own prefixes with uniform lane reads.  Lanes write unselected
        // positions to their own trash word.
        constexpr int NW3 = (NV + 2) / 3;
        constexpr int EPL = NV * kWaves / kWave;   // (step, wave) totals per lane
        static_assert(EPL * kWave == NV * kWaves && kWaves % EPL == 0, "whole totals per lane, a wave's own slot");
        if (eqT == need && T > 0u && to_lds) {
            uint32_t cw[NW3];
#pragma unroll
            for (int i = 0; i < NW3; ++i) cw[i] = 0u;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                uint32_t c = 0;
                if (v * kTile < n) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) c += key[v][e] >= T;
                }
                cw[v / 3] |= c << (10 * (v % 3));
            }
            uint32_t ci[NW3];
#pragma unroll
            for (int i = 0; i < NW3; ++i) ci[i] = wave_incl_scan(cw[i], lane);
            uint32_t* w3 = &sh.wtot[0][0];         // [wave][NW3] wave totals
            static_assert(kWaves * NW3 <= kNVLong * kWaves, "room for the packed wave totals");
            if (lane == 63) {
#pragma unroll
                for (int i = 0; i < NW3; ++i) w3[wave * NW3 + i] = ci[i];
            }
            __syncthreads();
            // entries EPL lane + i: step (EPL lane + i) / kWaves, wave (EPL lane + i) % kWaves
            uint32_t x[EPL], sum = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int ent = EPL * lane + i, sv = ent / kWaves, sw = ent % kWaves;
                x[i] = (w3[sw * NW3 + sv / 3] >> (10 * (sv % 3))) & 0x3FFu;
                sum += x[i];
            }
            // before entry EPL lane + (wave % EPL): this wave's slot in each lane
            uint32_t ew = wave_incl_scan(sum, lane) - sum;
#pragma unroll
            for (int i = 0; i + 1 < EPL; ++i) ew += (i < wave % EPL) ? x[i] : 0u;
            uint32_t* trash = &sh.trash[lane];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (v * kTile >= n) break;         // workgroup-uniform
                const int f = 10 * (v % 3);
                uint32_t pos = __builtin_amdgcn_readlane(ew, (v * kWaves + wave) / EPL) +
                               ((ci[v / 3] >> f) & 0x3FFu) - ((cw[v / 3] >> f) & 0x3FFu);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool pass = key[v][e] >= T;
                    *(pass ? (uint32_t*)&sh.sel[pos] : trash) = (uint32_t)(v * kTile + tid * 4 + e);
                    pos += pass;
                }
            }
        } else {
            // General case (some keys equal to T left out, or k beyond the
            // LDS assembly): the lowest-index keys equal to T are taken.  The
            // same two scans, over packed (gt << 16) | eq per step; the
            // per-step scans are recomputed after the barrier rather than
            // kept.
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const uint32_t incl = (v * kTile < n) ? wave_incl_scan(counts(v * kTile + tid * 4, key[v]), lane) : 0u;
                if (lane == 63) sh.wtot[v][wave] = incl;
            }
            __syncthreads();
            const uint32_t* flat = &sh.wtot[0][0];
            uint32_t x[EPL], sum = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                x[i] = flat[EPL * lane + i];
                sum += x[i];
            }
            uint32_t ew = wave_incl_scan(sum, lane) - sum;    // before entry EPL lane + (wave % EPL)
#pragma unroll
            for (int i = 0; i + 1 < EPL; ++i) ew += (i < wave % EPL) ? x[i] : 0u;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (v * kTile >= n) break;         // workgroup-uniform
                const uint32_t base = __builtin_amdgcn_readlane(ew, (v * kWaves + wave) / EPL);
                const uint32_t pk = counts(v * kTile + tid * 4, key[v]);
                const uint32_t pre = base + wave_incl_scan(pk, lane) - pk;
                place(v * kTile + tid * 4, key[v], pre >> 16, pre & 0xFFFFu);
            }
        }
    } else {
        uint32_t base_gt = 0, base_eq = 0;
        stream_steps([&](int s0, const uint32_t (&kk)[4]) {
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
        });
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
    // Row r (t = t_begin + r) has n = q_pos0 + t_begin + r + 1 candidates, so
    // with aligned rows the register-resident instance takes the rows with
    // n <= kRegRow and either n >= 4 or n <= k (those only write 0..n-1), a
    // contiguous range [r_lo, r_hi), and its long-row instance the rows with
    // kRegRow < n <= 2 kRegRow, [r_hi, r_2); the others stream.
    const bool aligned = ((uintptr_t)a.scores & 15u) == 0 && a.sc_bstride % 4 == 0 && a.sc_rstride % 4 == 0;
    const int64_t n0 = (int64_t)a.q_pos0 + a.t_begin + 1;                 // n of row 0
    const int64_t n_lo = a.k >= 3 ? 1 : 4;                                 // smallest n the instance takes
    const int r_lo = aligned ? (int)std::min<int64_t>(std::max<int64_t>(n_lo - n0, 0), a.t_count) : a.t_count;
    const int r_hi = aligned ? (int)std::max<int64_t>(std::min<int64_t>(kRegRow - n0 + 1, a.t_count), r_lo) : a.t_count;
    auto rows = [&](auto kernel, int r0, int r1) {
        if (r1 > r0)
            hipLaunchKernelGGL(kernel, dim3(r1 - r0, a.B), dim3(kT), 0, s, a.scores, a.idx, a.q_pos0, a.t_begin, r0,
                               a.sc_bstride, a.sc_rstride, a.idx_bstride, a.k, a.flag, a.Lq);
    };
    const int r_2 = aligned ? (int)std::max<int64_t>(std::min<int64_t>(2 * kRegRow - n0 + 1, a.t_count), r_hi) : a.t_count;
    rows(topk_radix_kernel<false, kNV>, 0, r_lo);
    rows(topk_radix_kernel<true, kNV>, r_lo, r_hi);
    rows(topk_radix_kernel<true, kNVLong>, r_hi, r_2);
    rows(topk_radix_kernel<false, kNV>, r_2, a.t_count);
    return hipGetLastError();
}

}  // namespace dsa
