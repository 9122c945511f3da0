// Backward of the sparse MQA/MLA attention on gfx950 (the sparse training
// stage of "DeepseekV3.2 拆解", section 预训练策略, trains the main model
// through the selected sets).  For row t, head h and selected entries i
// (rows s_i of the latent cache, value = first 512 of 576 columns):
//   P_i  = exp(scale q.kv_i - lse),  dP_i = dO . v_i,  D = dO . O
//   dZ_i = P_i (dP_i - D)
//   dq   = scale sum_i dZ_i kv_i;   dkv_i += scale dZ_i q  (576),  dkv_i += P_i dO  (first 512)
//
// Two kernels, both with bf16 MFMAs and fp32 accumulation:
//  1. dq: one workgroup per (row, group of up to 64 heads), one wave per 16
//     heads.  q^T and dO^T stay in registers as 16x16x32 operands.  The
//     selected rows stream through a two-slot LDS ring of 32 rows, copied
//     asynchronously one chunk ahead (first 512 columns at a 1040-byte pitch,
//     last 64 packed 8 rows per 1 KB).  Per chunk the wave forms S^T and
//     dP^T, then P and dZ, and accumulates dq^T = K^T dZ^T in 36 register
//     tiles; the K^T operand comes straight from the row-major rows through
//     LDS transpose reads.  P and dZ are also written (bf16, keys-major) for 2.
//  2. dkv: one workgroup per (row, 6 of the 18 column tiles of 32), one wave
//     per 2 tiles.  A tile of the first 512 columns takes both products,
//     scale dZ q and P dO, into one accumulator; the last 2 tiles take scale
//     dZ q only.  The B operands (q and dO, heads along K) stay in registers
//     for the whole row; per chunk the 32 x H weights (P and scale dZ) come
//     through LDS, and each entry's 576 contributions are stored (fp32) to
//     its slot of a key-major buffer: key s owns the slots [off[s], off[s] +
//     count[s]), and an entry's place among them is the rank an atomic
//     counter gave it in a pass over idx.
//  3. dkv[s] = the sum of key s's slots, in slot order, one wave per (key, 64
//     columns); keys no entry selects get 0.  Plain stores and streaming
//     reads replace one fp32 atomic per (entry, column); the slot order, and
//     so dkv's last bits, vary between runs.
#include "hw.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kBQK = 576;            // latent row width
constexpr int kBV = 512;             // value width
constexpr int kBNC = 32;             // selected rows per chunk
constexpr int kBKMax = 2048;         // largest k (the index list is staged in LDS)
constexpr int kRowPitch = 1040;      // ring bytes per row of the first 512 columns (+ one skew piece)
constexpr int kRingV = kBNC * kRowPitch;
constexpr int kRingSlot = kRingV + kBNC * 128;   // + the 64-column tails, 8 rows per 1 KB

// Chunk row held by row m (0..15) of a 16-row key tile in the S^T products:
// rows 4i + g of the accumulator (lane group g, element i) hold chunk rows
// g + 4i, so the four rows one transpose read gathers are 4 apart (distinct
// LDS banks at the 1040-byte pitch).
__device__ __forceinline__ constexpr int bwd_tile_row(int m) { return 4 * (m & 3) + (m >> 2); }

// Byte offset in a ring slot of 16-bit column d (d % 8 == 0 for 16-byte reads,
// d % 4 == 0 for 8-byte reads) of chunk row r: the first 512 columns at the
// row pitch, the tails packed 8 rows per 1 KB with piece p of row r at
// position p ^ (r % 8).
__device__ __forceinline__ uint32_t ring_off(int r, int d)
{
    if (d < kBV) return (uint32_t)(r * kRowPitch + 2 * d);
    const int p = (d - kBV) >> 3;
    return (uint32_t)(kRingV + (r >> 3) * 1024 + ((r & 7) * 8 + (p ^ (r & 7))) * 16 + 2 * (d & 7));
}

// ---------------------------------------------------------------- 1. dq, P, dZ

template <int NW>
__global__ __launch_bounds__(64 * NW)
void attn_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                        const int32_t* __restrict__ idx, const uint16_t* __restrict__ out,
                        const float* __restrict__ lse, const uint16_t* __restrict__ dout,
                        float* __restrict__ dq, uint16_t* __restrict__ wsP, uint16_t* __restrict__ wsZ,
                        int Lq, int Lk, int H, int k, float scale)
{
    __shared__ __attribute__((aligned(16))) uint8_t ring[2][kRingSlot];
    __shared__ __attribute__((aligned(16))) int32_t sel[kBKMax];          // the row's index list (-1 padded)
    __shared__ __attribute__((aligned(16))) uint16_t T[NW][2][kBNC * 16]; // P / dZ, [key][head] per wave
    __shared__ int wlast[NW];

    const int t = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int hb = blockIdx.z * 16 * NW + wave * 16;                    // this wave's first head
    const int h = hb + col;                                             // this lane's head (S^T column)
    const int64_t qrow = (int64_t)b * Lq + t;

    v8bf qT[kBQK / 32], doT[kBV / 32];
#pragma unroll
    for (int c = 0; c < kBQK / 32; ++c) qT[c] = as_bf8(*(const u32x4*)(q + (qrow * H + h) * kBQK + 32 * c + 8 * g));
#pragma unroll
    for (int c = 0; c < kBV / 32; ++c) doT[c] = as_bf8(*(const u32x4*)(dout + (qrow * H + h) * kBV + 32 * c + 8 * g));
    // D = dO . O for head h: lane group g covers dims {32 c + 8 g + e}
    float Dh = 0.f;
#pragma unroll
    for (int c = 0; c < kBV / 32; ++c) {
        const u32x4 o4 = *(const u32x4*)(out + (qrow * H + h) * kBV + 32 * c + 8 * g);
        const u32x4 d4 = __builtin_bit_cast(u32x4, doT[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Dh = fmaf(bf16_bits_to_f32(o4[e] & 0xFFFFu), bf16_bits_to_f32(d4[e] & 0xFFFFu), Dh);
            Dh = fmaf(bf16_bits_to_f32(o4[e] >> 16), bf16_bits_to_f32(d4[e] >> 16), Dh);
        }
    }
    Dh += __shfl_xor(Dh, 16, kWave);
    Dh += __shfl_xor(Dh, 32, kWave);
    const float lse2 = lse[qrow * H + h] * 1.4426950408889634f;
    const float scale_log2 = scale * 1.4426950408889634f;

    // Stage the index list; entries that cannot be read become -1.  Chunks
    // past the last valid entry are not visited.
    const int32_t* irow = idx + qrow * k;
    int last = -1;
    for (int i = tid; i < kBKMax; i += 64 * NW) {
        const int s = (i < k) ? irow[i] : -1;
        const bool ok = s >= 0 && s < Lk;
        sel[i] = ok ? s : -1;
        last = ok ? i : last;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, kWave));
    if (lane == 0) wlast[wave] = last;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) last = max(last, wlast[w]);
    const int nchunks = __builtin_amdgcn_readfirstlane((last + kBNC) / kBNC);

    v4f dqa[kBQK / 16];
#pragma unroll
    for (int m = 0; m < kBQK / 16; ++m) dqa[m] = v4f{0.f, 0.f, 0.f, 0.f};
    const uint16_t* kvb = kv + (int64_t)b * Lk * kBQK;

    // copies of chunk c into ring slot c % 2 (rows past the list copy row 0;
    // their weights are zero): row e on wave e % NW, tail group ti (rows
    // 8 ti .. 8 ti + 7) on wave ti % NW
    auto issue = [&](int c) {
        const uint32_t base = lds_byte_address(ring[c & 1]);
        for (int e = wave; e < kBNC; e += NW) {
            const int sr = max(sel[c * kBNC + e], 0);
            global_to_lds16_async(kvb + (int64_t)__builtin_amdgcn_readfirstlane(sr) * kBQK + lane * 8,
                                  __builtin_amdgcn_readfirstlane(base + (uint32_t)(e * kRowPitch)));
        }
        for (int ti = wave; ti < kBNC / 8; ti += NW) {
            const int r = 8 * ti + (lane >> 3);
            const int sr = max(sel[c * kBNC + r], 0);
            const int piece = (lane & 7) ^ (r & 7);
            global_to_lds16_async(kvb + (int64_t)sr * kBQK + kBV + piece * 8,
                                  __builtin_amdgcn_readfirstlane(base + (uint32_t)(kRingV + ti * 1024)));
        }
    };

    const int i16 = lane & 15;
    if (nchunks > 0) issue(0);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int c0 = ch * kBNC;
        // this wave's copies of chunk ch: after them it issued only the two
        // stores of chunk ch - 1's P and dZ (lane 0 always stores), which
        // may stay in flight
        if (ch == 0) wait_vmcnt0();
        else wait_vmcnt<2>();
        __syncthreads();                                                // everyone's; chunk ch - 1 consumed
        if (ch + 1 < nchunks) issue(ch + 1);
        const uint8_t* cur = ring[ch & 1];

        // S^T and dP^T: accumulator element i of tile j (lane group g, head
        // col) is chunk row 16 j + g + 4 i
        // Key fragments are read kPre steps ahead of their MFMAs over both
        // tiles (step u = 18 j + c); the order is pinned, as the compiler
        // would otherwise wait on each read right before its use.
        v4f st[2], dpt[2];
        {
            constexpr int kSt = kBQK / 32, kPre = 4;
            auto kfrag = [&](int u) -> u32x4 {
                const int j = u / kSt, c = u % kSt;
                return *(const u32x4*)(cur + ring_off(16 * j + bwd_tile_row(col), 32 * c + 8 * g));
            };
            u32x4 kf[kPre + 1];
#pragma unroll
            for (int u = 0; u < kPre; ++u) kf[u] = kfrag(u);
            v4f a = {0.f, 0.f, 0.f, 0.f}, bq = a;
#pragma unroll
            for (int u = 0; u < 2 * kSt; ++u) {
                const int c = u % kSt;
                if (u + kPre < 2 * kSt) kf[(u + kPre) % (kPre + 1)] = kfrag(u + kPre);
                const v8bf f = as_bf8(kf[u % (kPre + 1)]);
                a = mfma_bf16_16x16x32(f, qT[c], a);
                if (c < kBV / 32) bq = mfma_bf16_16x16x32(f, doT[c], bq);
                if (c == kSt - 1) {
                    st[u / kSt] = a;
                    dpt[u / kSt] = bq;
                    a = v4f{0.f, 0.f, 0.f, 0.f};
                    bq = a;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        float pv[8], zv[8];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = sel[c0 + 16 * j + g + 4 * i] >= 0;
                const float p = ok ? exp2f(fmaf(st[j][i], scale_log2, -lse2)) : 0.f;
                pv[4 * j + i] = p;
                zv[4 * j + i] = p * (dpt[j][i] - Dh) * scale;          // scale dZ, used by dq and dkv
            }
        // dq^T tiles: A = dZ (head col; K slots 8 g + 4 j + i = chunk rows
        // 16 j + g + 4 i), B = K^T over the same slots, dims 16 m + col: the
        // transpose read of lane group g gathers rows g + 4 (i16 / 4) (+16),
        // 4 dims 16 m + 4 (i16 % 4) each, and hands lane col dim 16 m + col
        const v8bf az = as_bf8(u32x4{pack_bf16x2(zv[0], zv[1]), pack_bf16x2(zv[2], zv[3]),
                                     pack_bf16x2(zv[4], zv[5]), pack_bf16x2(zv[6], zv[7])});
        const int rl = g + 4 * (i16 >> 2);
        {
            constexpr int kPre = 3;                                     // tiles read ahead (2 reads each)
            auto ktfrag = [&](int m) -> u32x4 {
                const int d = 16 * m + 4 * (i16 & 3);
                const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(cur + ring_off(rl, d)));
                const u32x2 hi2 = __builtin_bit_cast(u32x2, lds_read_tr16(cur + ring_off(rl + 16, d)));
                return u32x4{lo[0], lo[1], hi2[0], hi2[1]};
            };
            u32x4 kt[kPre + 1];
#pragma unroll
            for (int m = 0; m < kPre; ++m) kt[m] = ktfrag(m);
#pragma unroll
            for (int m = 0; m < kBQK / 16; ++m) {
                if (m + kPre < kBQK / 16) kt[(m + kPre) % (kPre + 1)] = ktfrag(m + kPre);
                dqa[m] = mfma_bf16_16x16x32(az, as_bf8(kt[m % (kPre + 1)]), dqa[m]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // P and dZ (bf16) to the workspace, keys-major: through this wave's
        // part of LDS so that a lane stores 8 heads of one key
        uint16_t* tp = T[wave][0];
        uint16_t* tz = T[wave][1];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 16 * j + g + 4 * i;
                const uint32_t pz = pack_bf16x2(pv[4 * j + i], zv[4 * j + i]);
                tp[kk * 16 + col] = (uint16_t)(pz & 0xFFFFu);
                tz[kk * 16 + col] = (uint16_t)(pz >> 16);
            }
        __builtin_amdgcn_wave_barrier();
        {
            const int kk = lane & 31, half = lane >> 5;
            if (c0 + kk < k) {
                const int64_t wo = (qrow * k + c0 + kk) * H + hb + 8 * half;
                *(u32x4*)(wsP + wo) = *(const u32x4*)(tp + kk * 16 + 8 * half);
                *(u32x4*)(wsZ + wo) = *(const u32x4*)(tz + kk * 16 + 8 * half);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    // keys never visited (past the last valid entry) get zero weights
    for (int i = nchunks * kBNC + (tid >> 1); i < k; i += 32 * NW) {
        const int64_t wo = (qrow * k + i) * H + blockIdx.z * 16 * NW + 8 * (tid & 1);
        for (int w = 0; w < 2 * NW; w += 2) {
            *(u32x4*)(wsP + wo + 8 * w) = u32x4{0u, 0u, 0u, 0u};
            *(u32x4*)(wsZ + wo + 8 * w) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // dq[h = hb + 4 g + i][16 m + col]
#pragma unroll
    for (int m = 0; m < kBQK / 16; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dq[(qrow * H + hb + 4 * g + i) * kBQK + 16 * m + col] = dqa[m][i];
}

// ---------------------------------------------------------------- 2. dkv

constexpr int kTilesPerWave = 2;
constexpr int kDkvTiles = kBQK / 32;                                    // 18 (16 with a value part)
constexpr int kDkvWaves = 3;                                            // 3 waves x 2 tiles: 18 = 3 x 6
constexpr int kDkvThreads = 64 * kDkvWaves;
constexpr int kTilesPerGroup = kDkvWaves * kTilesPerWave;               // 6 per workgroup

template <int KS>                                                       // K steps of 16 heads (H = 16 KS)
__global__ __launch_bounds__(kDkvThreads, 2)                            // two workgroups per CU
void attn_bwd_dkv_kernel(const uint16_t* __restrict__ q, const int32_t* __restrict__ idx,
                         const uint16_t* __restrict__ dout, const uint16_t* __restrict__ wsP,
                         const uint16_t* __restrict__ wsZ, const int32_t* __restrict__ rank,
                         const int32_t* __restrict__ off, float* __restrict__ contrib, int Lq, int Lk, int k,
                         float scale)
{
    constexpr int H = 16 * KS;
    constexpr int WP = H + 8;                                           // W row pitch (bf16): conflict-free reads
    constexpr int WTOT = 2 * kBNC * (H / 8);                            // 16-byte pieces of W per chunk
    constexpr int WPER = (WTOT + kDkvThreads - 1) / kDkvThreads;        // per thread (the last round partial)
    __shared__ __attribute__((aligned(16))) uint16_t W[2][2][kBNC * WP];  // [buffer][P | dZ][key][head]
    __shared__ __attribute__((aligned(16))) int32_t sel[kBKMax];           // the row's index list (-1 padded)
    __shared__ __attribute__((aligned(16))) int32_t slot[kBKMax];          // each entry's slot (-1: none)
    __shared__ int wlast[kDkvWaves];
    const int t = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hs = lane >> 5;
    const int64_t qrow = (int64_t)b * Lq + t;
    static_assert(kDkvTiles % kTilesPerGroup == 0, "every wave has whole tiles");
    const int tile0 = blockIdx.z * kTilesPerGroup + wave * kTilesPerWave;

    // B operands of tile T (dims 32 T + n): q, and for T < 16 also dO; heads
    // 16 st + 8 hs + e along K
    v8bf bq[kTilesPerWave][KS], bo[kTilesPerWave][KS];
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
        const int T = tile0 + j;
        const bool hasv = T < kBV / 32;
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            uint32_t uq[4] = {0u, 0u, 0u, 0u}, uo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const int64_t h0 = qrow * H + 16 * st + 8 * hs + e;
                uq[e / 2] = (uint32_t)q[h0 * kBQK + 32 * T + n] | ((uint32_t)q[(h0 + 1) * kBQK + 32 * T + n] << 16);
                if (hasv)
                    uo[e / 2] = (uint32_t)dout[h0 * kBV + 32 * T + n] |
                                ((uint32_t)dout[(h0 + 1) * kBV + 32 * T + n] << 16);
            }
            bq[j][st] = as_bf8(u32x4{uq[0], uq[1], uq[2], uq[3]});
            bo[j][st] = as_bf8(u32x4{uo[0], uo[1], uo[2], uo[3]});
        }
    }

    // Stage the index list; entries that cannot be read become -1.  Chunks
    // past the last valid entry are not visited.
    const int32_t* irow = idx + qrow * k;
    int last = -1;
    for (int i = tid; i < kBKMax; i += kDkvThreads) {
        const int s = (i < k) ? irow[i] : -1;
        const bool ok = s >= 0 && s < Lk;
        sel[i] = ok ? s : -1;
        slot[i] = ok ? off[(int64_t)b * Lk + s] + rank[qrow * k + i] : -1;
        last = ok ? i : last;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, kWave));
    if (lane == 0) wlast[wave] = last;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kDkvWaves; ++w) last = max(last, wlast[w]);
    const int nch = __builtin_amdgcn_readfirstlane((last + kBNC) / kBNC);

    // The weights of chunk c + 1 (piece p = tid + 192 e: matrix p / (32 H / 8),
    // key, 8 heads) are loaded into registers while chunk c computes, before
    // its atomics, and stored to the other LDS buffer after them.  Nothing
    // between the loads and the stores branches on memory work, so the
    // compiler's wait for the loads leaves this chunk's atomics in flight.
    auto load_w = [&](int c, u32x4 (&wr)[WPER]) {
#pragma unroll
        for (int e = 0; e < WPER; ++e) {
            const int p = (tid + kDkvThreads * e) % WTOT;               // past WTOT: a copy, not stored
            const int which = p / (kBNC * (H / 8)), rem = p % (kBNC * (H / 8));
            const int kk = rem / (H / 8), cc = rem % (H / 8);
            const int key = min(c * kBNC + kk, k - 1);                  // past k: zeroed when stored
            wr[e] = *(const u32x4*)((which ? wsZ : wsP) + (qrow * k + key) * H + 8 * cc);
        }
    };
    auto store_w = [&](int c, const u32x4 (&wr)[WPER]) {
#pragma unroll
        for (int e = 0; e < WPER; ++e) {
            const int p = tid + kDkvThreads * e;
            if (p >= WTOT) break;
            const int which = p / (kBNC * (H / 8)), rem = p % (kBNC * (H / 8));
            const int kk = rem / (H / 8), cc = rem % (H / 8);
            const bool in = c * kBNC + kk < k;
            *(u32x4*)(&W[c & 1][which][kk * WP + 8 * cc]) = in ? wr[e] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    u32x4 wr[WPER];
    if (nch > 0) {
        load_w(0, wr);
        store_w(0, wr);
    }
    for (int ch = 0; ch < nch; ++ch) {
        const int c0 = ch * kBNC;
        const int cn = min(ch + 1, nch - 1);                            // the last chunk reloads itself
        __syncthreads();                                                // W of ch complete; the other buffer free
        load_w(cn, wr);
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j) {
            const int T = tile0 + j;
            const uint16_t* wz = W[ch & 1][1] + n * WP + 8 * hs;        // scale dZ
            const uint16_t* wp = W[ch & 1][0] + n * WP + 8 * hs;        // P
            v16f acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
            for (int st = 0; st < KS; ++st)
                acc = mfma_bf16_32x32x16(as_bf8(*(const u32x4*)(wz + 16 * st)), bq[j][st], acc);
            if (T < kBV / 32) {
#pragma unroll
                for (int st = 0; st < KS; ++st)
                    acc = mfma_bf16_32x32x16(as_bf8(*(const u32x4*)(wp + 16 * st)), bo[j][st], acc);
            }
            const int d = 32 * T + n;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int sl = slot[c0 + 8 * (v >> 2) + 4 * hs + (v & 3)];
                if (sl >= 0) contrib[(int64_t)sl * kBQK + d] = acc[v];
            }
        }
        store_w(cn, wr);
    }
}

// ---------------------------------------------------------------- slots and the per-key sums

// rank[b, t, i] = this entry's place among the entries of its key (from an
// atomic counter, so the order among one key's entries varies between runs);
// count[b, s] ends as the number of entries of key s.  Entries that are not a
// row get -1.
__global__ __launch_bounds__(256)
void bwd_rank_kernel(const int32_t* __restrict__ idx, int32_t* __restrict__ rank, int32_t* __restrict__ count,
                     int64_t n_entries, int per_b, int Lk)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n_entries) return;
    const int s = idx[e];
    const int b = (int)(e / per_b);
    rank[e] = (s >= 0 && s < Lk) ? atomicAdd(&count[(int64_t)b * Lk + s], 1) : -1;
}

// off[j] = count[0] + ... + count[j - 1] over j < n (one workgroup of 1024
// threads: each scans a contiguous run, a block scan orders the runs).
__global__ __launch_bounds__(1024)
void bwd_offsets_kernel(const int32_t* __restrict__ count, int32_t* __restrict__ off, int64_t n)
{
    __shared__ uint32_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t per = (n + 1023) / 1024;
    const int64_t j0 = min((int64_t)tid * per, n), j1 = min(j0 + per, n);
    uint32_t local = 0;
    for (int64_t j = j0; j < j1; ++j) local += (uint32_t)count[j];
    const uint32_t incl = wave_incl_scan(local, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t base = incl - local;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    for (int64_t j = j0; j < j1; ++j) {
        off[j] = (int32_t)base;
        base += (uint32_t)count[j];
    }
}

// dkv[b, s, 64 c + lane] = the sum of column 64 c + lane over key s's slots,
// in slot order; one wave per (key, 64 columns), eight slots in flight.  Keys
// are visited in ascending s, the longest segments of a causal problem first.
constexpr int kRedCols = kBQK / 64;                                     // 9 column blocks
__global__ __launch_bounds__(256)
void bwd_key_sum_kernel(const float* __restrict__ contrib, const int32_t* __restrict__ off,
                        const int32_t* __restrict__ count, float* __restrict__ dkv, int64_t n_keys)
{
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= n_keys * kRedCols) return;                                 // whole waves leave
    const int lane = threadIdx.x & 63;
    const int64_t j = w / kRedCols;                                     // key (b * Lk + s)
    const int c = (int)(w % kRedCols);
    const int64_t r0 = off[j];
    const int cnt = count[j];
    const float* src = contrib + r0 * kBQK + 64 * c + lane;
    float acc = 0.f;
    int r = 0;
    for (; r + 8 <= cnt; r += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = src[(int64_t)(r + u) * kBQK];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += x[u];
    }
    for (; r < cnt; ++r) acc += src[(int64_t)r * kBQK];
    dkv[j * kBQK + 64 * c + lane] = acc;
}

__global__ __launch_bounds__(256)
void fill_zero_kernel(float* __restrict__ p, int64_t n4)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
        *(v4f*)(p + 4 * i) = v4f{0.f, 0.f, 0.f, 0.f};
}

}  // namespace

// Workspace: P and dZ (bf16, [B, Lq, k, H] each), the entries' ranks
// ([B, Lq, k] int32), the per-key counts and offsets ([B, Lk] int32 each) and
// the key-major contributions (one 576-float slot per entry of idx), each part
// 256-byte aligned.
struct BwdLayout {
    size_t p, rank, count, off, contrib, total;
};

BwdLayout bwd_layout(int B, int Lq, int Lk, int H, int k)
{
    auto r256 = [](size_t x) { return (x + 255u) & ~(size_t)255u; };
    const size_t entries = (size_t)B * Lq * k;
    BwdLayout L{};
    L.p = r256(2 * entries * H * sizeof(uint16_t));
    L.rank = r256(entries * sizeof(int32_t));
    L.count = r256((size_t)B * Lk * sizeof(int32_t));
    L.off = r256((size_t)B * Lk * sizeof(int32_t));
    L.contrib = r256(entries * kBQK * sizeof(float));
    L.total = L.p + L.rank + L.count + L.off + L.contrib;
    return L;
}

size_t attn_bwd_workspace_bytes(int B, int Lq, int Lk, int H, int k)
{
    return bwd_layout(B, Lq, Lk, H, k).total;
}

hipError_t launch_attn_bwd(const AttnBwdLaunch& a, hipStream_t s)
{
    if (a.B == 0 || a.Lq == 0) return hipSuccess;
    const BwdLayout Lw = bwd_layout(a.B, a.Lq, a.Lk, a.H, a.k);
    char* wp = (char*)a.workspace;
    uint16_t* wsP = (uint16_t*)wp;
    uint16_t* wsZ = wsP + (size_t)a.B * a.Lq * a.k * a.H;
    int32_t* rank = (int32_t*)(wp + Lw.p);
    int32_t* count = (int32_t*)(wp + Lw.p + Lw.rank);
    int32_t* off = (int32_t*)(wp + Lw.p + Lw.rank + Lw.count);
    float* contrib = (float*)(wp + Lw.p + Lw.rank + Lw.count + Lw.off);
    // counts = 0 (a kernel, not a memset, so the sequence can be captured in a graph)
    const int64_t n_keys = (int64_t)a.B * a.Lk;
    const int64_t c4 = (n_keys + 3) / 4;                                // the count region is 256-byte padded
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<int64_t>((c4 + 255) / 256, 65536)), dim3(256), 0, s,
                       (float*)count, c4);
    const int64_t n_entries = (int64_t)a.B * a.Lq * a.k;
    hipLaunchKernelGGL(bwd_rank_kernel, dim3((unsigned)((n_entries + 255) / 256)), dim3(256), 0, s, a.idx, rank, count,
                       n_entries, a.Lq * a.k, a.Lk);
    hipLaunchKernelGGL(bwd_offsets_kernel, dim3(1), dim3(1024), 0, s, (const int32_t*)count, off, n_keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nw = a.H >= 64 ? 4 : a.H / 16;
    const dim3 g1(a.Lq, a.B, a.H / (16 * nw));
#define DSA_DQ(NW)                                                                                            \
    hipLaunchKernelGGL(attn_bwd_dq_kernel<NW>, g1, dim3(64 * NW), 0, s, (const uint16_t*)a.q, (const uint16_t*)a.kv, \
                       a.idx, (const uint16_t*)a.out, a.lse, (const uint16_t*)a.dout, a.dq, wsP, wsZ, a.Lq, a.Lk, a.H, \
                       a.k, a.scale)
    switch (nw) {
    case 1: DSA_DQ(1); break;
    case 2: DSA_DQ(2); break;
    case 4: DSA_DQ(4); break;
    default: return hipErrorInvalidValue;
    }
#undef DSA_DQ
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2(a.Lq, a.B, (kDkvTiles + kTilesPerGroup - 1) / kTilesPerGroup);
#define DSA_DKV(KS)                                                                                           \
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<KS>, g2, dim3(kDkvThreads), 0, s, (const uint16_t*)a.q, a.idx,     \
                       (const uint16_t*)a.dout, wsP, wsZ, (const int32_t*)rank, (const int32_t*)off, contrib,   \
                       a.Lq, a.Lk, a.k, a.scale)
    switch (a.H / 16) {
    case 1: DSA_DKV(1); break;
    case 2: DSA_DKV(2); break;
    case 4: DSA_DKV(4); break;
    case 8: DSA_DKV(8); break;
    default: return hipErrorInvalidValue;
    }
#undef DSA_DKV
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t waves = n_keys * kRedCols;
    hipLaunchKernelGGL(bwd_key_sum_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, (const float*)contrib,
                       (const int32_t*)off, (const int32_t*)count, a.dkv, n_keys);
    return hipGetLastError();
}

}  // namespace dsa
