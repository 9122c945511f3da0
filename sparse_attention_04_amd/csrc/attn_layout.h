// Chunk layout in LDS shared by the 576/512 sparse-attention kernels
// (sparse_attn.hip, attn_mla.hip): 32 selected latent rows per chunk, each
// stored as its value part (the first d_v columns) and its tail (the
// remaining d_qk - d_v columns).  Device-side only.
#pragma once
#include <hip/hip_runtime.h>

namespace dsa {

template <int DQK, int DV, int NW>
struct W32Shape {
    static constexpr int NC = 32;                         // rows per chunk
    static constexpr int NBUF = 2;                        // ring slots
    static constexpr int VP = DV / 8;                     // 16-byte pieces of the value part
    static constexpr int TP = (DQK - DV) / 8;             // pieces of the tail
    static constexpr int VPITCH = VP * 16 + 16;           // bytes per value part in LDS (+1 skew piece)
    static constexpr int VBYTES = NC * VPITCH;            // value parts of one chunk
    static constexpr int TBYTES = NC * TP * 16;           // tails of one chunk
    static constexpr int BUF_BYTES = VBYTES + TBYTES;
    static constexpr int RPW = NC / NW;                   // value rows copied per wave
    static constexpr int TI = TBYTES / 1024;              // tail copy instructions per chunk
    static constexpr int SPW = RPW + TI / NW;             // copy instructions per wave per chunk
    static constexpr int QC = DQK / 16;                   // MFMA K steps for Q.K (all held in registers)
    static constexpr int DT = DV / 32;                    // 32-wide value tiles
    static constexpr int KMAX = 2048;                     // largest k whose index list is staged in LDS
    static_assert(VP == 64, "one copy instruction per value part");
    static_assert(TP == 8 && TI == 4 && TI % NW == 0, "8-piece tails, 8 rows per copy");
};

// chunk row held by S^T row slot m (a permutation of 0..31, see above)
__device__ __forceinline__ constexpr int slot_row(int m)
{
    return (m & 16) | (((m >> 3) & 1) << 1) | ((m >> 2) & 1) | ((m & 3) << 2);
}

}  // namespace dsa
