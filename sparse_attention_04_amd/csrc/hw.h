// Device-side helpers for gfx950 (CDNA4): vector types, MFMA wrappers,
// bf16 rounding and wave64 reductions.  Used by the kernels only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int kWave = 64;

// D(16x16 fp32) = A(16x128 e4m3) * B(128x16 e4m3) + C.  Lane l supplies row
// (l % 16) of A / column (l % 16) of B with 32 bytes of the K dimension
// chosen by (l / 16); A and B use the same K assignment, so a contiguous
// 32-byte slice per lane gives the correct dot product.  Lane l receives
// D[4*(l/16) + i][l % 16], i = 0..3.  Zero block scales select the unscaled
// v_mfma_f32_16x16x128_f8f6f4 (format 0 = e4m3 for both operands).
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, const v4f& c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D(16x16 fp32) = A(16x32 bf16) * B(32x16 bf16) + C; lane l supplies 8
// consecutive K values (slot 8*(l/16)..) of row/column l % 16.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v8bf& a, const v8bf& b, const v4f& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32 fp32) = A(32x16 bf16) * B(16x32 bf16) + C; lane l supplies 8
// consecutive K values (slot 8*(l/32)..) of row/column l % 32 and receives
// D[8*(v/4) + 4*(l/32) + (v%4)][l % 32] in element v = 0..15.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(const v8bf& a, const v8bf& b, const v16f& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read of 16-bit data (ds_read_b64_tr_b16).  Within each group
// of 16 lanes, lane i receives in element j the (i % 4)-th 16-bit value of the
// 8 bytes addressed by lane 4*j + i/4 of the same group.
__device__ __forceinline__ v4s lds_read_tr16(const void* lds_ptr)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)lds_ptr);
}

// Asynchronous 16-byte copy global -> LDS.  Lane l's 16 bytes land at
// lds_base + 16*l (lds_base must be the same for the whole wave); the global
// address is per lane.  Completion is tracked by vmcnt.
__device__ __forceinline__ void global_to_lds16(const void* gptr, void* lds_base)
{
    __builtin_amdgcn_global_load_lds(gptr, (lds_void*)lds_base, 16, 0, 0);
}

// The same copy written as a single asm block, for pipelines that fence it
// themselves (s_waitcnt vmcnt(0) + a barrier before the slot is read).  The
// compiler then does not see an LDS write here, so it adds no conservative
// vmcnt wait in front of unrelated LDS reads.  `lds_byte_addr` is the
// wave-uniform LDS byte address of lane 0's 16 bytes.  m0 is used only here.
__device__ __forceinline__ void global_to_lds16_async(const void* gptr, uint32_t lds_byte_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds_byte_addr)
                 : "memory");
}

// A pointer every lane of the wave holds, made wave-uniform (SGPRs): each
// half goes through readfirstlane, which returns a signed int, so the halves
// are taken as uint32_t before they are put together.
__device__ __forceinline__ const void* wave_uniform_ptr(const void* p)
{
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// The same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the saddr form, no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void global_to_lds16_saddr(const void* sbase, uint32_t voff, uint32_t lds_byte_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_byte_addr)
                 : "memory");
}

// 4-byte variant: lane l's 4 bytes land at lds_byte_addr + 4*l.
__device__ __forceinline__ void global_to_lds4_async(const void* gptr, uint32_t lds_byte_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(gptr), "s"(lds_byte_addr)
                 : "memory");
}

// s_waitcnt vmcnt(N) for a compile-time N (expcnt and lgkmcnt unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ uint32_t lds_byte_address(const void* p)
{
    return (uint32_t)(uintptr_t)(lds_void*)p;
}

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left unconstrained).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left unconstrained).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ v8bf as_bf8(const u32x4& u) { return __builtin_bit_cast(v8bf, u); }
__device__ __forceinline__ v8i as_i8(const u32x4& lo, const u32x4& hi)
{
    v8i r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even, with the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0.0 is folded onto +0.0 first so the two rank as one value.
__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP lane moves: row
// shifts by 1, 2, 4 and 8 give prefixes within each 16-lane row, then the two
// row broadcasts (lane 15 into row 1 and 3, lane 31 into rows 2 and 3) carry
// the row totals forward.  Lanes whose source is outside the pattern add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int /*lane*/)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// Inclusive prefix sum within each 16-lane row of the wave (the first four
// steps of wave_incl_scan).
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
    return v;
}

// Value of lane 63 (e.g. the total of an inclusive scan), wave-uniform.
__device__ __forceinline__ uint32_t wave_last(uint32_t v) { return __builtin_amdgcn_readlane(v, 63); }

}  // namespace dsa
