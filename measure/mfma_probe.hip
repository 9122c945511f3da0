// MFMA issue-rate and shader-clock probe for gfx950 -- measurement only.
//
// Built into its own library (libdsa_probe.so), apart from the C-ABI library
// of the forward path: nothing on that path calls it.  The benchmark uses it
// to read what the matrix units deliver at a kernel's occupancy, and at what
// clock, so that each kernel's fraction of the published peak can be read
// against what the chip sustains under load.
//
// The published dense peaks assume the matrix units issue every cycle at
// the peak engine clock (2.4 GHz).  Under sustained MFMA load the clock
// drops, and more so when the operands' bits toggle (power), so the probe
// runs on near-constant operands and on pseudo-random ones, and reads the
// shader clock counter (s_memtime) against the constant 100 MHz counter
// (s_memrealtime) over each workgroup's loop.
//
// C ABI (status codes as in include/dsa.h; the detail of a failure in
// dsa_probe_last_error()):
//
//   int dsa_probe_mfma(int kind, int waves_per_simd, int iters, int random_operands,
//                      float* sink, size_t sink_elems,
//                      unsigned long long* clocks, size_t clock_elems,
//                      double* flop, void* stream);
//
//   kind 0: v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3), 8 independent
//           accumulators per round;  kind 1: v_mfma_f32_32x32x16_bf16, 4 per
//           round.  waves_per_simd in {1, 2, 4, 8}: that many workgroups of
//           four waves (one per SIMD) share each CU of the current device.
//   random_operands: 0 = one operand pair for every MFMA, 1 = a different
//           pseudo-random operand pair for each accumulator (bits toggle
//           between consecutive MFMAs, as with real data).
//   sink (device, fp32): one value per wave, n_cu * waves_per_simd * 4
//           needed.  clocks (device, may be NULL): two per workgroup, the
//           elapsed shader cycles and 100 MHz ticks of its loop, n_cu *
//           waves_per_simd * 2 needed.  *flop (host) receives the launch's
//           FLOPs; the caller times the launch on `stream`.
//   Errors: kind or waves_per_simd out of range -> 4 (unsupported); iters
//           outside 1..2^24 -> 2 (shape); flop or sink NULL -> 1; a sink or
//           clock buffer too small -> 6 (workspace); a launch failure -> 7.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "../sparse_attention_04_amd/csrc/hw.h"

namespace {

using namespace dsa;

constexpr int kProbeThreads = 256;   // four waves: one per SIMD of a CU
constexpr int kLdsPerCu = 160 * 1024;

thread_local char g_err[256] = "";

int fail(int st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

__device__ __forceinline__ uint32_t mix(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// A 32-bit word of four e4m3 codes of random sign and mantissa with
// exponent -3 or -1 (|v| in [1/8, 15/16]), or of two bf16 values of random
// sign and mantissa with |v| in [0.5, 2).
__device__ __forceinline__ uint32_t rand_fp8x4(uint32_t h) { return (h & 0xB7B7B7B7u) | 0x20202020u; }
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t h) { return (h & 0x80FF80FFu) | 0x3F003F00u; }

// The dynamic LDS allocation (never touched unless iters < 0) only limits
// how many workgroups share a CU.
template <int KIND, bool RANDOM>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* __restrict__ sink,
                                                                   unsigned long long* __restrict__ clocks,
                                                                   int iters)
{
    extern __shared__ uint8_t occupancy_pad[];
    const int lane = threadIdx.x & 63;
    const uint32_t seed = (blockIdx.x * kProbeThreads + threadIdx.x) * 0x9E3779B9u;
    float r = 0.f;
    unsigned long long t0 = 0, r0 = 0, t1 = 0, r1 = 0;
    if constexpr (KIND == 0) {
        constexpr int NA = 8;
        v8i a[RANDOM ? NA : 1], b[RANDOM ? NA : 1];
#pragma unroll
        for (int j = 0; j < (RANDOM ? NA : 1); ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a[j][i] = RANDOM ? (int)rand_fp8x4(mix(seed + 16 * j + i)) : 0x38383838;   // e4m3 1.0
                b[j][i] = RANDOM ? (int)rand_fp8x4(mix(~seed + 16 * j + i)) : (0x30303030 ^ (lane & 1));
            }
        v4f acc[NA];
        // distinct start values: with equal ones the register allocator moves
        // two accumulators around inside the loop
#pragma unroll
        for (int j = 0; j < NA; ++j) acc[j] = v4f{(float)j, 0.f, 0.f, 0.f};
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < NA; ++j) acc[j] = mfma_fp8_16x16x128(a[RANDOM ? j : 0], b[RANDOM ? j : 0], acc[j]);
        }
        t1 = __builtin_amdgcn_s_memtime();
        r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
        for (int j = 0; j < NA; ++j) r += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    } else {
        constexpr int NA = 4;
        v8bf a[RANDOM ? NA : 1], b[RANDOM ? NA : 1];
#pragma unroll
        for (int j = 0; j < (RANDOM ? NA : 1); ++j)
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const uint32_t ha = rand_bf16x2(mix(seed + 16 * j + i)), hb = rand_bf16x2(mix(~seed + 16 * j + i));
                a[j][i] = RANDOM ? __builtin_bit_cast(__bf16, (uint16_t)ha) : (__bf16)(1.0f + 0.0078125f * (lane & 7));
                a[j][i + 1] = RANDOM ? __builtin_bit_cast(__bf16, (uint16_t)(ha >> 16)) : (__bf16)(1.0f);
                b[j][i] = RANDOM ? __builtin_bit_cast(__bf16, (uint16_t)hb) : (__bf16)(0.5f);
                b[j][i + 1] = RANDOM ? __builtin_bit_cast(__bf16, (uint16_t)(hb >> 16)) : (__bf16)(0.5f);
            }
        v16f acc[NA];
#pragma unroll
        for (int j = 0; j < NA; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[j][v] = (float)(j * 16 + v);
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < NA; ++j) acc[j] = mfma_bf16_32x32x16(a[RANDOM ? j : 0], b[RANDOM ? j : 0], acc[j]);
        }
        t1 = __builtin_amdgcn_s_memtime();
        r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
        for (int j = 0; j < NA; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) r += acc[j][v];
    }
    if (iters < 0) occupancy_pad[threadIdx.x] = (uint8_t)r;
    if (lane == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = r;
    if (clocks != nullptr && threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

template <int KIND, bool RANDOM>
hipError_t launch(int waves_per_simd, int iters, int n_cu, float* sink, unsigned long long* clocks, hipStream_t s)
{
    // one workgroup = one wave on each SIMD; waves_per_simd workgroups fit a CU
    const size_t lds = (size_t)(kLdsPerCu / waves_per_simd) - 1024;
    const void* fn = (const void*)mfma_probe_kernel<KIND, RANDOM>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mfma_probe_kernel<KIND, RANDOM>), dim3((unsigned)(n_cu * waves_per_simd)),
                       dim3(kProbeThreads), lds, s, sink, clocks, iters);
    return hipGetLastError();
}

}  // namespace

extern "C" {

const char* dsa_probe_last_error(void) { return g_err; }

int dsa_probe_mfma(int kind, int waves_per_simd, int iters, int random_operands, float* sink, size_t sink_elems,
                   unsigned long long* clocks, size_t clock_elems, double* flop, void* stream)
{
    const char* fn = "dsa_probe_mfma";
    if (kind != 0 && kind != 1)
        return fail(4, "%s: kind=%d is neither 0 (FP8 16x16x128) nor 1 (BF16 32x32x16)", fn, kind);
    if (waves_per_simd != 1 && waves_per_simd != 2 && waves_per_simd != 4 && waves_per_simd != 8)
        return fail(4, "%s: waves_per_simd=%d is not 1, 2, 4 or 8", fn, waves_per_simd);
    if (iters < 1 || iters > (1 << 24)) return fail(2, "%s: iters=%d outside 1..2^24", fn, iters);
    if (flop == nullptr) return fail(1, "%s: flop is NULL", fn);
    if (sink == nullptr) return fail(1, "%s: sink is NULL", fn);
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(7, "%s: %s", fn, hipGetErrorString(e));
    const size_t wgs = (size_t)n_cu * waves_per_simd;
    if (sink_elems < wgs * 4) return fail(6, "%s: sink holds %zu floats, %zu needed", fn, sink_elems, wgs * 4);
    if (clocks != nullptr && clock_elems < wgs * 2)
        return fail(6, "%s: clocks holds %zu values, %zu needed", fn, clock_elems, wgs * 2);
    const double per_mfma = kind == 0 ? 2.0 * 16 * 16 * 128 : 2.0 * 32 * 32 * 16;
    *flop = (double)wgs * 4 * iters * (kind == 0 ? 8 : 4) * per_mfma;
    hipStream_t s = (hipStream_t)stream;
    if (kind == 0)
        e = random_operands ? launch<0, true>(waves_per_simd, iters, n_cu, sink, clocks, s)
                            : launch<0, false>(waves_per_simd, iters, n_cu, sink, clocks, s);
    else
        e = random_operands ? launch<1, true>(waves_per_simd, iters, n_cu, sink, clocks, s)
                            : launch<1, false>(waves_per_simd, iters, n_cu, sink, clocks, s);
    if (e != hipSuccess) return fail(7, "%s: %s", fn, hipGetErrorString(e));
    g_err[0] = '\0';
    return 0;
}

}  // extern "C"
