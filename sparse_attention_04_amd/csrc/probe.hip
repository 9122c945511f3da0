// MFMA issue-rate probe: back-to-back independent matrix instructions with
// every operand in registers, at a chosen number of waves per SIMD.  The
// published dense peaks assume the matrix units never wait; at the low
// occupancies the hot-path kernels run at (one or two waves per SIMD, set by
// their register and LDS use), a single wave cannot issue every cycle, and
// this probe measures what such a wave can reach.  It is a measurement tool
// only: nothing on the hot path calls it.
#include <hip/hip_runtime.h>

#include "hw.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kProbeThreads = 256;   // four waves: one per SIMD of a CU
constexpr int kLdsPerCu = 160 * 1024;

// KIND 0: v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3), 8 independent accumulators.
// KIND 1: v_mfma_f32_32x32x16_bf16, 4 independent accumulators.
// The dynamic LDS allocation (never touched unless iters < 0) only limits
// how many workgroups share a CU.
template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* __restrict__ sink, int iters)
{
    extern __shared__ uint8_t occupancy_pad[];
    const int lane = threadIdx.x & 63;
    float r = 0.f;
    if constexpr (KIND == 0) {
        v8i a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = 0x38383838;                     // e4m3 1.0
            b[i] = 0x30303030 ^ (lane & 1);        // e4m3 0.5 (one byte 0.5625 on odd lanes)
        }
        v4f acc[8];
        // distinct start values: with equal ones the register allocator moves
        // two accumulators around inside the loop
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = v4f{(float)j, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = mfma_fp8_16x16x128(a, b, acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) r += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    } else {
        v8bf a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(1.0f + 0.0078125f * (lane & 7));
            b[i] = (__bf16)(0.5f);
        }
        v16f acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = mfma_bf16_32x32x16(a, b, acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) r += acc[j][v];
    }
    if (iters < 0) occupancy_pad[threadIdx.x] = (uint8_t)r;
    if (lane == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = r;
}

}  // namespace

int mfma_probe_mfmas_per_iter(int kind) { return kind == 0 ? 8 : 4; }

double mfma_probe_flop_per_mfma(int kind) { return kind == 0 ? 2.0 * 16 * 16 * 128 : 2.0 * 32 * 32 * 16; }

hipError_t launch_mfma_probe(int kind, int waves_per_simd, int iters, int n_cu, float* sink, hipStream_t s)
{
    // one workgroup = one wave on each SIMD; waves_per_simd workgroups fit a CU
    const size_t lds = (size_t)(kLdsPerCu / waves_per_simd) - 1024;
    const void* fn = kind == 0 ? (const void*)mfma_probe_kernel<0> : (const void*)mfma_probe_kernel<1>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(n_cu * waves_per_simd));
    if (kind == 0)
        hipLaunchKernelGGL(mfma_probe_kernel<0>, grid, dim3(kProbeThreads), lds, s, sink, iters);
    else
        hipLaunchKernelGGL(mfma_probe_kernel<1>, grid, dim3(kProbeThreads), lds, s, sink, iters);
    return hipGetLastError();
}

}  // namespace dsa
