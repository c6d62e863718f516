// FP16 matrix-core rate that the chip sustains on varied operands.
//
// A measurement aid for the attention kernels' roofline, with no counterpart
// in the method itself: the published dense FP16 peak assumes the full shader
// clock, which the chip holds only while its matrix cores switch few operand
// bits. This kernel issues nothing but v_mfma_f32_32x32x16_f16 on operands
// that differ from lane to lane (as random FP16 data does), four independent
// accumulators per wave, two 4-wave workgroups per CU, so the MFMA pipe of
// every SIMD stays busy; its rate is the attainable FP16 MFMA throughput under
// the board's power limit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa16measure.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kBlocks = 512;  // two per CU on 256 CUs
constexpr int kThreads = 256;

// an FP16 value in [-1, 1) from a 32-bit integer mix of the element index
__device__ _Float16 varied(uint32_t i)
{
    uint32_t x = i * 0x9E3779B1u;
    x ^= x >> 15;
    x *= 0x85EBCA77u;
    x ^= x >> 13;
    return (_Float16)((float)(int)(x & 0x3FFu) * (1.f / 512.f) - 1.f);
}

__global__ __launch_bounds__(kThreads) void mfma_ceiling_kernel(float* out, int iters)
{
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    h8 a0, a1, b0, b1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a0[i] = varied(g * 32u + i);
        a1[i] = varied(g * 32u + 8 + i);
        b0[i] = varied(g * 32u + 16 + i);
        b1[i] = varied(g * 32u + 24 + i);
    }
    f16x c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[g] = s;
}

}  // namespace

extern "C" int fa_mfma_ceiling(int iters, float* out, void* stream)
{
    if (!out) return FAM_ERR_NULL;
    if (iters < 1 || iters > (1 << 20)) return FAM_ERR_SHAPE;
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(kBlocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? FAM_OK : FAM_ERR_HIP + (int)e;
}
