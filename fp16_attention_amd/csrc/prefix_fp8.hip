// FP8 round trip of prefix keys with the valid-row gather ("[perf] FastH3
// two-Spark: gather packed FP4 inputs before head projections",
// prefix_quant.py: quantize_gather_prefix_kv; key_quant.py applies the same
// key round trip in its prefix preparation). For every (b, r, h), with x the
// FP32 values of K's token
// index[r], head h (D = 128, bfloat16):
//   scale = max |x| / 448, inv = scale == 0 ? 0 : 1 / scale,
//   k_out = RNE_bf16( decode( RNE_e4m3( clamp(x * inv, +-448) ) ) * scale ),
// each step rounding once in FP32; v_out is V's row, gathered alike. K stays
// bfloat16 for the attention that follows.
//
// HBM-bound: one 16-lane group per (b, r, h) vector; lane l holds elements
// 8l .. 8l+7 (16 bytes) of K and of V, the group's maximum is an exchange
// within the 16 lanes, and E4M3 encode/decode are the hardware conversions
// (OCP E4M3FN, round to nearest even on encode).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr int kPD = 128;  // head dimension

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two FP32 values -> their E4M3 round trip times scale, as two bfloat16 in one word
__device__ __forceinline__ uint32_t roundtrip2(float a, float b, float inv, float scale)
{
    const float x0 = fminf(fmaxf(a * inv, -448.f), 448.f);
    const float x1 = fminf(fmaxf(b * inv, -448.f), 448.f);
    const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    const f2 d = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
    const __bf16 y0 = (__bf16)(d.x * scale), y1 = (__bf16)(d.y * scale);
    return (uint32_t)__builtin_bit_cast(uint16_t, y0) | ((uint32_t)__builtin_bit_cast(uint16_t, y1) << 16);
}

// grid: ceil(B * rows * H / 16); 256 threads = 16 groups of 16 lanes
__global__ __launch_bounds__(256) void prefix_fp8_gather_kernel(const uint16_t* __restrict__ k,
                                                                const uint16_t* __restrict__ v, int N, int H,
                                                                const int32_t* __restrict__ index, int rows,
                                                                int64_t n_vec, uint16_t* __restrict__ ko,
                                                                uint16_t* __restrict__ vo)
{
    const int64_t vec = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // ((b * rows) + r) * H + h
    const int l = threadIdx.x & 15;
    // a group is all in or all out, so the exchanges below stay within live lanes
    if (vec >= n_vec) return;
    const int h = (int)(vec % H);
    const int64_t br = vec / H;
    const int r = (int)(br % rows);
    const int64_t b = br / rows;
    const int src = min(max(index[r], 0), N - 1);
    const int64_t in_off = ((b * N + src) * H + h) * kPD + l * 8;
    const u4 kw = *(const u4*)(k + in_off);
    const u4 vw = *(const u4*)(v + in_off);
    float x[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                  bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax / 448.f;
    const float inv = scale == 0.f ? 0.f : 1.f / scale;
    const u4 out = {roundtrip2(x[0], x[1], inv, scale), roundtrip2(x[2], x[3], inv, scale),
                    roundtrip2(x[4], x[5], inv, scale), roundtrip2(x[6], x[7], inv, scale)};
    const int64_t out_off = vec * kPD + l * 8;
    *(u4*)(ko + out_off) = out;
    *(u4*)(vo + out_off) = vw;
}

hipError_t launch_prefix_fp8_gather(const uint16_t* k, const uint16_t* v, int B, int N, int H,
                                    const int32_t* index, int rows, uint16_t* k_out, uint16_t* v_out,
                                    hipStream_t stream)
{
    const int64_t n_vec = (int64_t)B * rows * H;
    if (n_vec <= 0) return hipSuccess;
    const int64_t grid = (n_vec + 15) / 16;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefix_fp8_gather_kernel, dim3((unsigned)grid), dim3(256), 0, stream, k, v, N, H, index,
                       rows, n_vec, k_out, v_out);
    return hipGetLastError();
}

}  // namespace fa
