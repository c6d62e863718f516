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

// Per-row E4M3 quantization of the prefix attention's queries and keys
// ([P5] query_pool.py, the PREFIX_FP8 round trip of the prefix queries;
// prefix_quant.py, the same for the keys): per (b, h, row) of a bfloat16
// [B, H, L, 128] view, scale = max |x| / 448, inv = scale == 0 ? 0 : 1 / scale,
// code = RNE_e4m3(clamp(x * inv, +-448)), each step rounding once in FP32 (the
// round trip of prefix_fp8_gather_kernel without its decode). Codes go to a
// contiguous [B, H, L, 128] byte array, scales to FP32 [B, H, L].
// grid: ceil(B * H * L / 16); one 16-lane group per row, lane l holding
// elements 8l .. 8l+7.
__global__ __launch_bounds__(256) void fp8_rows_quantize_kernel(const uint16_t* __restrict__ x, int64_t x_sb,
                                                                int64_t x_sh, int64_t x_ss, int H, int L,
                                                                int64_t n_rows, uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales)
{
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b * H + h) * L + i
    const int l = threadIdx.x & 15;
    if (row >= n_rows) return;  // a group is all in or all out
    const int i = (int)(row % L);
    const int64_t bh = row / L;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const u4 w = *(const u4*)(x + b * x_sb + h * x_sh + i * x_ss + l * 8);
    float v[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                  bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax / 448.f;
    const float inv = scale == 0.f ? 0.f : 1.f / scale;
    uint32_t c[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const float x0 = fminf(fmaxf(v[4 * p] * inv, -448.f), 448.f);
        const float x1 = fminf(fmaxf(v[4 * p + 1] * inv, -448.f), 448.f);
        const float x2 = fminf(fmaxf(v[4 * p + 2] * inv, -448.f), 448.f);
        const float x3 = fminf(fmaxf(v[4 * p + 3] * inv, -448.f), 448.f);
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
        c[p] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, lo, true);
    }
    *(uint2*)(codes + row * kPD + l * 8) = make_uint2(c[0], c[1]);
    if (l == 0) scales[row] = scale;
}

hipError_t launch_fp8_rows_quantize(const uint16_t* x, int64_t x_sb, int64_t x_sh, int64_t x_ss, int B, int H, int L,
                                    uint8_t* codes, float* scales, hipStream_t stream)
{
    const int64_t n_rows = (int64_t)B * H * L;
    if (n_rows <= 0) return hipSuccess;
    const int64_t grid = (n_rows + 15) / 16;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fp8_rows_quantize_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, x_sb, x_sh, x_ss, H,
                       L, n_rows, codes, scales);
    return hipGetLastError();
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
