// VSA block selection ("[Video] Integrate H3 SM70 execution, metrics and VSA
// diagnostics", Purpose: top-k = 64 KV blocks per query block; tile means as
// in "[perf] FastH3 two-Spark: gather packed FP4 inputs before head
// projections", key_quant.py / query_pool.py: the tile sum divided by the
// valid count with one rounding, stored in FP32).
//
//   1. vsa_pool_kernel: qbar, kbar = RNE32(sum of a 64-row block / 64). The
//      sum runs in FP64, which is exact for 64 FP16 values (all are integer
//      multiples of 2^-24 below 2^16), so the lane/LDS summation order does
//      not change the result. HBM-bound: Q and K are read once.
//   2. vsa_score_topk_kernel: one workgroup per (b, h, query block):
//      s[j] = sum over d ascending of qbar[d] * kbar[j][d] as an FP64 FMA
//      chain (each FP32 x FP32 product is exact in FP64, so every step rounds
//      exactly like "acc + product"), then a bitonic sort of (s, j) in LDS
//      ordered by s descending and j ascending, and an in-order compaction of
//      the first topk indices, which writes them ascending.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

constexpr int kBlock = 64;
constexpr int kD = 128;
constexpr int kMaxNB = 1024;

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// grid: (B*H*NB, 2) — y selects Q (0) or K (1). 256 threads: thread t sums
// rows 4*(t/16) .. +3 of d-chunk t%16 (8 values), then 16 partial sums per
// column are combined in LDS.
__global__ __launch_bounds__(256) void vsa_pool_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k, int NB,
                                                       int64_t n_bhb, float* __restrict__ pooled)
{
    __shared__ double part[16][kD];
    const int tid = threadIdx.x;
    const int64_t bhb = blockIdx.x;  // (b*H + h) * NB + blk
    const int which = blockIdx.y;
    const uint16_t* src = (which ? k : q) + bhb * (int64_t)kBlock * kD;
    const int col = tid & 15, rg = tid >> 4;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        h8 x = *(const h8*)(src + (rg * 4 + r) * kD + col * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (double)(float)x[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg][col * 8 + e] = acc[e];
    __syncthreads();
    if (tid < kD) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) s += part[i][tid];
        pooled[((int64_t)which * n_bhb + bhb) * kD + tid] = (float)(s * (1.0 / kBlock));
    }
}

struct Entry {
    double s;
    int j;
};

// true when a ranks before c: larger score first, lower index on ties
__device__ __forceinline__ bool before(double as, int aj, double cs, int cj)
{
    return as > cs || (as == cs && aj < cj);
}

template <int NP>  // sort length: power of two >= NB
__global__ __launch_bounds__(256) void vsa_score_topk_kernel(const float* __restrict__ qbar,
                                                             const float* __restrict__ kbar, int NB,
                                                             int topk, int32_t* __restrict__ idx_out,
                                                             double* __restrict__ score_out)
{
    __shared__ double ss[NP];
    __shared__ int sj[NP];
    __shared__ float qv[kD];
    __shared__ unsigned char keep[NP];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;       // (b*H + h) * NB + i
    const int64_t bh = row / NB;
    if (tid < kD) qv[tid] = qbar[row * kD + tid];
    __syncthreads();

    const float* kb = kbar + bh * (int64_t)NB * kD;
    for (int j = tid; j < NP; j += 256) {
        double acc = -INFINITY;
        if (j < NB) {
            const float* kr = kb + (int64_t)j * kD;
            acc = 0.0;
            for (int d = 0; d < kD; d += 4) {
                float4 kv = *(const float4*)(kr + d);
                acc = fma((double)qv[d], (double)kv.x, acc);
                acc = fma((double)qv[d + 1], (double)kv.y, acc);
                acc = fma((double)qv[d + 2], (double)kv.z, acc);
                acc = fma((double)qv[d + 3], (double)kv.w, acc);
            }
            if (score_out) score_out[row * NB + j] = acc;
        }
        ss[j] = acc;
        sj[j] = j;
        keep[j] = 0;
    }
    __syncthreads();

    // bitonic sort, "before" order
    for (int size = 2; size <= NP; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < NP / 2; t += 256) {
                int lo = 2 * t - (t & (stride - 1));
                int hi = lo + stride;
                bool up = (lo & size) == 0;  // ascending-in-"before" segment
                double a = ss[lo], c = ss[hi];
                int aj = sj[lo], cj = sj[hi];
                bool swap = up ? before(c, cj, a, aj) : before(a, aj, c, cj);
                if (swap) {
                    ss[lo] = c;
                    ss[hi] = a;
                    sj[lo] = cj;
                    sj[hi] = aj;
                }
            }
            __syncthreads();
        }
    }
    for (int t = tid; t < topk; t += 256) keep[sj[t]] = 1;
    __syncthreads();

    // in-order compaction by the first wave
    if (tid < 64) {
        int base = 0;
        int32_t* out = idx_out + row * topk;
        for (int j0 = 0; j0 < NB; j0 += 64) {
            int j = j0 + tid;
            bool f = j < NB && keep[j];
            unsigned long long mask = __ballot(f);
            int pos = base + __popcll(mask & ((1ull << tid) - 1ull));
            if (f) out[pos] = j;
            base += __popcll(mask);
        }
    }
}

hipError_t launch_vsa_select(const uint16_t* q, const uint16_t* k, int B, int H, int L, int D,
                             int topk, int32_t* idx_out, double* score_out, float* pooled,
                             hipStream_t stream)
{
    if (D != kD) return hipErrorInvalidValue;
    const int NB = L / kBlock;
    const int64_t n_bhb = (int64_t)B * H * NB;
    if (n_bhb <= 0) return hipSuccess;
    hipLaunchKernelGGL(vsa_pool_kernel, dim3((unsigned)n_bhb, 2), dim3(256), 0, stream, q, k, NB,
                       n_bhb, pooled);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float* qbar = pooled;
    const float* kbar = pooled + n_bhb * kD;
    dim3 grid((unsigned)n_bhb);
    if (NB <= 256)
        hipLaunchKernelGGL(vsa_score_topk_kernel<256>, grid, dim3(256), 0, stream, qbar, kbar, NB,
                           topk, idx_out, score_out);
    else if (NB <= 512)
        hipLaunchKernelGGL(vsa_score_topk_kernel<512>, grid, dim3(256), 0, stream, qbar, kbar, NB,
                           topk, idx_out, score_out);
    else if (NB <= kMaxNB)
        hipLaunchKernelGGL(vsa_score_topk_kernel<kMaxNB>, grid, dim3(256), 0, stream, qbar, kbar, NB,
                           topk, idx_out, score_out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace fa
