// VSA block selection ("[Video] Integrate H3 SM70 execution, metrics and VSA
// diagnostics", Purpose: top-k = 64 KV blocks per query block; tile means as
// in "[perf] FastH3 two-Spark: gather packed FP4 inputs before head
// projections", key_quant.py / query_pool.py: the tile sum divided by the
// valid count with one rounding, stored in FP32).
//
//   1. vsa_pool_kernel: qbar, kbar = RNE32(sum of a block's rows / their
//      count); blocks hold 64 rows, the last one of a sequence whose length is
//      not a multiple of 64 fewer. One wave per block; each lane sums 16 rows
//      of 8 columns in FP64, which is exact for FP16 inputs (all are integer
//      multiples of 2^-24 below 2^16, and 64 of them fit in 53 bits), so the
//      order of the partial sums does not change the result. HBM-bound: Q and
//      K are read once.
//   2. vsa_scores_kernel: s[i][j] = sum over d ascending of qbar[i][d] *
//      kbar[j][d], one FP64 FMA chain per (i, j) (each FP32 x FP32 product is
//      exact in FP64, so every step rounds exactly like "acc + product").
//      A workgroup computes a 64 x 64 tile of one (b, h) on the FP64 matrix
//      cores, whose 16x16x4 step is four such FMAs in ascending k.
//   3. vsa_topk_kernel: one wave per query block. The scores are mapped to
//      order-preserving 64-bit keys and a bitwise radix select finds the
//      topk-th largest value T, stopping as soon as the keys that share T's
//      leading bits are exactly the ones still needed; the selection is every
//      block with s > T plus the lowest-index blocks with s == T, written in
//      ascending order with a ballot compaction.
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

// The FP32 value nearest to sum / count, ties to even, for an exact FP64 sum
// of FP16 values and a count of at most 64: the FP64 quotient rounded to FP32
// is the answer or one of its neighbours, and their distances |c * count -
// sum| are exact in FP64 (a 24-bit c times a 7-bit count).
__device__ __forceinline__ float mean_rn(double sum, int count)
{
    // a power-of-two count (every full block): sum / count is exact in FP64
    // (the sum is a multiple of 2^-24 below 2^22), so its one rounding to FP32
    // is the answer
    if ((count & (count - 1)) == 0) return (float)(sum * (1.0 / count));
    const float c0 = (float)(sum / count);
    const float cand[2] = {nextafterf(c0, -INFINITY), nextafterf(c0, INFINITY)};
    float best = c0;
    double err = fabs((double)c0 * count - sum);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const double e = fabs((double)cand[i] * count - sum);
        if (e < err || (e == err && (__float_as_uint(cand[i]) & 1u) == 0)) {
            best = cand[i];
            err = e;
        }
    }
    return best;
}

// grid: (B*H*NB / 4 rounded up, 2) — y selects Q (0) or K (1); 4 waves, one
// block each. Lane l reads columns 8*(l%16) .. +7 of rows l/16 + 4i, i < 16,
// of the block's valid rows, with nontemporal loads (Q and K are read once
// here; measured 8% faster than cached loads).
__global__ __launch_bounds__(256) void vsa_pool_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k, int64_t n_bhb, int L,
                                                       int NB, float* __restrict__ pooled)
{
    const int lane = threadIdx.x & 63;
    const int64_t bhb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*H + h) * NB + blk
    if (bhb >= n_bhb) return;
    const int which = blockIdx.y;
    const int64_t bh = bhb / NB;
    const int blk = (int)(bhb - bh * NB);
    const int count = min(kBlock, L - blk * kBlock);
    const uint16_t* src = (which ? k : q) + (bh * L + (int64_t)blk * kBlock) * kD;
    const int col = lane & 15, r0 = lane >> 4;
    h8 x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = r0 + 4 * i;
        x[i] = row < count ? __builtin_bit_cast(h8, __builtin_nontemporal_load((const u4*)(src + row * kD + col * 8))) : h8{};
    }
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (double)(float)x[i][e];
    // lanes col, col+16, col+32, col+48 hold the four partial sums of a column
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc[e] += __shfl_xor(acc[e], 16);
        acc[e] += __shfl_xor(acc[e], 32);
    }
    if (lane < 16) {
        float* dst = pooled + ((int64_t)which * n_bhb + bhb) * kD + col * 8;
        float4 lo = {mean_rn(acc[0], count), mean_rn(acc[1], count), mean_rn(acc[2], count),
                     mean_rn(acc[3], count)};
        float4 hi = {mean_rn(acc[4], count), mean_rn(acc[5], count), mean_rn(acc[6], count),
                     mean_rn(acc[7], count)};
        *(float4*)dst = lo;
        *(float4*)(dst + 4) = hi;
    }
}

// grid: (ceil(NB/64)^2, B*H); 4 waves per 64 x 64 tile of one (b, h), each
// wave a 32 x 32 quarter, on the FP64 matrix cores: each k-step feeds four
// v_mfma_f64_16x16x4f64, one per 16 x 16 part of the quarter. That
// instruction folds its four products into each output as four FMAs in
// ascending k, so the 32 steps are the same ascending-d FMA chain per (i, j)
// as an FP64 loop. The tile's 64 query means and 64 key means are staged in
// LDS 64 dimensions at a time, as FP32 rows padded to 68 floats (35 KB, four
// workgroups per CU), so the operand reads below hit 64 distinct banks. At
// step s lane l supplies row l % 16, dimension 4 s + l / 16 of the A (query)
// and B (key) operands, widened to FP64 exactly; output register r of lane l
// is row l / 16 + 4 r, column l % 16.
constexpr int kST = 64;       // score tile edge
constexpr int kDC = 64;       // dimensions per staged chunk
constexpr int kRowPad = 68;   // floats per staged row
__global__ __launch_bounds__(256) void vsa_scores_kernel(const float* __restrict__ qbar,
                                                         const float* __restrict__ kbar, int NB,
                                                         double* __restrict__ scores)
{
    typedef double d4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) float qs[kST][kRowPad];
    __shared__ __attribute__((aligned(16))) float ks[kST][kRowPad];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tiles = (NB + kST - 1) / kST;
    const int i0 = (blockIdx.x / tiles) * kST, j0 = (blockIdx.x % tiles) * kST;
    const int64_t bh = blockIdx.y;
    const float* qb = qbar + bh * (int64_t)NB * kD;
    const float* kb = kbar + bh * (int64_t)NB * kD;
    const int rr = lane & 15, kq = lane >> 4;
    const int qr = 32 * (wave >> 1) + rr, kr = 32 * (wave & 1) + rr;
    d4 c00 = {0, 0, 0, 0}, c01 = c00, c10 = c00, c11 = c00;
    for (int d0 = 0; d0 < kD; d0 += kDC) {
        if (d0 > 0) __syncthreads();  // every wave is done with the previous chunk
        // 64 rows x 16 float4 per tensor, 4 per thread each; rows past NB are
        // zeros (their scores are not written)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = tid + 256 * u;  // float4 index in the 64 x 16 grid
            const int r = e >> 4, c4 = e & 15;
            float4 qv = {0.f, 0.f, 0.f, 0.f}, kv = qv;
            if (i0 + r < NB) qv = *(const float4*)(qb + (int64_t)(i0 + r) * kD + d0 + 4 * c4);
            if (j0 + r < NB) kv = *(const float4*)(kb + (int64_t)(j0 + r) * kD + d0 + 4 * c4);
            *(float4*)&qs[r][4 * c4] = qv;
            *(float4*)&ks[r][4 * c4] = kv;
        }
        __syncthreads();
        // the operands of step s + 2 are read while the MFMAs of step s issue
        constexpr int kSteps = kDC / 4, kAhead = 2;
        float op[kAhead][4];
#pragma unroll
        for (int t = 0; t < kAhead; ++t) {
            op[t][0] = qs[qr][4 * t + kq];
            op[t][1] = qs[qr + 16][4 * t + kq];
            op[t][2] = ks[kr][4 * t + kq];
            op[t][3] = ks[kr + 16][4 * t + kq];
        }
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            const int slot = st % kAhead;
            const double a0 = op[slot][0], a1 = op[slot][1], b0 = op[slot][2], b1 = op[slot][3];
            if (st + kAhead < kSteps) {
                const int k0 = 4 * (st + kAhead);
                op[slot][0] = qs[qr][k0 + kq];
                op[slot][1] = qs[qr + 16][k0 + kq];
                op[slot][2] = ks[kr][k0 + kq];
                op[slot][3] = ks[kr + 16][k0 + kq];
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this step's MFMAs
            c00 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, c00, 0, 0, 0);
            c01 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, c01, 0, 0, 0);
            c10 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, c10, 0, 0, 0);
            c11 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, c11, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    const int col = lane & 15, rq = lane >> 4;
    auto put = [&](const d4& c, int ti, int tj) {
        const int j = j0 + 32 * (wave & 1) + 16 * tj + col;
        if (j >= NB) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 32 * (wave >> 1) + 16 * ti + rq + 4 * r;
            if (i < NB) scores[(bh * NB + i) * (int64_t)NB + j] = c[r];
        }
    };
    put(c00, 0, 0);
    put(c01, 0, 1);
    put(c10, 1, 0);
    put(c11, 1, 1);
}

// Order-preserving map of a double to uint64 (larger value -> larger key);
// -0 is folded into +0 first, so equal values compare equal.
__device__ __forceinline__ uint64_t order_key(double s)
{
    s = s + 0.0;
    const uint64_t u = __builtin_bit_cast(uint64_t, s);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// grid: ceil(B*H*NB / 4); 4 waves, one query block (row) each. PER keys per
// lane (key j = lane + 64 * m, m < PER), PER * 64 >= NB.
template <int PER>
__global__ __launch_bounds__(256) void vsa_topk_kernel(const double* __restrict__ scores, int NB, int topk,
                                                       int64_t rows, int32_t* __restrict__ idx_out)
{
    constexpr int kPerLane = PER;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const double* sr = scores + row * NB;
    // all loads first (indices clamped into the row), so they are in flight
    // together; then the keys
    double sv[kPerLane];
#pragma unroll
    for (int m = 0; m < kPerLane; ++m) sv[m] = sr[min(lane + 64 * m, NB - 1)];
    uint64_t key[kPerLane];
#pragma unroll
    for (int m = 0; m < kPerLane; ++m)
        key[m] = lane + 64 * m < NB ? order_key(sv[m]) : 0ull;  // key 0 is below every real key
    // Radix select, most significant bit first: T is the largest value with
    // at least topk keys >= T. After bits 63..b of T are fixed (in prefix),
    // `need` more keys must come from the `match` keys whose bits 63..b equal
    // prefix's; once match == need those are all taken and the lower bits of
    // T no longer matter, so the walk stops there. The bits every key shares
    // (sign and most of the exponent, for scores of one magnitude) are fixed
    // up front from the AND and OR of all keys.
    uint64_t k_and = ~0ull, k_or = 0ull;
#pragma unroll
    for (int m = 0; m < kPerLane; ++m) {
        if (lane + 64 * m < NB) {
            k_and &= key[m];
            k_or |= key[m];
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        k_and &= __shfl_xor(k_and, o);
        k_or |= __shfl_xor(k_or, o);
    }
    const uint64_t differ = k_and ^ k_or;  // bits where some keys differ
    const int top = differ ? 63 - __clzll(differ) : -1;  // highest such bit
    const uint64_t common = top < 0 ? ~0ull : top >= 63 ? 0ull : ~((2ull << top) - 1ull);  // bits above top
    uint64_t prefix = k_and & common;
    int need = topk, match = NB, low = top + 1;  // low: bits below `low` are undecided
    for (int bit = (match == need ? -1 : top); bit >= 0; --bit) {
        const uint64_t cand = prefix | (1ull << bit);
        const uint64_t hi_mask = ~((1ull << bit) - 1ull);  // bits bit..63
        // a key past the row is 0 and never equals cand (cand has a bit set)
        int cnt = 0;
#pragma unroll
        for (int m = 0; m < kPerLane; ++m) cnt += __popcll(__builtin_amdgcn_ballot_w64((key[m] & hi_mask) == cand));
        if (cnt >= need) {
            prefix = cand;
            match = cnt;
        } else {
            need -= cnt;
            match -= cnt;
        }
        low = bit;
        if (match == need) break;
    }
    // keep keys whose bits 63..low exceed prefix's, and the `need` lowest-index
    // keys whose bits 63..low equal them (all of them after an early stop)
    int32_t* out = idx_out + row * topk;
    const uint64_t tp = low >= 64 ? 0ull : prefix >> low;
    int base = 0, eq_taken = 0;
#pragma unroll
    for (int m = 0; m < kPerLane; ++m) {
        const int j = lane + 64 * m;
        const bool valid = j < NB;
        const uint64_t kt = low >= 64 ? 0ull : key[m] >> low;
        const bool gt = valid && kt > tp;
        const bool eq = valid && kt == tp;
        const uint64_t eq_mask = __ballot(eq);
        const int eq_before = __popcll(eq_mask & ((1ull << lane) - 1ull));
        const bool take = gt || (eq && eq_taken + eq_before < need);
        const uint64_t take_mask = __ballot(take);
        if (take) out[base + __popcll(take_mask & ((1ull << lane) - 1ull))] = j;
        base += __popcll(take_mask);
        eq_taken += __popcll(eq_mask);
    }
}

// The pooled tile means of one tensor (the pooled V of the VSA coarse
// branch): the pooling kernel with only its first (y = 0) input.
hipError_t launch_vsa_tile_means(const uint16_t* x, int B, int H, int L, int D, float* out, hipStream_t stream)
{
    if (D != kD) return hipErrorInvalidValue;
    const int NB = (L + kBlock - 1) / kBlock;
    const int64_t n_bhb = (int64_t)B * H * NB;
    if (n_bhb <= 0) return hipSuccess;
    if ((n_bhb + 3) / 4 > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(vsa_pool_kernel, dim3((unsigned)((n_bhb + 3) / 4), 1), dim3(256), 0, stream, x, x, n_bhb, L,
                       NB, out);
    return hipGetLastError();
}

hipError_t launch_vsa_select(const uint16_t* q, const uint16_t* k, int B, int H, int L, int D,
                             int topk, int32_t* idx_out, double* scores, float* pooled,
                             hipStream_t stream)
{
    if (D != kD) return hipErrorInvalidValue;
    const int NB = (L + kBlock - 1) / kBlock;
    if (NB > kMaxNB) return hipErrorInvalidValue;
    const int64_t n_bhb = (int64_t)B * H * NB;
    if (n_bhb <= 0) return hipSuccess;
    hipLaunchKernelGGL(vsa_pool_kernel, dim3((unsigned)((n_bhb + 3) / 4), 2), dim3(256), 0, stream, q, k,
                       n_bhb, L, NB, pooled);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float* qbar = pooled;
    const float* kbar = pooled + n_bhb * kD;
    const int tiles = (NB + kST - 1) / kST;
    hipLaunchKernelGGL(vsa_scores_kernel, dim3((unsigned)(tiles * tiles), (unsigned)(B * H)), dim3(256), 0,
                       stream, qbar, kbar, NB, scores);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (NB <= 9 * 64)
        hipLaunchKernelGGL(vsa_topk_kernel<9>, dim3((unsigned)((n_bhb + 3) / 4)), dim3(256), 0, stream, scores,
                           NB, topk, n_bhb, idx_out);
    else
        hipLaunchKernelGGL(vsa_topk_kernel<kMaxNB / 64>, dim3((unsigned)((n_bhb + 3) / 4)), dim3(256), 0,
                           stream, scores, NB, topk, n_bhb, idx_out);
    return hipGetLastError();
}

}  // namespace fa
