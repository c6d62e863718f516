// VSA block lists of 128-token blocks ("[perf] FastH3 two-Spark: gather
// packed FP4 inputs before head projections", block_lists.py: descending
// variable-length key-block lists per 128-token query block built from two
// 64-token halves, per-half valid counts and 4-bit quadrant masks).
//
// From a square tile mask over T tiles of `tile` = 64 * HT tokens and the
// valid tokens of each tile: halves are 64 tokens (HT per tile), block c is
// halves a = 2c, e = 2c + 1, with va = clamp(valid[a / HT] - (a % HT) * 64,
// 0, 64) (0 past the sequence). For query block r (halves q0 = 2r, q1 = 2r+1)
// the quadrant mask of key block c is
//   [m(q0,a) & va>0] + 2 [m(q0,e) & ve>0] + 4 [m(q1,a) & va>0] + 8 [m(q1,e) & ve>0],
// m(q, k) = mask[q / HT][k / HT] inside the sequence, and a padded odd last
// query half q1 sees key half 0 only. Key blocks with a nonzero mask are
// listed in descending order, the rest of the row is zero, and the count is
// stored.
//
// One wave per (b, h, query block): lane l takes key blocks NB-1-(64 m + l),
// so 64 consecutive descending columns per step; a ballot and a prefix
// popcount give each kept column its list position. The mask reads are two
// rows of bytes, the valid counts a small vector: the kernel is bound by its
// list writes (B * H * NB^2 * 5 bytes).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

namespace {

__device__ __forceinline__ int half_valid(const int32_t* valid, int T, int HT, int half)
{
    if (half >= T * HT) return 0;
    return min(max(valid[half / HT] - (half % HT) * 64, 0), 64);
}

__device__ __forceinline__ bool half_mask(const uint8_t* m, int T, int HT, int qh, int kh)
{
    if (qh >= T * HT) return kh == 0;  // the padded odd query half sees key half 0 only
    if (kh >= T * HT) return false;
    return m[(int64_t)(qh / HT) * T + kh / HT] != 0;
}

__global__ __launch_bounds__(256) void vsa_block_lists_kernel(const uint8_t* __restrict__ mask,
                                                              const int32_t* __restrict__ valid, int T, int HT,
                                                              int NB, int64_t rows, int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ kv_valid,
                                                              uint8_t* __restrict__ quad)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * H + h) * NB + r
    if (row >= rows) return;
    const int64_t bh = row / NB;
    const int r = (int)(row - bh * NB);
    const uint8_t* m = mask + bh * (int64_t)T * T;
    int32_t* list = idx + row * NB;
    uint8_t* qlist = quad ? quad + row * NB : nullptr;
    const int q0 = 2 * r, q1 = 2 * r + 1;
    int n = 0;
    for (int base = 0; base < NB; base += 64) {
        const int c = NB - 1 - (base + lane);
        int bits = 0;
        if (c >= 0) {
            const int a = 2 * c, e = 2 * c + 1;
            const bool va = half_valid(valid, T, HT, a) > 0, ve = half_valid(valid, T, HT, e) > 0;
            bits = (half_mask(m, T, HT, q0, a) && va) + 2 * (half_mask(m, T, HT, q0, e) && ve) +
                   4 * (half_mask(m, T, HT, q1, a) && va) + 8 * (half_mask(m, T, HT, q1, e) && ve);
        }
        const uint64_t keep = __ballot(bits != 0);
        if (bits) {
            const int pos = n + __popcll(keep & ((1ull << lane) - 1ull));
            list[pos] = c;
            if (qlist) qlist[pos] = (uint8_t)bits;
        }
        n += __popcll(keep);
    }
    for (int t = n + lane; t < NB; t += 64) {
        list[t] = 0;
        if (qlist) qlist[t] = 0;
    }
    if (lane == 0) counts[row] = n;
    if (row == 0)
        for (int h = lane; h < 2 * NB; h += 64) kv_valid[h] = half_valid(valid, T, HT, h);
}

}  // namespace

hipError_t launch_vsa_block_lists(const uint8_t* mask, const int32_t* valid, int B, int H, int T, int tile,
                                  int32_t* idx, int32_t* counts, int32_t* kv_valid, uint8_t* quad,
                                  hipStream_t stream)
{
    const int HT = tile / 64;
    const int NB = (T * HT + 1) / 2;
    const int64_t rows = (int64_t)B * H * NB;
    if (rows <= 0) return hipSuccess;
    if ((rows + 3) / 4 > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(vsa_block_lists_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, mask, valid,
                       T, HT, NB, rows, idx, counts, kv_valid, quad);
    return hipGetLastError();
}

}  // namespace fa
