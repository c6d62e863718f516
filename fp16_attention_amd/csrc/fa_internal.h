// Internal launch interface between the C-ABI layer (abi.cpp) and the HIP
// kernels. Not installed; the public interface is include/fa16attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "work_items.h"

namespace fa {

// KV_BF16: Q, K, V and O are BF16 (dense attention only); it streams like
// KV_FP16 and differs in the MFMA type and the rounding of P and O.
// KV_E4M3_PAGED: E4M3 codes decoded exactly to FP16 in registers; used when
// k_scale is a power of two that keeps every decode * k_scale an exact FP16
// value, so folding k_scale into the softmax constant changes nothing.
// KV_E4M3_PAGED_SCALED: for any other k_scale, each workgroup converts every
// K code tile once, in LDS, into the FP16 values the conversion defines,
// RNE16(RNE32(decode * k_scale)); V is decoded exactly in registers.
// KV_FP8QK: dense attention whose queries and keys are E4M3 codes with an
// FP32 scale per row (QK^T on the FP8 matrix cores, the row scales applied to
// the FP32 scores); V, P and O are BF16.
enum KvSource { KV_FP16 = 0, KV_E4M3_PAGED = 1, KV_BF16 = 2, KV_E4M3_PAGED_SCALED = 3, KV_FP8QK = 4 };

// Everything one attention launch needs; passed by value as the kernel
// argument. Strides are in elements. The Geometry part (shape, split and
// work items) is what the work-item decode reads.
struct AttnArgs : Geometry {
    const _Float16* q;
    int64_t q_sb, q_sh, q_ss;
    const _Float16* k;
    int64_t k_sb, k_sh, k_ss;
    const _Float16* v;
    int64_t v_sb, v_sh, v_ss;
    _Float16* o;
    int64_t o_sb, o_sh, o_ss;
    float* lse;  // optional [B, Hq, Lq]

    // paged E4M3 source
    const uint8_t* kc;
    const uint8_t* vc;
    const int32_t* table;
    int64_t table_stride;
    int num_pages;
    int page_shift;  // log2(page_size)

    // block lists
    const int32_t* idx;  // [B, Hq, nqb, topk]

    // FP8 queries and keys (KV_FP8QK): codes [B, Hq, Lq, D] (kc: [B, Hkv, Lkv, D])
    // contiguous, FP32 row scales [B, Hq, Lq] and [B, Hkv, Lkv]
    const uint8_t* qc;
    const float* qsc;
    const float* ksc;

    // split-KV partial states (FP32): o_part [nseg][B*Hq][part_lq][D]
    // unnormalised, ml_part [nseg][B*Hq][part_lq][2] = (running max in log2
    // units, running sum). part_lq = Lq for the causal prefill; for block
    // lists only the dense-prefix query rows are split. A query tile whose
    // keys span nt 64-key units has segments of seg_units(nt, nseg) units.
    float* o_part;
    float* ml_part;

    float c;       // softmax scale * log2(e) (times k_scale for KV_E4M3_PAGED)
    float oscale;  // output scale (v_scale for E4M3, else 1)
    float kscale;  // KV_E4M3_PAGED_SCALED: the K conversion scale
};

struct MergeArgs {
    const float* o_part;
    const float* ml_part;
    _Float16* o;
    int64_t o_sb, o_sh, o_ss;
    float* lse;
    int64_t lse_sh;  // LSE elements per (b, h)
    int B, Hq, Lq, nseg, n_qt, rows_per_tile;
    int64_t offset;
    int Lkv;
    float oscale;
};

// Supplies a call's workspace once all its arguments are validated: used by
// the allocation-free decode entry point to hand in the library's own scratch
// array; returns 0 or an fa_status code.
struct WorkspaceSource {
    int (*get)(size_t need, void** ptr, size_t* bytes);
};

// The paged E4M3 decode of attn_fwd_paged_e4m3_decode with its workspace
// taken from `wsrc` (abi.cpp).
int paged_decode_from(const WorkspaceSource* wsrc, const void* q, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                      const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* page_table,
                      int64_t table_stride, int num_phys_pages, int page_size, float k_scale, float v_scale,
                      void* o, int64_t o_sb, int64_t o_sh, int64_t o_ss, float* lse, int B, int Hq, int Hkv, int D,
                      int q_rows, int q_real, int kv_len, float scale, void* stream);

hipError_t launch_attn(const AttnArgs& a, int D, KvSource src, KeyMode mode, bool split,
                       hipStream_t stream);
hipError_t launch_merge(const MergeArgs& m, int D, hipStream_t stream);
// Dense D = 128, FP16 or BF16: the items of a geometry from
// dense_tail_split's tail, each on an 8-wave workgroup whose halves split its
// keys at key_split.
hipError_t launch_dense_halves(const AttnArgs& a, KvSource src, hipStream_t stream);

hipError_t launch_e4m3_bridge(const uint8_t* kc, const uint8_t* vc, const int32_t* table,
                              int64_t table_stride, int num_pages, int B, int Hkv, int D,
                              int kv_len, float k_scale, float v_scale, uint16_t* k_out,
                              uint16_t* v_out, hipStream_t stream);

// E4M3 codes and FP32 scales of the rows of a bfloat16 [B, H, L, 128] view.
hipError_t launch_fp8_rows_quantize(const uint16_t* x, int64_t x_sb, int64_t x_sh, int64_t x_ss, int B, int H, int L,
                                    uint8_t* codes, float* scales, hipStream_t stream);

// K: FP8 round trip per (row, head) with the row gather; V: the gather.
hipError_t launch_prefix_fp8_gather(const uint16_t* k, const uint16_t* v, int B, int N, int H,
                                    const int32_t* index, int rows, uint16_t* k_out, uint16_t* v_out,
                                    hipStream_t stream);

// scores: FP64 [B*H*NB*NB] buffer the score kernel writes and the top-k kernel
// reads; pooled: FP32 [2][B*H*NB][D] means.
hipError_t launch_vsa_select(const uint16_t* q, const uint16_t* k, int B, int H, int L, int D,
                             int topk, int32_t* idx_out, double* scores, float* pooled,
                             hipStream_t stream);

// Pooled FP32 tile means [B*H*NB][D] of x [B,H,L,D] FP16 (64-row tiles).
hipError_t launch_vsa_tile_means(const uint16_t* x, int B, int H, int L, int D, float* out, hipStream_t stream);

// 128-token block lists from a [B,H,T,T] tile mask over tiles of `tile`
// tokens: idx [B,H,NB,NB], counts [B,H,NB], kv_valid [2*NB], quad (nullable).
hipError_t launch_vsa_block_lists(const uint8_t* mask, const int32_t* valid, int B, int H, int T, int tile,
                                  int32_t* idx, int32_t* counts, int32_t* kv_valid, uint8_t* quad,
                                  hipStream_t stream);

}  // namespace fa
