/*
 * fa16attn — FP16 fused scaled-dot-product attention forward for AMD MI355X
 * (gfx950), as a plain C ABI.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "[Kernel] Share SM70 projection, attention and row reduction paths"
 *        — Purpose: the default D128 attention backend of a video diffusion
 *        transformer, with explicit query tiling; FP32 accumulation.
 *   [P3] "[Video] Integrate H3 SM70 execution, metrics and VSA diagnostics"
 *        — Purpose: VSA with top-k = 64 KV blocks per query block and
 *        prefix-dense queries; a native FP16 VSA kernel.
 *   [P4] "[Kernel][SM70] Integrate FP32 v37 prefill and exact E4M3 bridge"
 *        — Purpose and Implementation: FP16 causal prefill, B1/Hq6/Hkv1/D256,
 *        Q 64..8192 in multiples of 64, Q < KV <= 262144, KV a multiple of 32,
 *        real-query causal offsets kept when padded; FP32 prefix/tail state
 *        and a final merge; exact E4M3 paged-to-FP16 conversion with unit and
 *        non-unit scales; bounded per-device workspace.
 *   [P5] "[perf] FastH3 two-Spark: gather packed FP4 inputs before head
 *        projections" — minimax_h3_prefix.cu: BHSD operands with a unit
 *        stride along D and per-tensor batch/head/row strides, an FP32 LSE
 *        [B,H,Lq], the softmax scale 1/sqrt(D) rounded to FP32;
 *        minimax_h3_swiglu_gemm.cu / h3_swiglu_gemm_binding.py: integer
 *        return codes, a raw stream pointer, a caller-owned workspace and a
 *        binding that raises on a nonzero code.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     memory) on the current HIP device, except where stated.
 *   - Tensors are described by element strides; the last (D) stride is 1.
 *     Base pointers of FP16 tensors must be 16-byte aligned and every batch,
 *     head and row stride a multiple of 8 elements.
 *   - The caller owns every buffer, the workspace and the stream. The library
 *     allocates no device memory and never synchronises: a call validates its
 *     arguments on the host, enqueues its kernels on `stream` (a hipStream_t;
 *     NULL = the null stream) and returns. Outputs are valid once the stream
 *     reaches that point. Arguments are checked before any HIP call, so a
 *     rejected call has no side effects.
 *   - Results are bitwise reproducible run to run for the same inputs and
 *     shapes: no atomics take part in any reduction and merges run in a fixed
 *     order.
 *   - Calls on different streams may run concurrently if they share no
 *     output or workspace memory.
 *   - FP16 is IEEE binary16, passed as uint16_t bit patterns where a C type is
 *     needed. E4M3 is the OCP E4M3FN byte format (bias 7, no infinities,
 *     NaN = 0x7F/0xFF, max 448).
 */
#ifndef FA16ATTN_H
#define FA16ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA16ATTN_ABI_VERSION 1

/* Return codes. 0 is success; 1..6 are argument errors detected on the host
 * before any HIP call; FA_ERR_HIP + e reports HIP error e from a launch. */
enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,       /* a size is out of the supported domain */
    FA_ERR_UNSUPPORTED = 3, /* a head dimension, page size or block size not built */
    FA_ERR_ALIGN = 4,       /* D stride != 1, misaligned base, stride not a multiple of 8 */
    FA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than the size query returns */
    FA_ERR_ALIAS = 6,       /* an output overlaps an input or another output */
    FA_ERR_HIP = 1000
};

/* A 4-D [B, H, S, D] tensor view: element strides for batch, head and row;
 * the D stride is 1. */
typedef struct fa_tensor {
    void* data;
    int64_t stride_b;
    int64_t stride_h;
    int64_t stride_s;
} fa_tensor;

/* ABI version of the loaded library (FA16ATTN_ABI_VERSION). */
int fa_abi_version(void);

/* Static description of a return code; never NULL. */
const char* fa_error_string(int code);

/*
 * Dense non-causal attention ([P1] Purpose; [P5] minimax_h3_prefix.cu).
 *   O[b,h,i,:] = sum_j softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:]) V[b,h,j,:]
 * q [B,H,Lq,D], k and v [B,H,Lkv,D], o [B,H,Lq,D]: FP16. QK^T and PV are
 * accumulated in FP32, the softmax runs in FP32 and P is rounded to FP16
 * before the PV product; O is rounded to FP16 (nearest even).
 * lse: optional FP32 [B,H,Lq] contiguous, natural-log sum of exp of the
 * scaled scores; NULL to skip.
 * Domain: B,H >= 1; Lq >= 0 (0 is a no-op); 1 <= Lkv; D in {128, 256};
 * B*H*ceil(Lq/128) < 2^31. o must not overlap q, k, v or lse.
 * At D = 128 (here and for BF16 operands), when the 128-row query tiles fill
 * whole rounds of the chip and then at most half a round more, that rest is
 * computed with each tile's
 * keys in two halves whose FP32 softmax states are merged (the same bounds
 * apply; the rounding order of those rows differs from one pass over the
 * keys). Two kernels run on the stream then.
 */
int attn_fwd_dense(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse, int B, int H,
                   int Lq, int Lkv, int D, float scale, void* stream);

/*
 * attn_fwd_dense on BF16 operands ([P5] the BF16 dense attention of the GB10
 * shape, minimax_h3_prefix.cu): q, k, v and o hold BF16 values; QK^T and PV
 * accumulate in FP32, P is rounded to BF16 before the PV product and O to BF16
 * (nearest even). Arguments, domain and errors as attn_fwd_dense.
 */
int attn_fwd_dense_bf16(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse, int B, int H,
                        int Lq, int Lkv, int D, float scale, void* stream);

/*
 * Dense attention of the prefix with FP8 queries and keys ([P5]
 * query_pool.py: the PREFIX_FP8 round trip of the prefix queries with a
 * per-(row, head) amax / 448 scale; prefix_quant.py: the same for the prefix
 * keys; the example configuration's prefix_precision: fp8).
 * q, k, v: bfloat16 [B,H,Lq,D], [B,H,Lkv,D], [B,H,Lkv,D] views; o: bfloat16
 * [B,H,Lq,D]; lse: optional FP32 [B,H,Lq] contiguous.
 * Every row x of q and of k is quantized as the round trip does:
 * scale = max |x| / 448, code = RNE_e4m3(clamp(x * (scale == 0 ? 0 :
 * 1 / scale), +-448)), in FP32. QK^T runs on the FP8 matrix cores on the codes
 * (exact products, FP32 accumulation) and the FP32 scores are multiplied by
 * the query's and the key's scale: the attention is over the dequantized
 * values decode(code) * scale, without the round trip's bfloat16 storage
 * rounding of them. The softmax runs in FP32, P is rounded to bfloat16, PV
 * accumulates in FP32 on bfloat16 matrix cores and O is rounded to bfloat16.
 * workspace: attn_fwd_prefix_fp8_workspace(...) bytes, 256-byte aligned, not
 * overlapping any operand: the codes of q [B,H,Lq,D] and of k [B,H,Lkv,D]
 * (each padded to 256 bytes), then the scales of q [B,H,Lq] and of k
 * [B,H,Lkv] (FP32, each padded to 256 bytes).
 * Domain: D == 128; B, H >= 1; Lq >= 0 (0 is a no-op); Lkv >= 1.
 */
size_t attn_fwd_prefix_fp8_workspace(int B, int H, int Lq, int Lkv, int D);
int attn_fwd_prefix_fp8(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse, int B, int H, int Lq,
                        int Lkv, int D, float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal prefill against a prefix KV with grouped-query heads ([P4]
 * Implementation). Query row i (0 <= i < q_rows) of query head h sees keys
 * j <= (kv_len - q_real) + i of kv head h / (Hq / Hkv). Rows i >= q_real are
 * padding: they follow the same rule (and so see every key); real rows never
 * depend on padded rows.
 * q [B,Hq,q_rows,D], k and v [B,Hkv,kv_len,D], o [B,Hq,q_rows,D]: FP16;
 * lse optional FP32 [B,Hq,q_rows].
 * The key range of each query tile is split into segments whose FP32 states
 * (running max, running sum, unnormalised O) go to the workspace and are
 * merged in segment order by a second kernel.
 * Domain: B >= 1, Hkv >= 1, Hq % Hkv == 0; D in {128, 256};
 * 64 <= q_rows <= 8192, q_rows % 64 == 0; 1 <= q_real <= q_rows;
 * q_real < kv_len <= 262144; kv_len % 32 == 0.
 * workspace: device memory of at least attn_fwd_prefix_causal_workspace(...)
 * bytes, 256-byte aligned; may be NULL when that size is 0. Its contents are
 * scratch and are overwritten.
 */
size_t attn_fwd_prefix_causal_workspace(int B, int Hq, int Hkv, int D, int q_rows, int kv_len);
int attn_fwd_prefix_causal(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse, int B,
                           int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The causal prefill of attn_fwd_prefix_causal reading K and V from a paged
 * E4M3 cache ([P4] Purpose, Implementation).
 * k_cache, v_cache: uint8 [num_phys_pages, page_size, Hkv, D], E4M3 codes.
 * page_table: int32 [B, table_stride], entry t / page_size of row b is the
 * physical page of logical token t (t < kv_len). Entries must lie in
 * [0, num_phys_pages); an entry outside is clamped into range (no fault, the
 * result for that sequence is then unspecified).
 * K is attended as the FP16 values of the exact conversion,
 * RNE16(RNE32(decode(code) * k_scale)) ([P4] Implementation: the attention
 * runs on the cache converted exactly to FP16 with its scale):
 *  - k_scale a power of two in [2^-15, 2^7]: those are decode * k_scale
 *    exactly, so each code is decoded to FP16 exactly in registers as the MFMA
 *    operand and k_scale joins the softmax scale; V is decoded exactly and
 *    v_scale multiplies the FP32 output;
 *  - any other k_scale, with a workspace of at least
 *    attn_fwd_paged_e4m3_bridged_workspace(..., k_scale) bytes: the exact
 *    bridge (kv_e4m3_paged_to_fp16) writes FP16 K and V into the workspace and
 *    the FP16 causal kernel attends to them (V too is then the bridge's FP16
 *    values), the order the page converts in;
 *  - any other k_scale with a smaller workspace: each workgroup converts every
 *    K code tile once into an FP16 tile in LDS with the same two roundings; V
 *    as in the first case.
 * Domain as attn_fwd_prefix_causal, plus page_size == 32,
 * table_stride >= kv_len / 32, num_phys_pages >= 1, finite scales > 0.
 * workspace: at least attn_fwd_paged_e4m3_workspace(...) bytes (the split-KV
 * states), 256-byte aligned; attn_fwd_paged_e4m3_bridged_workspace returns
 * that size plus 4 * B * Hkv * kv_len * D bytes of FP16 K and V when k_scale
 * is not a power of two in that range, and the same size otherwise.
 */
size_t attn_fwd_paged_e4m3_workspace(int B, int Hq, int Hkv, int D, int q_rows, int kv_len);
size_t attn_fwd_paged_e4m3_bridged_workspace(int B, int Hq, int Hkv, int D, int q_rows, int kv_len,
                                             float k_scale);
int attn_fwd_paged_e4m3(fa_tensor q, const uint8_t* k_cache, const uint8_t* v_cache,
                        const int32_t* page_table, int64_t table_stride, int num_phys_pages,
                        int page_size, float k_scale, float v_scale, fa_tensor o, float* lse, int B,
                        int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len, float scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-phase attention against a paged E4M3 cache ([P4] Purpose: the
 * E4M3 decode kernels; Test plan and results: decode replays at 256000 input
 * tokens): q_rows (1..16) new positions per sequence against kv_len cached
 * tokens, causal with the rule of attn_fwd_prefix_causal (position i sees keys
 * j <= kv_len - q_real + i). The rows of all Hq / Hkv query heads of a kv head
 * are computed together, so each cache byte is read once per kv head; the key
 * range is split into segments whose FP32 states are merged by a second
 * kernel. Arguments, layouts and scales as attn_fwd_paged_e4m3, without the
 * bridged plan: with a k_scale that is not a power of two the K operands take
 * the same converted values, formed once per workgroup in LDS, or, when the
 * packed rows (Hq / Hkv) * q_rows fit one 32-row wave, in registers where
 * the MFMAs use them (such one-wave workgroups run four to a CU, on segments
 * of at least 256 keys).
 * Domain: B >= 1, Hkv >= 1, Hq % Hkv == 0; D in {128, 256};
 * 1 <= q_rows <= 16 with (Hq / Hkv) * q_rows <= 128; 1 <= q_real <= q_rows;
 * q_real < kv_len <= 262144; kv_len % 32 == 0; page_size == 32;
 * table_stride >= kv_len / 32; num_phys_pages >= 1; finite scales > 0.
 * workspace: at least attn_fwd_paged_e4m3_decode_workspace(...) bytes (never
 * 0 for a valid shape), 256-byte aligned.
 */
size_t attn_fwd_paged_e4m3_decode_workspace(int B, int Hq, int Hkv, int D, int q_rows, int kv_len);
int attn_fwd_paged_e4m3_decode(fa_tensor q, const uint8_t* k_cache, const uint8_t* v_cache,
                               const int32_t* page_table, int64_t table_stride, int num_phys_pages,
                               int page_size, float k_scale, float v_scale, fa_tensor o, float* lse, int B,
                               int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len, float scale,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_paged_e4m3_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Arguments, layouts, domain and results as
 * attn_fwd_paged_e4m3_decode, without the workspace: the split-KV partial
 * states go to a device array of the library, FA_NOALLOC_SCRATCH_BYTES per
 * GPU, held from the library's load on that GPU until the process ends. The
 * call allocates nothing (no hipMalloc, hipFree or allocating library call);
 * on its first call on a GPU it looks up the array's device address there.
 * Returns FA_ERR_WORKSPACE, before any HIP call, when the shape's partial
 * states, attn_fwd_paged_e4m3_decode_workspace(...) bytes, exceed
 * FA_NOALLOC_SCRATCH_BYTES (the decode at KV 256000, Hq 6, Hkv 1, D 256,
 * 16 positions takes 24.8 MB). All calls on one GPU share its array: calls
 * that overlap on one GPU (other streams, other host threads) race, and a
 * caller must order them.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_fwd_paged_e4m3_decode_noalloc(fa_tensor q, const uint8_t* k_cache, const uint8_t* v_cache,
                                       const int32_t* page_table, int64_t table_stride, int num_phys_pages,
                                       int page_size, float k_scale, float v_scale, fa_tensor o, float* lse,
                                       int B, int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len,
                                       float scale, void* stream);

/*
 * Exact paged E4M3 -> FP16 conversion ([P4] Implementation, the "exact E4M3
 * bridge"). For every logical token t < kv_len of row b and kv head g:
 *   k_out[b,g,t,:] = RNE16(RNE32(decode(k_cache[page][t % page_size][g][:]) * k_scale))
 * and likewise v_out with v_scale, where page = page_table[b*table_stride +
 * t/page_size]; one FP32 multiply then one FP16 conversion, both rounding to
 * nearest even; FP16 subnormals are kept. A NaN code becomes 0x7E00 with the
 * code's sign. Outputs are contiguous FP16 [B, Hkv, kv_len, D].
 * Domain: B, Hkv >= 1 with 2 * B * Hkv <= 65535; D in {128, 256};
 * page_size == 32; 1 <= kv_len <= 2^26; table_stride >= ceil(kv_len / 32);
 * page entries in [0, num_phys_pages) (clamped otherwise); scales finite.
 */
int kv_e4m3_paged_to_fp16(const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* page_table,
                          int64_t table_stride, int num_phys_pages, int page_size, int B, int Hkv,
                          int D, int kv_len, float k_scale, float v_scale, uint16_t* k_out,
                          uint16_t* v_out, void* stream);

/*
 * FP8 round trip of prefix keys with the valid-row gather ([P5]
 * prefix_quant.py, quantize_gather_prefix_kv; key_quant.py applies the same
 * key round trip in its prefix preparation). k, v: bfloat16 [B, N, H, D] contiguous; index: int32 [rows], the
 * source token of each output row (clamped into [0, N)). For every (b, r, h),
 * with x the FP32 values of k[b, index[r], h, :]:
 *   scale = max |x| / 448, inv = (scale == 0 ? 0 : 1 / scale),
 *   k_out[b, r, h, :] = RNE_bf16(decode(RNE_e4m3(clamp(x * inv, -448, 448))) * scale),
 * every step rounding once in FP32 (OCP E4M3FN); v_out[b, r, h, :] =
 * v[b, index[r], h, :]. Outputs are bfloat16 [B, rows, H, D] contiguous and
 * must not overlap the inputs or each other.
 * Domain: D == 128; B, N, H >= 1; rows >= 0 (0 is a no-op).
 */
int kv_prefix_fp8_gather(const uint16_t* k, const uint16_t* v, int B, int N, int H, int D,
                         const int32_t* index, int rows, uint16_t* k_out, uint16_t* v_out, void* stream);

/*
 * The top-k of a VSA keep ratio ([P5] the VSA_sparsity setting, 0.8 with
 * 64-token tiles): with NB = ceil(L / block) blocks, keep
 * max(1, ceil((1 - sparsity) * NB)) of them (116 of 576 at 0.8), a product
 * within 1e-9 * NB of an integer taken as that integer. Host only.
 * Returns that count, or -FA_ERR_SHAPE for block < 1, L < 1 or a sparsity
 * outside [0, 1).
 */
int vsa_topk_for_sparsity(int L, int block, double sparsity);

/*
 * VSA block selection ([P3] Purpose; [P5] key_quant.py and query_pool.py for
 * the tile means). With NB = ceil(L / block) (the last block may hold fewer
 * than block rows when L is not a multiple of block):
 *   qbar[b,h,t,:] = RNE32(sum of the block's FP16 query rows / their count),
 *   kbar likewise from k,
 *   s[b,h,i,j]    = sum over d ascending of qbar[b,h,i,d] * kbar[b,h,j,d] in FP64,
 * and idx_out[b,h,i,:] = the topk block indices j with the largest s[b,h,i,j]
 * (equal scores ranked by the lower j), written in ascending order.
 * q, k: FP16 [B,H,L,D] contiguous. idx_out: int32 [B,H,NB,topk] contiguous.
 * score_out: optional FP64 [B,H,NB,NB] (NULL to skip).
 * Domain: D == 128; block == 64; L >= 1; 1 <= NB <= 1024; 1 <= topk <= NB.
 * workspace: at least vsa_block_select_workspace(...) bytes (the FP32 pooled
 * means, then the FP64 block scores when score_out is NULL), 256-byte aligned.
 */
size_t vsa_block_select_workspace(int B, int H, int L, int D, int block);
int vsa_block_select(const uint16_t* q, const uint16_t* k, int B, int H, int L, int D, int block,
                     int topk, int32_t* idx_out, double* score_out, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Pooled tile means ([P5] kv_pool.py: the FP32 value tile means, the tile's
 * valid-row sum divided by its valid count with one rounding; the same means
 * as vsa_block_select's): out[b,h,t,:] = RNE32(sum of the tile's rows / their
 * count) over tiles of `block` rows, the last holding L - (NB - 1) * block.
 * Used for the pooled V of the VSA coarse branch.
 * x: FP16 [B,H,L,D] contiguous; out: FP32 [B,H,NB,D] contiguous, NB =
 * ceil(L / block). Domain: D == 128; block == 64; B, H, L >= 1.
 */
int vsa_tile_means(const uint16_t* x, int B, int H, int L, int D, int block, float* out, void* stream);

/*
 * VSA 128-token block lists from a tile mask ([P5] block_lists.py,
 * tile_mask_to_fp4_blocks). mask: uint8 [B,H,T,T] contiguous, nonzero when
 * query tile i attends to key tile j; tiles hold `tile` = 64 * HT tokens
 * (64 or 128); valid: int32 [T], the valid tokens of each tile. The sequence
 * splits into 64-token halves (T * HT) and blocks of two halves,
 * NB = ceil(T * HT / 2). With va = clamp(valid[a / HT] - (a % HT) * 64, 0, 64)
 * for half a (0 past the sequence) and m(q, k) = mask[q / HT][k / HT] (a
 * padded odd last query half sees key half 0 only), query block r (halves
 * 2r, 2r+1) and key block c (halves a = 2c, e = 2c+1) have the quadrant mask
 *   [m(2r,a) & va>0] + 2 [m(2r,e) & ve>0] + 4 [m(2r+1,a) & va>0] + 8 [m(2r+1,e) & ve>0].
 * Outputs: indices int32 [B,H,NB,NB]: per (b, h, r) the key blocks with a
 * nonzero mask in descending order, then zeros; counts int32 [B,H,NB]: their
 * number; kv_valid int32 [2 * NB]: va per half; quadrants uint8 [B,H,NB,NB]
 * (optional, 64-token tiles only): the masks in list order, then zeros.
 * Domain: tile in {64, 128}; B, H, T >= 1; T * tile / 64 <= 1024.
 */
int vsa_tile_mask_to_block_lists(const uint8_t* mask, const int32_t* valid, int B, int H, int T, int tile,
                                 int32_t* indices, int32_t* counts, int32_t* kv_valid, uint8_t* quadrants,
                                 void* stream);

/*
 * VSA block-sparse attention ([P3] Purpose). Query block bq = i / block of
 * head h attends to the keys of the blocks idx[b,h,bq,0..topk) when
 * bq >= dense_prefix_qblocks, and to every key when bq < dense_prefix_qblocks.
 * With NB = ceil(L / block), the last block may be partial; keys past L are
 * never attended to and rows past L are not written.
 * q, k, v, o: FP16 [B,H,L,D] views; idx: int32 [B,H,NB,topk] contiguous,
 * entries distinct and in [0, NB) (out-of-range entries are clamped);
 * lse: optional FP32 [B,H,L].
 * Domain: D == 128; block == 64; L >= 1; 1 <= topk <= NB;
 * 0 <= dense_prefix_qblocks <= NB.
 * workspace: at least vsa_block_sparse_attn_workspace(...) bytes, 256-byte
 * aligned, not overlapping any operand (may be NULL when that size is 0).
 * The dense-prefix query blocks are split into key segments whose FP32
 * partial states (max, sum, unnormalised output) go to the workspace and are
 * merged in segment order by a second kernel on the same stream.
 */
size_t vsa_block_sparse_attn_workspace(int B, int H, int L, int D, int block, int topk,
                                       int dense_prefix_qblocks);
int vsa_block_sparse_attn(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, const int32_t* idx,
                          float* lse, int B, int H, int L, int D, int block, int topk,
                          int dense_prefix_qblocks, float scale, void* workspace,
                          size_t workspace_bytes, void* stream);


#ifdef __cplusplus
}
#endif

#endif /* FA16ATTN_H */
