// Fused FP16 attention forward for gfx950 (MI355X).
//
// One kernel template serves every variant on the hot path:
//   - dense non-causal attention ("[Kernel] Share SM70 projection, attention
//     and row reduction paths", Purpose: the default D128 attention),
//   - causal prefill against a prefix KV with grouped-query heads, split over
//     the key range into FP32 partial states that a second kernel merges
//     ("[Kernel][SM70] Integrate FP32 v37 prefill and exact E4M3 bridge",
//     Implementation),
//   - the same prefill reading K/V from a paged E4M3 cache, decoded to FP16
//     in registers on the way into LDS (same page, Purpose),
//   - block-sparse attention over per-query-block KV block lists with dense
//     prefix query blocks ("[Video] Integrate H3 SM70 execution, metrics and
//     VSA diagnostics", Purpose).
//
// Work decomposition (MI355X-first, not the pages' SM70/SM121 designs):
//   - A workgroup owns WAVES x 32 query rows of one (batch, head) and streams
//     64-key tiles of K and V through LDS, double-buffered: tile t+1 is loaded
//     from HBM/L2 into registers while tile t is consumed from LDS.
//   - Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_f16: the MFMA result puts one query per lane
//     (lane % 32) and 16 keys per lane, so the row max and row sum need only
//     in-lane work plus one exchange between the two lane halves.
//   - The output is also kept transposed, O^T = V^T P^T, so the per-query
//     rescale factor is a per-lane scalar. P never leaves registers: the
//     score accumulator registers are exactly the B operand of the PV MFMA
//     once the V^T tile in LDS stores each 16-key group in the matching
//     permuted key order.
//   - The softmax runs in base 2 with the scale folded into one FP32 factor
//     c = scale * log2(e), so each probability is one FMA and one v_exp_f32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// LDS layout of one stage (K tile + V^T tile), in FP16 elements.
//   K   [64 keys][D + 8]: rows padded by 16 bytes so the 32 rows one MFMA
//       operand read touches spread over all banks.
//   V^T [D][64 keys]: 16-byte chunks of each row XOR-swizzled by
//       (d + d/8) mod 8, which keeps both the transposing writes (8 rows d
//       apart) and the operand reads (32 consecutive rows) free of bank
//       conflicts. Within each 16-key group the keys are stored in the order
//       0-3, 8-11, 4-7, 12-15 (see vt_pos).
template <int D>
struct Lds {
    static constexpr int kKStride = D + 8;
    static constexpr int kKElems = kTileN * kKStride;
    static constexpr int kVtElems = D * kTileN;
    static constexpr int kStage = kKElems + kVtElems;
    static constexpr int kElems = 2 * kStage;
};

__device__ __forceinline__ int vt_swz(int d) { return (d + (d >> 3)) & 7; }

// Element offset of (row d, 8-key chunk c) in the swizzled V^T tile.
__device__ __forceinline__ int vt_chunk(int d, int c) { return d * kTileN + ((c ^ vt_swz(d)) << 3); }

__device__ __forceinline__ float wave_half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float wave_half_sum(float x) { return x + __shfl_xor(x, 32); }

// Pack the low (sel = 0) or high (sel = 1) FP16 halves of two dwords.
__device__ __forceinline__ uint32_t pack_halves(uint32_t lo_src, uint32_t hi_src, int sel)
{
    return __builtin_amdgcn_perm(hi_src, lo_src, sel ? 0x07060302u : 0x05040100u);
}

// Four E4M3 bytes -> four FP16 values, exactly (scale 1: every E4M3 value is
// an FP16 value, so no rounding happens).
__device__ __forceinline__ u2 e4m3x4_to_f16(uint32_t w)
{
    h2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    h2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    u2 r;
    r.x = __builtin_bit_cast(uint32_t, lo);
    r.y = __builtin_bit_cast(uint32_t, hi);
    return r;
}

// ---------------------------------------------------------------------------
// Global -> register -> LDS staging of one 64-key tile.
// ---------------------------------------------------------------------------
template <int D, int SRC, int NT>
struct Stager;

// FP16 K/V rows.
template <int D, int NT>
struct Stager<D, KV_FP16, NT> {
    static constexpr int kKChunks = kTileN * D / 8 / NT;   // 16-byte K chunks per thread
    static constexpr int kVTasks = (kTileN / 4) * (D / 8) / NT;  // 4 keys x 8 d per task
    u4 kr[kKChunks];
    u4 vr[kVTasks][4];

    __device__ __forceinline__ void load(const AttnArgs& a, const _Float16* kbase,
                                         const _Float16* vbase, int key0, int key_last, int tid)
    {
#pragma unroll
        for (int i = 0; i < kKChunks; ++i) {
            int c = tid + NT * i;
            int row = c / (D / 8), col = c % (D / 8);
            int key = min(key0 + row, key_last);
            kr[i] = *(const u4*)(kbase + (int64_t)key * a.k_ss + col * 8);
        }
#pragma unroll
        for (int i = 0; i < kVTasks; ++i) {
            int t = tid + NT * i;
            int grp = t / (D / 8), col = t % (D / 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int key = min(key0 + 4 * grp + j, key_last);
                vr[i][j] = *(const u4*)(vbase + (int64_t)key * a.v_ss + col * 8);
            }
        }
    }

    __device__ __forceinline__ void store(_Float16* ks, _Float16* vt, int tid) const
    {
#pragma unroll
        for (int i = 0; i < kKChunks; ++i) {
            int c = tid + NT * i;
            int row = c / (D / 8), col = c % (D / 8);
            *(u4*)(ks + row * Lds<D>::kKStride + col * 8) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < kVTasks; ++i) {
            int t = tid + NT * i;
            int grp = t / (D / 8), col = t % (D / 8);
            store_vt(vt, grp, col, vr[i][0], vr[i][1], vr[i][2], vr[i][3]);
        }
    }

    // Rows 4*grp..4*grp+3 (keys) x columns 8*col..8*col+7 (d) -> V^T.
    static __device__ __forceinline__ void store_vt(_Float16* vt, int grp, int col, u4 r0, u4 r1,
                                                    u4 r2, u4 r3)
    {
        // key group of 4 -> position inside its 16-key group: 0, 8, 4, 12
        int chunk = 2 * (grp >> 2) + (grp & 1);
        int within = (grp & 2) ? 4 : 0;
        uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
        uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
        uint32_t w2[4] = {r2.x, r2.y, r2.z, r2.w};
        uint32_t w3[4] = {r3.x, r3.y, r3.z, r3.w};
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            int d = col * 8 + dd;
            u2 val;
            val.x = pack_halves(w0[dd >> 1], w1[dd >> 1], dd & 1);
            val.y = pack_halves(w2[dd >> 1], w3[dd >> 1], dd & 1);
            *(u2*)(vt + vt_chunk(d, chunk) + within) = val;
        }
    }
};

// Paged E4M3 K/V rows: raw bytes are staged in registers and decoded to FP16
// when written to LDS.
template <int D, int NT>
struct Stager<D, KV_E4M3_PAGED, NT> {
    static constexpr int kKChunks = kTileN * D / 16 / NT;  // 16-byte (16-code) K chunks
    static constexpr int kVTasks = (kTileN / 4) * (D / 8) / NT;
    u4 kr[kKChunks];
    u2 vr[kVTasks][4];

    static __device__ __forceinline__ const uint8_t* row_ptr(const AttnArgs& a, const uint8_t* cache,
                                                             const int32_t* table, int g, int key)
    {
        int page = table[key >> a.page_shift];
        page = min(max(page, 0), a.num_pages - 1);
        int slot = key & ((1 << a.page_shift) - 1);
        return cache + (((int64_t)page << a.page_shift) + slot) * ((int64_t)a.Hkv * D) + (int64_t)g * D;
    }

    __device__ __forceinline__ void load(const AttnArgs& a, const int32_t* table, int g, int key0,
                                         int key_last, int tid)
    {
#pragma unroll
        for (int i = 0; i < kKChunks; ++i) {
            int c = tid + NT * i;
            int row = c / (D / 16), col = c % (D / 16);
            int key = min(key0 + row, key_last);
            kr[i] = *(const u4*)(row_ptr(a, a.kc, table, g, key) + col * 16);
        }
#pragma unroll
        for (int i = 0; i < kVTasks; ++i) {
            int t = tid + NT * i;
            int grp = t / (D / 8), col = t % (D / 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int key = min(key0 + 4 * grp + j, key_last);
                vr[i][j] = *(const u2*)(row_ptr(a, a.vc, table, g, key) + col * 8);
            }
        }
    }

    __device__ __forceinline__ void store(_Float16* ks, _Float16* vt, int tid) const
    {
#pragma unroll
        for (int i = 0; i < kKChunks; ++i) {
            int c = tid + NT * i;
            int row = c / (D / 16), col = c % (D / 16);
            u2 a0 = e4m3x4_to_f16(kr[i].x), a1 = e4m3x4_to_f16(kr[i].y);
            u2 a2 = e4m3x4_to_f16(kr[i].z), a3 = e4m3x4_to_f16(kr[i].w);
            u4 lo = {a0.x, a0.y, a1.x, a1.y};
            u4 hi = {a2.x, a2.y, a3.x, a3.y};
            _Float16* dst = ks + row * Lds<D>::kKStride + col * 16;
            *(u4*)dst = lo;
            *(u4*)(dst + 8) = hi;
        }
#pragma unroll
        for (int i = 0; i < kVTasks; ++i) {
            int t = tid + NT * i;
            int grp = t / (D / 8), col = t % (D / 8);
            u4 rows[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u2 x = e4m3x4_to_f16(vr[i][j].x), y = e4m3x4_to_f16(vr[i][j].y);
                rows[j] = u4{x.x, x.y, y.x, y.y};
            }
            Stager<D, KV_FP16, NT>::store_vt(vt, grp, col, rows[0], rows[1], rows[2], rows[3]);
        }
    }
};

// ---------------------------------------------------------------------------
// The attention kernel.
// ---------------------------------------------------------------------------
template <int D, int WAVES, int SRC, int MODE, bool SPLIT>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_kernel(const AttnArgs a)
{
    constexpr int M = WAVES * kRowsPerWave;
    constexpr int KK = D / 16;  // MFMA k-steps over D for S
    constexpr int DB = D / 32;  // 32-wide d blocks of O^T
    __shared__ __attribute__((aligned(16))) _Float16 lds[Lds<D>::kElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;

    // ---- work item -> (b, h, query tile, key range) ----------------------
    int item = blockIdx.x;
    if (a.per_xcd > 0) item = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
    if (item >= a.n_items) return;

    int b, h, qt, seg = 0;
    if (MODE == KEYS_CAUSAL) {
        int j = item % a.group;
        int r = item / a.group;
        qt = r % a.n_qt;
        r /= a.n_qt;
        seg = r % a.nseg;
        r /= a.nseg;
        int g = r % a.Hkv;
        b = r / a.Hkv;
        h = g * a.group + j;
    } else if (MODE == KEYS_BLOCKS) {
        // dense-prefix query blocks (the longest items) come first
        const int n_dense = a.B * a.Hq * a.dense_prefix;
        int bh;
        if (item < n_dense) {
            bh = item / a.dense_prefix;
            qt = item % a.dense_prefix;
        } else {
            int r = item - n_dense;
            int sparse = a.nqb - a.dense_prefix;
            bh = r / sparse;
            qt = a.dense_prefix + r % sparse;
        }
        h = bh % a.Hq;
        b = bh / a.Hq;
    } else {
        qt = item % a.n_qt;
        int r = item / a.n_qt;
        h = r % a.Hq;
        b = r / a.Hq;
    }
    const int g = h / a.group;
    const int q0 = qt * M;

    int tile_begin = 0, n_tiles;
    const int32_t* blist = nullptr;
    int key_end = a.Lkv;
    if (MODE == KEYS_CAUSAL) {
        int last_row = min(q0 + M, a.Lq) - 1;
        key_end = (int)min((int64_t)a.Lkv, a.offset + last_row + 1);
        int nt = (key_end + kTileN - 1) / kTileN;
        tile_begin = seg * a.seg_tiles;
        n_tiles = min(nt, tile_begin + a.seg_tiles) - tile_begin;
        if (n_tiles <= 0) return;  // the merge skips segments past the key range
    } else if (MODE == KEYS_BLOCKS) {
        int qb = qt;  // M == 64: one query block per workgroup
        if (qb < a.dense_prefix) {
            n_tiles = a.Lkv / kTileN;
        } else {
            n_tiles = a.topk;
            blist = a.idx + (((int64_t)b * a.Hq + h) * a.nqb + qb) * a.topk;
        }
    } else {
        n_tiles = (a.Lkv + kTileN - 1) / kTileN;
    }
    const int key_last = key_end - 1;
    const int nblk = a.Lkv / kTileN;

    auto tile_key0 = [&](int it) -> int {
        if (MODE == KEYS_BLOCKS && blist) {
            int blk = blist[it];
            blk = min(max(blk, 0), nblk - 1);
            return blk * kTileN;
        }
        return (tile_begin + it) * kTileN;
    };

    // ---- pointers ------------------------------------------------------------
    const _Float16* kbase = nullptr;
    const _Float16* vbase = nullptr;
    const int32_t* table = nullptr;
    if (SRC == KV_FP16) {
        kbase = a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh;
        vbase = a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh;
    } else {
        table = a.table + (int64_t)b * a.table_stride;
    }

    // ---- Q fragment in registers: lane holds Q[row][16kk + 8hlf .. +7] ------
    const int my_row = q0 + wave * kRowsPerWave + l32;
    h8 qf[KK];
    {
        int row = min(my_row, a.Lq - 1);
        const _Float16* qp = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh + (int64_t)row * a.q_ss;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const h8*)(qp + 16 * kk + 8 * hlf);
    }

    f16x oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    float m_run = -INFINITY;  // running max of scores * c (log2 units)
    float l_run = 0.f;        // this lane half's share of the running sum

    Stager<D, SRC, WAVES * 64> st;
    auto stage_load = [&](int it) {
        int key0 = tile_key0(it);
        if constexpr (SRC == KV_FP16)
            st.load(a, kbase, vbase, key0, key_last, tid);
        else
            st.load(a, table, g, key0, key_last, tid);
    };

    stage_load(0);
    st.store(lds, lds + Lds<D>::kKElems, tid);
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int key0 = tile_key0(it);
        if (it + 1 < n_tiles) stage_load(it + 1);

        const _Float16* ks = lds + (it & 1) * Lds<D>::kStage;
        const _Float16* vt = ks + Lds<D>::kKElems;

        // ---- S^T = K Q^T for 64 keys x 32 queries (two 32x32 blocks) -------
        f16x s0, s1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s0[r] = 0.f;
            s1[r] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            h8 k0 = *(const h8*)(ks + l32 * Lds<D>::kKStride + 16 * kk + 8 * hlf);
            h8 k1 = *(const h8*)(ks + (32 + l32) * Lds<D>::kKStride + 16 * kk + 8 * hlf);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, qf[kk], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, qf[kk], s1, 0, 0, 0);
        }

        // ---- masks: register r of block kb holds key kb*32 + 8(r/4) + 4hlf + r%4
        bool need_mask;
        if (MODE == KEYS_CAUSAL)
            need_mask = (int64_t)key0 + kTileN > a.offset + q0 + 1 || key0 + kTileN > key_end;
        else if (MODE == KEYS_DENSE)
            need_mask = key0 + kTileN > key_end;
        else
            need_mask = false;
        if (need_mask) {
            int64_t lim = (MODE == KEYS_CAUSAL) ? min((int64_t)key_last, a.offset + my_row)
                                                : (int64_t)key_last;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int kr = key0 + 8 * (r >> 2) + 4 * hlf + (r & 3);
                if (kr > lim) s0[r] = -INFINITY;
                if (kr + 32 > lim) s1[r] = -INFINITY;
            }
        }

        // ---- online softmax (base 2) --------------------------------------
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
        mx = wave_half_max(mx);
        const float m_new = fmaxf(m_run, mx * a.c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;

        float psum = 0.f;
        h8 pk[4];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p0 = __builtin_amdgcn_exp2f(fmaf(s0[r], a.c, -m_use));
            float p1 = __builtin_amdgcn_exp2f(fmaf(s1[r], a.c, -m_use));
            psum += p0 + p1;
            pk[r >> 3][r & 7] = (_Float16)p0;
            pk[2 + (r >> 3)][r & 7] = (_Float16)p1;
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;

        // ---- O^T += V^T P^T ---------------------------------------------------
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = db * 32 + l32;
#pragma unroll
            for (int kstep = 0; kstep < 4; ++kstep) {
                h8 vf = *(const h8*)(vt + vt_chunk(d, 2 * kstep + hlf));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pk[kstep], oacc[db], 0, 0, 0);
            }
        }

        if (it + 1 < n_tiles) {
            _Float16* nks = lds + ((it + 1) & 1) * Lds<D>::kStage;
            st.store(nks, nks + Lds<D>::kKElems, tid);
        }
        __syncthreads();
    }

    // ---- epilogue ------------------------------------------------------------
    const float l_tot = wave_half_sum(l_run);
    if (my_row >= a.Lq) return;
    const int64_t bh = (int64_t)b * a.Hq + h;
    if (SPLIT) {
        float* op = a.o_part + (((int64_t)seg * a.B * a.Hq + bh) * a.Lq + my_row) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                int d = db * 32 + 8 * g4 + 4 * hlf;
                float4 v4 = {oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2],
                             oacc[db][4 * g4 + 3]};
                *(float4*)(op + d) = v4;
            }
        if (hlf == 0) {
            float2 ml = {m_run, l_tot};
            *(float2*)(a.ml_part + (((int64_t)seg * a.B * a.Hq + bh) * a.Lq + my_row) * 2) = ml;
        }
    } else {
        const float inv = a.oscale / l_tot;
        _Float16* op = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)my_row * a.o_ss;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                int d = db * 32 + 8 * g4 + 4 * hlf;
                h4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (_Float16)(oacc[db][4 * g4 + e] * inv);
                *(h4*)(op + d) = v4;
            }
        if (a.lse && hlf == 0)
            a.lse[bh * a.Lq + my_row] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
    }
}

// ---------------------------------------------------------------------------
// Merge of split-KV partial states, in segment order:
//   M = max_s m_s, w_s = 2^(m_s - M), O = sum_s w_s O_s / sum_s w_s l_s.
// One wave per query row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const MergeArgs m)
{
    const int lane = threadIdx.x & 63;
    const int64_t row_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t total = (int64_t)m.B * m.Hq * m.Lq;
    if (row_id >= total) return;
    const int i = (int)(row_id % m.Lq);
    const int64_t bh = row_id / m.Lq;
    const int b = (int)(bh / m.Hq), h = (int)(bh % m.Hq);

    // segments that exist for this row's query tile
    const int qt = i / m.rows_per_tile;
    const int last_row = min((qt + 1) * m.rows_per_tile, m.Lq) - 1;
    const int key_end = (int)min((int64_t)m.Lkv, m.offset + last_row + 1);
    const int nt = (key_end + kTileN - 1) / kTileN;
    const int nseg = min(m.nseg, (nt + m.seg_tiles - 1) / m.seg_tiles);

    const int64_t seg_stride = (int64_t)m.B * m.Hq * m.Lq;
    float mmax = -INFINITY;
    for (int s = 0; s < nseg; ++s) mmax = fmaxf(mmax, m.ml_part[(s * seg_stride + row_id) * 2]);
    constexpr int PER = D / 64;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float den = 0.f;
    for (int s = 0; s < nseg; ++s) {
        const float ms = m.ml_part[(s * seg_stride + row_id) * 2];
        const float ls = m.ml_part[(s * seg_stride + row_id) * 2 + 1];
        if (ls == 0.f) continue;  // no visible key in this segment
        const float w = __builtin_amdgcn_exp2f(ms - mmax);
        den += w * ls;
        const float* op = m.o_part + (s * seg_stride + row_id) * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += w * op[e];
    }
    const float inv = m.oscale / den;
    _Float16* out = m.o + (int64_t)b * m.o_sb + (int64_t)h * m.o_sh + (int64_t)i * m.o_ss + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = (_Float16)(acc[e] * inv);
    if (m.lse && lane == 0) m.lse[row_id] = (mmax + __log2f(den)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <int D, int WAVES, int SRC, int MODE, bool SPLIT>
static hipError_t launch_one(const AttnArgs& a, hipStream_t stream)
{
    int grid = a.per_xcd > 0 ? a.per_xcd * 8 : a.n_items;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((attn_fwd_kernel<D, WAVES, SRC, MODE, SPLIT>), dim3(grid), dim3(WAVES * 64), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, KvSource src, KeyMode mode, bool split,
                           hipStream_t stream)
{
    if (mode == KEYS_DENSE) return launch_one<D, 4, KV_FP16, KEYS_DENSE, false>(a, stream);
    if (mode == KEYS_BLOCKS) return hipErrorInvalidValue;
    if (src == KV_FP16)
        return split ? launch_one<D, 4, KV_FP16, KEYS_CAUSAL, true>(a, stream)
                     : launch_one<D, 4, KV_FP16, KEYS_CAUSAL, false>(a, stream);
    return split ? launch_one<D, 4, KV_E4M3_PAGED, KEYS_CAUSAL, true>(a, stream)
                 : launch_one<D, 4, KV_E4M3_PAGED, KEYS_CAUSAL, false>(a, stream);
}

hipError_t launch_attn(const AttnArgs& a, int D, KvSource src, KeyMode mode, bool split,
                       hipStream_t stream)
{
    if (mode == KEYS_BLOCKS) {
        if (D != 128 || src != KV_FP16 || split) return hipErrorInvalidValue;
        return launch_one<128, 2, KV_FP16, KEYS_BLOCKS, false>(a, stream);
    }
    if (D == 128) return launch_d<128>(a, src, mode, split, stream);
    if (D == 256) return launch_d<256>(a, src, mode, split, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeArgs& m, int D, hipStream_t stream)
{
    int64_t rows = (int64_t)m.B * m.Hq * m.Lq;
    int grid = (int)((rows + 3) / 4);
    if (grid <= 0) return hipSuccess;
    if (D == 128)
        hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(grid), dim3(256), 0, stream, m);
    else if (D == 256)
        hipLaunchKernelGGL(attn_merge_kernel<256>, dim3(grid), dim3(256), 0, stream, m);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace fa
