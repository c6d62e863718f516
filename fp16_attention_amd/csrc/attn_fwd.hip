// Fused FP16 attention forward for gfx950 (MI355X).
//
// One kernel template serves every variant on the hot path:
//   - dense non-causal attention ("[Kernel] Share SM70 projection, attention
//     and row reduction paths", Purpose: the default D128 attention),
//   - causal prefill against a prefix KV with grouped-query heads, split over
//     the key range into FP32 partial states that a second kernel merges
//     ("[Kernel][SM70] Integrate FP32 v37 prefill and exact E4M3 bridge",
//     Implementation),
//   - the same prefill reading K/V from a paged E4M3 cache: the codes stream
//     through LDS and are decoded exactly to FP16 in registers as the MFMA
//     operands, or, for a k_scale that is not a power of two, K is converted
//     once per workgroup into FP16 tiles in LDS (same page, Purpose),
//   - block-sparse attention over per-query-block KV block lists with dense
//     prefix query blocks ("[Video] Integrate H3 SM70 execution, metrics and
//     VSA diagnostics", Purpose).
//
// Work decomposition (MI355X-first, not the pages' SM70/SM121 designs):
//   - A workgroup owns WAVES x 32 query rows of one (batch, head); every wave
//     keeps its 32 query rows in registers as the MFMA B operand and streams
//     tiles of K and V through LDS (64 keys for dense D = 128, else 32).
//   - LDS holds a ring of R K slots and R V slots. FP16 tiles move from
//     HBM/L2 into LDS with buffer_load ... lds (no register staging; rows past
//     the end of the key range read as zero through the buffer range check),
//     R - 1 iterations ahead of their use (at D = 256 a group's loads are
//     spread over the MFMA steps of the iteration that issues them). Paged
//     E4M3 code tiles (one 32-token page each) move into the ring the same
//     way, half the bytes of FP16 tiles; each wave decodes the codes of every
//     operand it reads exactly to FP16 in registers, right before the MFMA
//     that consumes it (scaled K: from the workgroup's converted FP16 tile). K and V are stored row-major with 16-byte chunks
//     XOR-swizzled by the row, which keeps the K operand reads and the
//     transposing V reads (16-bit or 8-bit) free of bank conflicts.
//   - Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_f16: each lane owns one query (lane % 32) and 16
//     keys per 32-key block, so the row max and row sum are in-lane work plus
//     one exchange between the two lane halves.
//   - The output is kept transposed too, O^T = V^T P^T. The V^T operand comes
//     straight from the row-major V tile with ds_read_b64_tr_b16, and P never
//     leaves registers: the score accumulators are the B operand once each
//     16-key group is read in the matching key order.
//   - The scores of tile t+1 are issued on the matrix cores before the softmax
//     of tile t runs on the VALU, so the two overlap inside a wave.
//   - The softmax runs in base 2 with c = scale * log2(e) folded into one FMA.
//     The running maximum is only raised when a score exceeds it by more than
//     2^8, so the O accumulators are rescaled a handful of times per row
//     instead of every tile; P then stays below 2^8, exact in FP16 range, and
//     the normalisation divides by the sum of the same FP16 probabilities that
//     multiply V.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa_internal.h"

namespace fa {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s4 lds_s4_t;
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i_t;

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// D(32x32, FP32) += A(32x16) B(16x32) on FP16 or BF16 operands, both carried
// as eight 16-bit values per lane.
template <bool BF>
__device__ __forceinline__ f16x mma(h8 a, h8 b, f16x c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0,
                                                       0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// FP32 -> the 16-bit output format, rounding to nearest even.
template <bool BF>
__device__ __forceinline__ _Float16 to_out(float x)
{
    if constexpr (BF)
        return __builtin_bit_cast(_Float16, (__bf16)x);
    else
        return (_Float16)x;
}

// Word 3 of a raw buffer resource (32-bit data, no swizzle) on the gfx9 family.
constexpr uint32_t kRsrcWord3 = 0x00020000u;
// The running maximum (log2 units) is raised only when exceeded by this much.
constexpr float kRescaleSlack = 8.0f;

#ifndef FA_NO_SCHED_HINTS
#define SCHED_GROUP(mask, n, id) __builtin_amdgcn_sched_group_barrier(mask, n, id)
#else
#define SCHED_GROUP(mask, n, id) ((void)0)
#endif

// s_waitcnt immediates (gfx9 encoding): vmcnt in [3:0] and [15:14], expcnt in
// [6:4], lgkmcnt in [11:8].
constexpr int kWaitVm0 = 0x0F70;
// vmcnt(0) and lgkmcnt(0)
constexpr int kWaitAll = 0x0070;

// Workgroup barrier for the K/V ring: the caller's s_waitcnt (vmcnt(n) with
// lgkmcnt(0)) makes this wave's loads into LDS older than the n most recent
// ones, and its LDS accesses, complete; s_barrier then orders them before
// every wave's later LDS reads. A C++ fence here would wait for all loads
// into LDS (vmcnt(0)), so the compiler is only kept from moving memory
// accesses across the barrier.
template <int WAITCNT>
__device__ __forceinline__ void ring_barrier()
{
    __builtin_amdgcn_s_waitcnt(WAITCNT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// LDS tile layout: 64 rows (keys) of D FP16, row-major, 2*D bytes per row;
// 16-byte chunk c of row r sits at position c ^ swz(r % 16).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk)
{
    return row * (2 * D) + ((chunk ^ swz(row & 15)) << 4);
}

// Lanes l and l ^ 32 hold the same query row. v_permlane32_swap trades the
// upper half of one register with the lower half of another; applied to two
// copies of x it leaves x of lanes 0-31 in the first and x of lanes 32-63 in
// the second, in every lane, without the LDS round trip of a bpermute. The
// elements are copied out before the bit casts: a bit cast of a vector
// element expression reads element 0.
__device__ __forceinline__ float2 half_pair(float x)
{
    const unsigned a = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    const unsigned lo = r[0], hi = r[1];
    return {__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi)};
}
// The same for lanes l and l ^ 16 through v_permlane16_swap, which trades
// the odd 16-lane rows of one register with the even rows of another.
__device__ __forceinline__ float2 row_pair(float x)
{
    const unsigned a = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    const unsigned lo = r[0], hi = r[1];
    return {__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi)};
}
__device__ __forceinline__ float wave_half_max(float x) { const float2 p = half_pair(x); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float wave_half_sum(float x) { const float2 p = half_pair(x); return p.x + p.y; }

// Three-input maximum; the compiler emits one v_max3_f32 per call. It must
// stay compiled code (no inline asm): the scores it reads come straight from
// MFMA accumulators, and only compiled instructions get the wait states that
// a VALU read of a fresh MFMA result needs (there is no hardware interlock
// for it).
__device__ __forceinline__ float vmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Four E4M3 bytes -> four FP16 values, exactly (scale 1: every E4M3 value is
// an FP16 value, so no rounding happens). The packed pairs are only ever
// moved as whole dwords: extracting one half of this builtin's result with
// .x / .y was compiled into a copy of the low half into both halves. The
// conversion's scale operand only applies its power-of-two part, so any other
// scale is applied separately (convert8 below).
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
// FP16 tiles: buffer_load_dwordx4 ... lds. Wave w's j-th load writes the
// 1 KB block (w + WAVES * j) of the tile; lane i of it writes bytes
// [16 i, 16 i + 16) of that block, so each lane loads the global chunk that
// belongs at that LDS position.
// ---------------------------------------------------------------------------
template <int D, int WAVES, int KT>
struct DirectLoader {
    static constexpr int kLoads = (KT * D * 2 / 1024) / WAVES;  // per wave per tile
    int koff[kLoads];
    int voff[kLoads];

    __device__ __forceinline__ void init(int64_t k_ss, int64_t v_ss, int wave, int lane)
    {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int byte = (wave + WAVES * j) * 1024 + lane * 16;
            const int row = byte / (2 * D);
            const int pos = (byte % (2 * D)) >> 4;
            const int chunk = pos ^ swz(row & 15);
            koff[j] = (int)(((int64_t)row * k_ss + chunk * 8) * 2);
            voff[j] = (int)(((int64_t)row * v_ss + chunk * 8) * 2);
        }
    }

    // rows: number of valid rows from base (the rest read as zero)
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const _Float16* base, int64_t ss, int rows)
    {
        return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, rows * (int)ss * 2, kRsrcWord3);
    }
    // this wave's j-th load of a tile
    static __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t r, const int* off, unsigned char* tile,
                                                     int wave, int j)
    {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(tile + (wave + WAVES * j) * 1024), 16, off[j], 0,
                                                 0, 0);
    }
    static __device__ __forceinline__ void issue(const _Float16* base, int64_t ss, const int* off,
                                                 int rows, unsigned char* tile, int wave)
    {
        const __amdgpu_buffer_rsrc_t r = rsrc(base, ss, rows);
#pragma unroll
        for (int j = 0; j < kLoads; ++j) issue_one(r, off, tile, wave, j);
    }
};

// ---------------------------------------------------------------------------
// Paged E4M3 tiles. A 32-key tile is one page: its codes move into an LDS byte
// slot with buffer_load ... lds (row-major, D bytes per row; wave w's j-th
// load covers the 1 KB block (w + WAVES * j) of the tile, each lane one 16-code
// chunk). Chunk c of row r sits at position c ^ bswz<D>(r), which keeps the
// 8-byte K operand reads and the byte-transposing V reads free of bank
// conflicts. The MFMA operands are decoded from these codes in registers.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(4))) const int32_t const_i32;

// p[i] through the scalar cache: a read-only, wave-uniform table entry.
__device__ __forceinline__ int scalar_load(const int32_t* p, int i)
{
    return __builtin_bit_cast(const const_i32*, p)[i];
}

template <int D>
__device__ __forceinline__ int bswz(int r)
{
    return D == 256 ? (r & 15) : ((r >> 1) & 7);  // 16 chunks per row, or 8 (then rows pair up in a bank line)
}

// byte offset of code d of row r in a byte tile
template <int D>
__device__ __forceinline__ int btile_off(int r, int d)
{
    return r * D + ((((d >> 4) ^ bswz<D>(r))) << 4) + (d & 15);
}

template <int D, int WAVES, int KT>
struct ByteLoader {
    static constexpr int kLoads = (KT * D / 1024) / WAVES;  // per wave per tile
    int off[kLoads];

    // row_stride: bytes between consecutive tokens of one kv head (Hkv * D)
    __device__ __forceinline__ void init(int row_stride, int wave, int lane)
    {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int pos = (wave + WAVES * j) * 1024 + lane * 16;
            const int row = pos / D;
            const int chunk = ((pos % D) >> 4) ^ bswz<D>(row);
            off[j] = row * row_stride + chunk * 16;
        }
    }

    // base: the tile's first code of this kv head; bytes: the valid extent
    // (rows * row_stride; the rest of the tile reads as zero, code +0)
    __device__ __forceinline__ void issue(const uint8_t* base, int bytes, unsigned char* tile, int wave) const
    {
        __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRsrcWord3);
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void_t*)(tile + (wave + WAVES * j) * 1024), 16, off[j], 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// The attention kernel.
//
// Tiling<D, SRC, MODE>: KT keys per K/V tile and R slots per K and V ring.
// The causal FP16/BF16 K/V stream through rings of four 32-key slots (64 KB
// of LDS at D = 128, so two workgroups share a CU; 128 KB at D = 256), giving
// each load three iterations to arrive: all workgroups on an XCD read the
// same tiles at about the same time, so every tile costs them the latency of
// an L2 miss together. Dense D = 128 uses two 64-key slots instead (the same
// 64 KB). Block lists (two 32-key tiles per selected block) use two slots:
// their two-wave workgroups then take 32 KB, four per CU, which keeps two
// waves on every SIMD. The paged E4M3 source streams through four byte slots
// of 32-key pages (32 KB at D = 256; two for decode), decoded in registers as
// operands.
// ---------------------------------------------------------------------------
template <int D, int SRC, int MODE, bool KREG = false>
struct Tiling {
    // dense D = 128: 64-key tiles in a two-slot ring (half the barriers and
    // per-tile overhead of 32-key tiles, same LDS, two workgroups per CU).
    // Dense D = 256 keeps 32-key tiles: two score blocks per tile would not
    // fit the registers next to its FP32 output accumulators.
    static constexpr bool WIDE = D == 128 && MODE == KEYS_DENSE;
    static constexpr int KT = WIDE ? 64 : 32;
    // decode items stream only a few dozen tiles each: there the two-slot
    // ring's shorter unrolled loop measured faster than four slots
    // (the scaled E4M3 source converts K two tiles ahead, so it needs four,
    // unless its small decode workgroups convert K in registers)
    static constexpr int R = WIDE ? 2
                             : ((SRC == KV_E4M3_PAGED_SCALED && !KREG) || (MODE != KEYS_BLOCKS && MODE != KEYS_DECODE))
                                 ? 4
                                 : 2;
    static constexpr int PH = R;  // phases of the unrolled loop
};

template <int D, int WAVES, int SRC, int MODE, bool SPLIT, bool HALVES = false>
__global__ __launch_bounds__(WAVES * 64, (D == 128 && !HALVES ? 2 : 1) * (WAVES < 4 ? 4 / WAVES : 1))
void attn_fwd_kernel(const AttnArgs a)
{
    // HALVES: 8 waves over 128 rows; waves 0-3 stream keys [0, key_split),
    // waves 4-7 keys [key_split, Lkv) for the same rows, through one ring whose
    // slots hold both halves' tiles; the two states merge in LDS at the end
    static_assert(!HALVES || (WAVES == 8 && (SRC == KV_FP16 || SRC == KV_BF16) && MODE == KEYS_DENSE && !SPLIT),
                  "dense halves");
    constexpr int NHALF = HALVES ? 2 : 1;
    constexpr int M = (WAVES / NHALF) * kRowsPerWave;
    constexpr int KT = Tiling<D, SRC, MODE>::KT;
    constexpr int NSB = KT / 32;  // 32-key score blocks per tile
    constexpr int KS = KT / 16;   // 16-key PV k-steps per tile
    constexpr int KK = D / 16;    // MFMA k-steps over D for S
    constexpr int DB = D / 32;    // 32-wide d blocks of O^T
    // FP8 source: Q and K are E4M3 codes with per-row scales (QK^T on the FP8
    // matrix cores, 32x32x64), V is BF16 and streams as the 16-bit sources do
    constexpr bool F8 = SRC == KV_FP8QK;
    // 16-bit V tiles (else E4M3 codes, decoded in registers)
    constexpr bool VDIRECT = SRC != KV_E4M3_PAGED && SRC != KV_E4M3_PAGED_SCALED;
    // 16-bit K and V tiles
    constexpr bool DIRECT = VDIRECT && !F8;
    // The scaled E4M3 source converts each K code tile once per workgroup into
    // an FP16 tile (each wave a quarter of it, between its PV MFMAs), from
    // which every wave reads its K operands as the 16-bit sources do. Decode
    // workgroups of a single wave (at most 32 packed rows) instead convert the
    // K operands in registers where the MFMAs consume them, as V is decoded:
    // a lone wave has no one to share the tile with, and without its FP16
    // slots and deeper ring four such workgroups fit a CU's LDS.
    constexpr bool KREG = SRC == KV_E4M3_PAGED_SCALED && WAVES < 4;
    constexpr bool KCONV = SRC == KV_E4M3_PAGED_SCALED && !KREG;
    static_assert(!KREG || MODE == KEYS_DECODE, "register-converted K: decode only");
    constexpr int ROW = (VDIRECT ? 2 : 1) * D;      // bytes per LDS row of the V ring slots
    constexpr int KRROW = (DIRECT ? 2 : 1) * D;     // bytes per LDS row of the K ring slots
    constexpr int KROW = (DIRECT || KCONV ? 2 : 1) * D;  // bytes per row of the K operand tiles
    constexpr int TB = NHALF * KT * ROW;            // V slot bytes
    constexpr int TBK = NHALF * KT * KRROW;         // K slot bytes
    constexpr int R = Tiling<D, SRC, MODE, KREG>::R;
    // D = 256: the loads of a ring group are spread over the next iteration's
    // MFMA steps instead of being issued together after the barrier (the
    // tile's bytes then arrive in LDS spread out too; measured 3-4% faster on
    // the causal prefill, neutral at D = 128)
    constexpr bool SPREAD = DIRECT && D == 256;
    // P, the PV product and O in BF16
    constexpr bool BF = SRC == KV_BF16 || F8;
    constexpr int PH = Tiling<D, SRC, MODE, KREG>::PH;
    static_assert(R >= 2 && R <= 4, "ring depth");
    static_assert(VDIRECT || KT == 32, "an E4M3 tile is one 32-token page");
    static_assert(!F8 || (D == 128 && KT == 64 && R == 2 && MODE == KEYS_DENSE), "FP8 source: dense D128");
    // One array per ring slot: the compiler then sees that the LDS reads of
    // one slot do not alias the loads in flight into another (with one array
    // per ring it waits for every load into LDS, vmcnt(0), before each read).
    __shared__ __attribute__((aligned(1024))) unsigned char kslot0[TBK];
    __shared__ __attribute__((aligned(1024))) unsigned char kslot1[TBK];
    __shared__ __attribute__((aligned(1024))) unsigned char kslot2[R > 2 ? TBK : 16];
    __shared__ __attribute__((aligned(1024))) unsigned char kslot3[R > 3 ? TBK : 16];
    // F8: the FP32 scales of K(j)'s keys, one copy per wave, in kscl(j % R)
    __shared__ __attribute__((aligned(16))) float kscl0[F8 ? WAVES * KT : 4];
    __shared__ __attribute__((aligned(16))) float kscl1[F8 ? WAVES * KT : 4];
    __shared__ __attribute__((aligned(1024))) unsigned char vslot0[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char vslot1[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char vslot2[R > 2 ? TB : 16];
    __shared__ __attribute__((aligned(1024))) unsigned char vslot3[R > 3 ? TB : 16];
    // FP16 K tiles of the scaled E4M3 source: K(j) in khalf(j % 2)
    __shared__ __attribute__((aligned(1024))) unsigned char khalf0[KCONV ? KT * 2 * D : 16];
    __shared__ __attribute__((aligned(1024))) unsigned char khalf1[KCONV ? KT * 2 * D : 16];
    // s_waitcnt that leaves the (ring depth - 2) most recent load groups in
    // flight (ring depth - 3 when K is converted a tile earlier)
    using DLT = DirectLoader<D, WAVES, NHALF * KT>;  // the FP16 tiles (both halves' with HALVES)
    constexpr int kGroupLoads = (DIRECT ? DLT::kLoads : ByteLoader<D, WAVES, KT>::kLoads) +
                                (VDIRECT ? DLT::kLoads : ByteLoader<D, WAVES, KT>::kLoads) +
                                (F8 ? 1 : 0);
    constexpr int kVmLeft = (R - (KCONV ? 3 : 2)) * kGroupLoads;
    static_assert(kVmLeft < 64, "vmcnt range");
    constexpr int kWaitGroups = (kVmLeft & 15) | ((kVmLeft >> 4) << 14) | 0x0070;  // and lgkmcnt(0)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index in a scalar register: the LDS destinations of the loads into
    // LDS (M0) are then computed on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int half = HALVES ? wave >> 2 : 0;  // the half of the keys this wave streams
    const int rwave = HALVES ? wave & 3 : wave;  // the wave's 32 rows within the tile

    // ---- work item -> (b, h, query tile, key range) ----------------------
    // (the decode every launcher and the host-side checker share)
    const int item = item_of_block(a, blockIdx.x);
    if (item < 0) return;
    constexpr bool CAUSAL = MODE == KEYS_CAUSAL || MODE == KEYS_DECODE;
    const Item wi = decode_item(MODE, a, item, M);
    if (wi.empty) return;  // a segment past the key range: the merge skips it
    const int b = wi.b, h = wi.h, qt = wi.qt, seg = wi.seg;
    const int g = h / a.group;
    const int q0 = qt * M;
    // keys [key_begin, key_stop) are streamed; key_end bounds every row's keys
    // (HALVES: this wave's half; both halves run the iterations of the first,
    // the longer, and tiles past the second's keys are masked out)
    const int key_begin = HALVES ? half * a.key_split : wi.key_begin;
    const int key_stop = HALVES ? (half ? wi.key_stop : a.key_split) : wi.key_stop;
    const int key_end = wi.key_end;
    const int32_t* blist = wi.list ? a.idx + (((int64_t)b * a.Hq + h) * a.nqb + qt) * a.topk : nullptr;
    const int n_tiles = wi.list ? a.topk * (kTileN / KT)
                                : ((HALVES ? a.key_split : key_stop - key_begin) + KT - 1) / KT;
    const int key_last = key_end - 1;
    const int nblk = (a.Lkv + kTileN - 1) / kTileN;  // the last block may be partial

    auto tile_key0 = [&](int it) -> int {
        if (MODE == KEYS_BLOCKS && blist) {
            constexpr int kPer = kTileN / KT;  // tiles per selected block
            int blk = scalar_load(blist, it / kPer);  // wave-uniform: keeps the load addresses scalar
            blk = min(max(blk, 0), nblk - 1);
            return blk * kTileN + (it % kPer) * KT;
        }
        return key_begin + it * KT;
    };

    // ---- K/V sources -----------------------------------------------------
    const _Float16* kbase = nullptr;
    const _Float16* vbase = nullptr;
    const int32_t* table = nullptr;
    DLT dl;
    ByteLoader<D, WAVES, KT> bl;
    // F8: K codes and scales of this (b, kv head), contiguous rows of D codes
    const uint8_t* kcbase = nullptr;
    const float* kscbase = nullptr;
    if (VDIRECT) {
        kbase = a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh;
        vbase = a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh;
        dl.init(a.k_ss, a.v_ss, wave, lane);
    } else {
        table = a.table + (int64_t)b * a.table_stride;
        bl.init(a.Hkv * D, wave, lane);
    }
    if constexpr (F8) {
        kcbase = a.kc + ((int64_t)b * a.Hkv + g) * a.Lkv * D;
        kscbase = a.ksc + ((int64_t)b * a.Hkv + g) * a.Lkv;
        bl.init(D, wave, lane);
    }
    // Every load group issues the same number of loads, so that s_waitcnt
    // counts stay exact: a tile past the end is loaded with zero valid rows
    // (the buffer range check returns zeros) into its free slot.
    // rows of the tile at key0 that exist (a block list's partial last block
    // can leave none); wave-uniform, so the buffer descriptor stays scalar
    auto valid_rows = [&](bool ok, int key0) {
        return __builtin_amdgcn_readfirstlane(ok ? max(0, min(KT, key_end - key0)) : 0);
    };
    // E4M3: tile it is page table[tile_key0(it) / 32] (tiles are page aligned)
    auto issue_b = [&](const uint8_t* cache, int it, unsigned char* slot) {
        const bool ok = it < n_tiles;
        const int key0 = tile_key0(ok ? it : n_tiles - 1);
        const int page = min(max(scalar_load(table, key0 >> 5), 0), a.num_pages - 1);
        const int rows = ok ? min(KT, key_end - key0) : 0;
        bl.issue(cache + ((int64_t)page * 32 * a.Hkv + g) * D, rows * a.Hkv * D, slot, wave);
    };
    // HALVES: a slot holds tile it of both halves, rows [0, KT) from keys
    // it * KT and rows [KT, 2 KT) from keys key_split + it * KT. A wave's
    // loads j < kLoads / 2 fill the first half's rows, the others the second's,
    // read through a descriptor whose base is KT rows before that tile, so the
    // loader's row offsets (of rows KT .. 2 KT - 1) land on it; rows past a
    // half's keys read as zero.
    auto issue_halves = [&](const _Float16* base, int64_t ss, const int* off, int it, unsigned char* slot) {
        const bool ok = it < n_tiles;
        const int k0 = ok ? it * KT : 0;
        const int k1 = a.key_split + k0;
        const int r0 = __builtin_amdgcn_readfirstlane(ok ? max(0, min(KT, a.key_split - k0)) : 0);
        const int r1 = __builtin_amdgcn_readfirstlane(ok ? max(0, min(KT, key_end - k1)) : 0);
        const __amdgpu_buffer_rsrc_t d0 = DLT::rsrc(base + (int64_t)k0 * ss, ss, r0);
        const __amdgpu_buffer_rsrc_t d1 = DLT::rsrc(base + (int64_t)(k1 - KT) * ss, ss, KT + r1);
#pragma unroll
        for (int j = 0; j < DLT::kLoads; ++j) DLT::issue_one(j < DLT::kLoads / 2 ? d0 : d1, off, slot, wave, j);
    };
    auto issue_k = [&](int it, unsigned char* slot) {
        if constexpr (F8) {
            // the tile's codes, and its keys' scales (each wave its own copy of
            // the KT scales, one dword per lane, in the scale slot of this K slot)
            const bool ok = it < n_tiles;
            const int key0 = tile_key0(ok ? it : n_tiles - 1);
            const int rows = valid_rows(ok, key0);
            bl.issue(kcbase + (int64_t)key0 * D, rows * D, slot, wave);
            float* sc = slot == kslot0 ? kscl0 : kscl1;
            const __amdgpu_buffer_rsrc_t r =
                __builtin_amdgcn_make_buffer_rsrc((void*)(kscbase + key0), 0, rows * 4, kRsrcWord3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(sc + wave * KT), 4, lane * 4, 0, 0, 0);
        } else if constexpr (!DIRECT) {
            issue_b(a.kc, it, slot);
        } else if constexpr (HALVES) {
            issue_halves(kbase, a.k_ss, dl.koff, it, slot);
        } else {
            const bool ok = it < n_tiles;
            const int key0 = tile_key0(ok ? it : n_tiles - 1);
            DLT::issue(kbase + (int64_t)key0 * a.k_ss, a.k_ss, dl.koff, valid_rows(ok, key0), slot, wave);
        }
    };
    auto issue_v = [&](int it, unsigned char* slot) {
        if constexpr (!VDIRECT) {
            issue_b(a.vc, it, slot);
        } else if constexpr (HALVES) {
            issue_halves(vbase, a.v_ss, dl.voff, it, slot);
        } else {
            const bool ok = it < n_tiles;
            const int key0 = tile_key0(ok ? it : n_tiles - 1);
            DLT::issue(vbase + (int64_t)key0 * a.v_ss, a.v_ss, dl.voff, valid_rows(ok, key0), slot, wave);
        }
    };

    // ---- this lane's query row: head qh, position my_row ------------------------
    // Decode packs the group's heads: tile row r is head h + r / Lq, position
    // r % Lq; rows past the group are computed on a clamped head and dropped.
    int my_row = q0 + rwave * kRowsPerWave + l32, qh = h;
    bool row_ok = my_row < a.Lq;
    if (MODE == KEYS_DECODE) {
        const int r = my_row, j = r / a.Lq;
        my_row = r - j * a.Lq;
        qh = h + min(j, a.group - 1);
        row_ok = j < a.group;
    }

    // ---- Q fragment in registers: lane holds Q[row][16kk + 8hlf .. +7] ------
    // (F8: codes d = 64kk + 32hlf .. +31 of the row, and its scale folded into
    // the lane's softmax constant crow)
    constexpr int KK8 = D / 64;  // FP8 MFMA k-steps over D
    v8i qf8[F8 ? KK8 : 1];
    float crow = a.c;
    h8 qf[F8 ? 1 : KK];
    if constexpr (F8) {
        const int row = min(my_row, a.Lq - 1);
        const int64_t qrow = ((int64_t)b * a.Hq + qh) * a.Lq + row;
        const uint8_t* qp = a.qc + qrow * D;
#pragma unroll
        for (int kk = 0; kk < KK8; ++kk) {
            const u4 lo = *(const u4*)(qp + 64 * kk + 32 * hlf), hi = *(const u4*)(qp + 64 * kk + 32 * hlf + 16);
            qf8[kk] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        crow = a.c * a.qsc[qrow];
    } else {
        int row = min(my_row, a.Lq - 1);
        const _Float16* qp = a.q + (int64_t)b * a.q_sb + (int64_t)qh * a.q_sh + (int64_t)row * a.q_ss;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const h8*)(qp + 16 * kk + 8 * hlf);
        // With D = 256 the FP32 output accumulators take half the register
        // file; the read-only Q operands live in AGPRs (MFMA sources may) so
        // that the accumulators stay in VGPRs, where the rescale can scale them.
        if constexpr (D > 128) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) asm volatile("; q fragment to AGPRs" : "=a"(qf[kk]) : "0"(qf[kk]));
        }
    }

    // ---- per-lane LDS offsets ------------------------------------------------
    // K operand of S^T = K Q^T: row l32 (+32 per score block), d = 16kk + 8hlf .. +7.
    // FP16 V^T operand of O^T += V^T P^T through ds_read_b64_tr_b16: within
    // each 16-lane group G, source lane s points at 4 FP16 of key row
    // 4*(G/2) + s/4 (+8 for the second read), d = 32db + 16(G%2) + 4(s%4); the
    // transposing read then hands lane (G, t) the 4 keys of d = 32db+16(G%2)+t.
    // Both hand lane (G, t) the keys 4(G/2) + 0..3 and 8 + 4(G/2) + 0..3 of
    // its k-step, the order in which the score registers (and so P) hold them.
    // E4M3 V^T operand through ds_read_b64_tr_b8: the read gives lane (G, t)
    // element j from source lanes 2j and 2j+1 of its group, column
    // d = 32db + 16(G%2) + t; so source lane s of group G points at 8 codes of
    // key row 4*(G/2) + (s/2)%4 + 8*(s/8), d = 32db + 16(G%2) + 8(s%2).
    // F8 K operand of the 32x32x64 MFMA: row l32 (+32 per score block), the
    // 32 codes d = 64kk + 32hlf .. +31 as two 16-code chunks (the query codes
    // are held in the same d order, so every product pairs equal d).
    const int grp = lane >> 4, sl = lane & 15;
    int koff_s[KK];
    int koff8[F8 ? KK8 : 1][2];
    int voff_a[DB], voff_b[DB];
    if constexpr (F8) {
#pragma unroll
        for (int kk = 0; kk < KK8; ++kk)
#pragma unroll
            for (int c = 0; c < 2; ++c) koff8[kk][c] = btile_off<D>(l32, 64 * kk + 32 * hlf + 16 * c);
    }
    if constexpr (VDIRECT) {
        const int vrow = 4 * (grp >> 1) + (sl >> 2);
        const int vbyte = (sl & 1) * 8;
        const int vchunk = 2 * (grp & 1) + ((sl & 3) >> 1);
        const int hoff = half * KT * ROW;  // HALVES: this half's rows of the slot
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) koff_s[kk] = tile_off<D>(l32, 2 * kk + hlf) + hoff;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            voff_a[db] = tile_off<D>(vrow, 4 * db + vchunk) + vbyte + hoff;
            voff_b[db] = tile_off<D>(vrow + 8, 4 * db + vchunk) + vbyte + hoff;
        }
    } else {
        const int vrow = 4 * (grp >> 1) + ((sl >> 1) & 3) + 8 * (sl >> 3);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            koff_s[kk] = KCONV ? tile_off<D>(l32, 2 * kk + hlf) : btile_off<D>(l32, 16 * kk + 8 * hlf);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            voff_a[db] = btile_off<D>(vrow, 32 * db + 16 * (grp & 1) + 8 * (sl & 1));
            voff_b[db] = 0;
        }
    }

    f16x oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    float m_run = -INFINITY;  // reference maximum of scores * c (log2 units)
    float l_run = 0.f;        // this lane half's share of the sum of P

    // Operand fetch and use. FP16: the LDS read is the operand. E4M3: the
    // read brings 8 codes, decoded exactly to FP16 only where the MFMA
    // consumes them, so the read stays in flight meanwhile. Row offsets of
    // score block kb and k-step kstep are multiples of 16 rows, where both
    // swizzles repeat.
    using KRaw = std::conditional_t<VDIRECT, h8, u2>;  // V operand reads
    using KRawK = std::conditional_t<F8, v8i, std::conditional_t<DIRECT || KCONV, h8, u2>>;  // K operand reads
    auto kfetch = [&](const unsigned char* kt, int kb, int kk) -> KRawK {
        if constexpr (F8) {
            const u4 lo = *(const u4*)(kt + koff8[kk][0] + kb * 32 * KROW);
            const u4 hi = *(const u4*)(kt + koff8[kk][1] + kb * 32 * KROW);
            return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            return *(const KRawK*)(kt + koff_s[kk] + kb * 32 * KROW);
        }
    };
    auto decode8 = [](u2 w) -> h8 {
        const u2 lo = e4m3x4_to_f16(w.x), hi = e4m3x4_to_f16(w.y);
        return __builtin_bit_cast(h8, u4{lo.x, lo.y, hi.x, hi.y});
    };
    // Scaled K codes -> RNE16(RNE32(decode * k_scale)), the converted cache's
    // values: exact FP32 decode, FP32 multiply, FP16 pack rounding to nearest
    // even (the products are pinned in VGPRs so that the compiler cannot fuse
    // multiply and conversion into one rounding). Two codes per call.
    const float kscale = a.kscale;
    auto convert2 = [kscale](f2 d) -> uint32_t {
        float x0 = d.x * kscale, x1 = d.y * kscale;
        asm volatile("" : "+v"(x0), "+v"(x1));
        return __builtin_bit_cast(uint32_t, h2{(_Float16)x0, (_Float16)x1});
    };
    auto opuse_k = [&](const KRawK& r) -> h8 {
        if constexpr (DIRECT || KCONV) {
            return r;
        } else if constexpr (F8) {
            return h8{};  // unused: F8 codes go to the FP8 MFMA as they are
        } else if constexpr (KREG) {
            // the 8 codes' converted values, in the order decode8 gives
            const u4 w = {convert2(__builtin_amdgcn_cvt_pk_f32_fp8(r.x, false)),
                          convert2(__builtin_amdgcn_cvt_pk_f32_fp8(r.x, true)),
                          convert2(__builtin_amdgcn_cvt_pk_f32_fp8(r.y, false)),
                          convert2(__builtin_amdgcn_cvt_pk_f32_fp8(r.y, true))};
            return __builtin_bit_cast(h8, w);
        } else {
            return decode8(r);
        }
    };
    // Conversion of one K code tile into its FP16 tile, in 16-code chunks:
    // wave w converts chunks (w + WAVES * j) * 64 + lane, j < CV. A chunk is
    // read from the byte tile (row-major, bswz-swizzled), converted in eight
    // pairs and written as two 8-value chunks of the FP16 tile (tile_off
    // layout, as the 16-bit sources' tiles).
    constexpr int CV = KCONV ? (KT * D / 16) / (WAVES * 64) : 1;  // chunks per lane per tile
    static_assert(!KCONV || (KT * D / 16) % (WAVES * 64) == 0, "K conversion chunks");
    auto cv_row = [&](int j) { return ((wave + WAVES * j) * 64 + lane) / (D / 16); };
    auto cv_chunk = [&](int j) { return ((wave + WAVES * j) * 64 + lane) % (D / 16); };
    auto cv_read = [&](const unsigned char* bs, int j) -> u4 {
        const int row = cv_row(j);
        return *(const u4*)(bs + row * D + ((cv_chunk(j) ^ bswz<D>(row)) << 4));
    };
    // pair u (0..7) of a chunk: codes 2u, 2u+1
    auto cv_pair = [&](const u4& w, int u) -> uint32_t {
        const uint32_t word = u < 2 ? w.x : u < 4 ? w.y : u < 6 ? w.z : w.w;
        return (u & 1) ? convert2(__builtin_amdgcn_cvt_pk_f32_fp8(word, true))
                       : convert2(__builtin_amdgcn_cvt_pk_f32_fp8(word, false));
    };
    auto cv_write = [&](unsigned char* hs, int j, const u4& lo, const u4& hi) {
        const int row = cv_row(j), c = cv_chunk(j);
        *(u4*)(hs + tile_off<D>(row, 2 * c)) = lo;
        *(u4*)(hs + tile_off<D>(row, 2 * c + 1)) = hi;
    };
    // the whole conversion at once (prologue)
    auto convert_tile = [&](const unsigned char* bs, unsigned char* hs) {
#pragma unroll
        for (int j = 0; j < CV; ++j) {
            const u4 w = cv_read(bs, j);
            u4 lo, hi;
#pragma unroll
            for (int u = 0; u < 4; ++u) lo[u] = cv_pair(w, u);
#pragma unroll
            for (int u = 0; u < 4; ++u) hi[u] = cv_pair(w, u + 4);
            cv_write(hs, j, lo, hi);
        }
    };

    auto opuse_v = [&](const KRaw& r) -> h8 {
        if constexpr (VDIRECT)
            return r;
        else
            return decode8(r);
    };

    // one MFMA of S^T = K Q^T at k-step kk: FP16/BF16 32x32x16, or F8 32x32x64
    // on E4M3 codes (the unscaled form: scale operands 0)
    constexpr int KKS = F8 ? KK8 : KK;  // k-steps of S over D
    constexpr bool BFS = SRC == KV_BF16;
    auto mma_s = [&](const KRawK& kop, int kk, f16x acc) -> f16x {
        if constexpr (F8)
            return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop, qf8[kk], acc, 0, 0, 0, 0, 0, 0);
        else
            return mma<BFS>(opuse_k(kop), qf[kk], acc);
    };

    // S^T = K Q^T for KT keys x 32 queries (NSB blocks of 32 x 32)
    auto compute_s = [&](const unsigned char* kt, f16x (&s)[NSB]) {
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KKS; ++kk)
#pragma unroll
            for (int kb = 0; kb < NSB; ++kb) {
                s[kb] = mma_s(kfetch(kt, kb, kk), kk, s[kb]);
            }
    };

    // F8: the scores of a tile times their keys' scales (register r of score
    // block kb holds key 32kb + 8(r/4) + 4hlf + r%4); sc: this wave's copy of
    // the tile's KT scales. Applied before masking, so masked keys stay -inf.
    auto kscale_tile = [&](f16x (&s)[NSB], const float* sc) {
        if constexpr (F8) {
#pragma unroll
            for (int kb = 0; kb < NSB; ++kb)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const float4 v = *(const float4*)(sc + 32 * kb + 8 * gq + 4 * hlf);
                    s[kb][4 * gq] *= v.x;
                    s[kb][4 * gq + 1] *= v.y;
                    s[kb][4 * gq + 2] *= v.z;
                    s[kb][4 * gq + 3] *= v.w;
                }
        }
    };

    // O^T += V^T P^T
    auto vread = [&](const unsigned char* vt, int i) -> KRaw {
        const int kstep = i / DB, db = i % DB;
        if constexpr (VDIRECT) {
            s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(vt + kstep * 16 * ROW + voff_a[db]));
            s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(vt + kstep * 16 * ROW + voff_b[db]));
            return __builtin_bit_cast(h8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            return __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                              (lds_v2i_t*)(vt + kstep * 16 * ROW + voff_a[db])));
        }
    };
    auto compute_pv = [&](const unsigned char* vt, const h8* pk) {
#pragma unroll
        for (int i = 0; i < KS * DB; ++i) {
            const int kstep = i / DB, db = i % DB;
            oacc[db] = mma<BF>(opuse_v(vread(vt, i)), pk[kstep], oacc[db]);
        }
    };

    // Mask the keys a row may not see (register r of score block kb holds key
    // kb*32 + 8(r/4) + 4hlf + r%4), then return the row maximum times c.
    auto tile_needs_mask = [&](int key0) -> bool {
        if (CAUSAL) return (int64_t)key0 + KT > a.offset + q0 + 1 || key0 + KT > key_end;
        return key0 + KT > key_end;  // dense, block lists: the key tail
    };
    auto row_max = [&](f16x (&s)[NSB], int key0, bool masked) -> float {
        if (masked && tile_needs_mask(key0)) {
            const int64_t lim = CAUSAL ? min((int64_t)key_last, a.offset + my_row) : (int64_t)key_last;
            const int64_t rel = lim - key0 - 4 * hlf;  // mask register r when 8(r/4) + r%4 + 32kb > rel
#pragma unroll
            for (int kb = 0; kb < NSB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (8 * (r >> 2) + (r & 3) + 32 * kb > rel) s[kb][r] = -INFINITY;
        }
        float mx;
        if constexpr (NSB == 2) {
            float t[11];
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                t[i] = vmax3(s[0][3 * i], s[0][3 * i + 1], s[0][3 * i + 2]);
                t[5 + i] = vmax3(s[1][3 * i], s[1][3 * i + 1], s[1][3 * i + 2]);
            }
            t[10] = fmaxf(s[0][15], s[1][15]);
            float u0 = vmax3(t[0], t[1], t[2]), u1 = vmax3(t[3], t[4], t[5]), u2 = vmax3(t[6], t[7], t[8]);
            mx = vmax3(vmax3(u0, u1, u2), t[9], t[10]);
        } else {
            float t[5];
#pragma unroll
            for (int i = 0; i < 5; ++i) t[i] = vmax3(s[0][3 * i], s[0][3 * i + 1], s[0][3 * i + 2]);
            mx = vmax3(vmax3(t[0], t[1], t[2]), vmax3(t[3], t[4], s[0][15]), t[0]);
        }
        return wave_half_max(mx) * crow;
    };

    // Raise the reference maximum of the rows whose scores exceed it by more
    // than the slack, rescaling their O and l (wave-uniform branch).
    auto raise_max = [&](float mc) {
        const bool raise = mc > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            // rows that do not raise keep their state exactly (alpha = 1; also
            // for a row whose reference is still -inf)
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mc) : 1.f;
            m_run = raise ? mc : m_run;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        }
    };

    // One exponential unit: scores r, r+1 of score block kb -> P (FP16) in the
    // PV operand order (register r of block kb is k-step 2kb + r/8, slot r%8).
    // Units run block by block (u / 8 is the block), as the score MFMAs of the
    // next tile do, so a block's scores die as its successor's accumulate.
    const h2 ones = {(_Float16)1.f, (_Float16)1.f};
    const bf2 ones_bf = {(__bf16)1.f, (__bf16)1.f};
    auto exp_unit = [&](const f16x (&s)[NSB], int u, float m_use, h8* pk) {
        const int kb = u / 8, r = 2 * (u % 8);
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], crow, -m_use));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], crow, -m_use));
        h2 p;
        if constexpr (BF) {
            const bf2 pb = {(__bf16)e0, (__bf16)e1};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pb, ones_bf, l_run, false);
            p = __builtin_bit_cast(h2, pb);
        } else {
            p = h2{(_Float16)e0, (_Float16)e1};
            l_run = __builtin_amdgcn_fdot2(p, ones, l_run, false);
        }
        pk[2 * kb + (r >> 3)][r & 7] = p.x;
        pk[2 * kb + (r >> 3)][(r & 7) + 1] = p.y;
    };
    constexpr int NU = 8 * NSB;  // exponential units per tile
    auto exp_tile = [&](const f16x (&s)[NSB], h8* pk) {
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
        for (int u = 0; u < NU; ++u) exp_unit(s, u, m_use, pk);
    };

    // ---- pipeline --------------------------------------------------------------
    // K(j) and V(j) live in slot j % R (FP16 tiles, or E4M3 code tiles). Load
    // group g is {K(g+1), V(g)}; at the end of iteration it the slots of
    // K(it+1) and V(it) are free and group it+R is issued into them, so every
    // group has R-1 iterations to arrive. Invariant entering iteration it:
    // S(it) is in scur with its maximum folded into m_run; K(it+1) and V(it)
    // are in LDS; groups it+1 .. it+R-1 are in flight.
    // F8: the scales of K(j) are in kscl(j % 2) (the dense ring has two slots)
    auto kscl = [&](auto p) -> const float* {
        if constexpr (decltype(p)::value % 2 == 0)
            return kscl0;
        else
            return kscl1;
    };
    auto kslot = [&](auto p) -> unsigned char* {
        constexpr int S = decltype(p)::value % R;
        if constexpr (S == 0) return kslot0;
        else if constexpr (S == 1) return kslot1;
        else if constexpr (S == 2) return kslot2;
        else return kslot3;
    };
    auto vslot = [&](auto p) -> unsigned char* {
        constexpr int S = decltype(p)::value % R;
        if constexpr (S == 0) return vslot0;
        else if constexpr (S == 1) return vslot1;
        else if constexpr (S == 2) return vslot2;
        else return vslot3;
    };
    // KCONV: the FP16 K tile of K(j) is khslot(j % 2)
    auto khslot = [&](auto p) -> unsigned char* {
        if constexpr (decltype(p)::value % 2 == 0)
            return khalf0;
        else
            return khalf1;
    };
    // the tile the K operands of S(j) are read from
    auto ktile = [&](auto p) -> const unsigned char* {
        if constexpr (KCONV)
            return khslot(p);
        else
            return kslot(p);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    using P4 = std::integral_constant<int, 4>;

    // Prologue. KCONV also loads group 1 up front and converts K(0) and K(1);
    // thereafter iteration it converts K(it+2) between its PV MFMAs, so the
    // ring wait keeps one group fewer in flight (K(it+2)'s codes must be in LDS
    // when iteration it starts).
    issue_k(0, kslot0);
    issue_v(0, vslot0);
    issue_k(1, kslot1);
    if constexpr (KCONV) {
        issue_k(2, kslot(P2{}));
        issue_v(1, vslot(P1{}));
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if constexpr (KCONV) {
        convert_tile(kslot0, khalf0);
        convert_tile(kslot1, khalf1);
        __syncthreads();
    }
    f16x scur[NSB];
    compute_s(ktile(P0{}), scur);
    kscale_tile(scur, kscl0 + wave * KT);
    raise_max(row_max(scur, tile_key0(0), true));
    __syncthreads();
    {
        // groups 1 .. R-1 (SPREAD: 1 .. R-2; iteration 0 issues group R-1;
        // KCONV: group 1 is already in)
        constexpr int last = SPREAD ? R - 2 : R - 1;
        if constexpr (last >= 1 && !KCONV) {
            issue_k(2, kslot(P2{}));
            issue_v(1, vslot(P1{}));
        }
        if constexpr (last >= 2) {
            issue_k(3, kslot(P3{}));
            issue_v(2, vslot(P2{}));
        }
        if constexpr (last >= 3) {
            issue_k(4, kslot(P4{}));
            issue_v(3, vslot(P3{}));
        }
    }

    // end of iteration it (phase p = it % R): wait for group it+1, then refill
    // the slots read in this iteration with group it+R (SPREAD: iteration it+1
    // issues that group itself, see spread_group)
    auto refill = [&](auto p, int it) {
        using PN = std::integral_constant<int, decltype(p)::value + 1>;
        if constexpr (SPREAD) {
            (void)it;
            ring_barrier<kWaitGroups>();
        } else {
            ring_barrier<kWaitGroups>();
            issue_k(it + R + 1, kslot(PN{}));
            issue_v(it + R, vslot(p));
        }
    };

    // SPREAD: iteration it (phase p) issues group it+R-1, i.e. K(it+R) into
    // the slot of K(it) and V(it+R-1) into the slot of V(it-1); both were last
    // read in iteration it-1, before the barrier that ended it.
    using DL = DirectLoader<D, WAVES, KT>;
    struct SpreadGroup {
        __amdgpu_buffer_rsrc_t k, v;
    };
    auto spread_group = [&](int it) -> SpreadGroup {
        const int ki = it + R, vi = it + R - 1;
        const bool kok = ki < n_tiles, vok = vi < n_tiles;
        const int kk0 = tile_key0(kok ? ki : n_tiles - 1), vk0 = tile_key0(vok ? vi : n_tiles - 1);
        return {DL::rsrc(kbase + (int64_t)kk0 * a.k_ss, a.k_ss, valid_rows(kok, kk0)),
                DL::rsrc(vbase + (int64_t)vk0 * a.v_ss, a.v_ss, valid_rows(vok, vk0))};
    };

    // Steady state: tile it+1 exists and needs no mask. Written as explicit
    // steps separated by scheduling fences: block B issues the score MFMAs of
    // tile it+1 with the exponentials of tile it between them, block C the PV
    // MFMAs of tile it with the row maximum of tile it+1 between them; every
    // LDS operand read is issued two to four MFMAs ahead, the first V reads
    // already in the last steps of block B.
    auto iteration_main = [&](auto p, int it) {
        using PN = std::integral_constant<int, decltype(p)::value + 1>;
        using PK2 = std::integral_constant<int, decltype(p)::value + 2>;
        const unsigned char* kt = ktile(PN{});
        const unsigned char* vt = vslot(p);
        constexpr int NB = NSB * KKS;  // score MFMAs
        constexpr int NC = KS * DB;   // PV MFMAs
        f16x sn[NSB];
        h8 pk[KS];
        using PV = std::integral_constant<int, decltype(p)::value + R - 1>;
        constexpr int NL = SPREAD ? DL::kLoads : 1;  // loads per tile, one every NB / NL (NC / NL) steps
        static_assert(!SPREAD || (NB % NL == 0 && NC % NL == 0 && NB / NL >= 2 && NC / NL >= 2), "load spread");
        SpreadGroup sg;
        if constexpr (SPREAD) sg = spread_group(it);

        // V operands: the first PC are read in the last steps of block B
        KRaw vop[NC];
        constexpr int PC = D == 256 ? 3 : 2;  // V operand reads in flight

        // ---- block B ----
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        KRawK kop[NB];
        auto kread = [&](int i) { return kfetch(kt, i / KKS, i % KKS); };
        // K operand reads in flight (FP16 K operands of the scaled E4M3 source
        // take twice the registers of codes: one fewer at D = 256)
        constexpr int PB = D == 256 ? (KCONV ? 3 : 4) : 3;
#pragma unroll
        for (int i = 0; i < PB; ++i) kop[i] = kread(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i + PB < NB) kop[i + PB] = kread(i + PB);
            const int kb = i / KKS, kk = i % KKS;
            sn[kb] = mma_s(kop[i], kk, kk == 0 ? f16x{} : sn[kb]);
            if (i >= NB - PC) vop[i - (NB - PC)] = vread(vt, i - (NB - PC));
            if constexpr (SPREAD) {
                if (i % (NB / NL) == 1) DL::issue_one(sg.k, dl.koff, kslot(p), wave, i / (NB / NL));
            }
            // exponential units spread evenly over the steps
#pragma unroll
            for (int u = (i * NU) / NB; u < ((i + 1) * NU) / NB; ++u) exp_unit(scur, u, m_use, pk);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- block C ----
        __builtin_amdgcn_sched_barrier(0);
        float macc = -INFINITY, mfull = -INFINITY;
        constexpr int NMX = 8 * NSB;  // max3 units: two scores each
        // Steps carrying the max units. With one wave per SIMD (D = 256) the
        // maximum is finished, and exchanged between the lane halves, in the
        // first half of the block, so the remaining MFMAs cover its latency;
        // with two waves per SIMD (D = 128) the other wave covers it, and the
        // units are better spread over the whole block.
        constexpr bool XCHG_EARLY = D == 256;
        constexpr int MX0 = XCHG_EARLY ? 1 : 2;
        constexpr int MXS = XCHG_EARLY ? NC / 2 : NC - 2;
        // KCONV: this wave's chunks of K(it+2) are read at step 0 and converted
        // pair by pair over steps CU0 .. CU0+CUS-1, each chunk written to the
        // FP16 tile K(it) vacated once its eight pairs are done
        constexpr int NCU = 8 * CV;
        constexpr int CU0 = 2;
        constexpr int CUS = NC - 3;
        u4 cw[CV], clo[CV], chi[CV];
        // the step of chunk j's first pair, less two
        auto cv_read_step = [](int j) {
            int i = CU0;
            while (((i - CU0 + 1) * NCU) / CUS <= 8 * j) ++i;
            return i - 2 < 0 ? 0 : i - 2;
        };
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            if (i + PC < NC) vop[i + PC] = vread(vt, i + PC);
            const int kstep = i / DB, db = i % DB;
            oacc[db] = mma<BF>(opuse_v(vop[i]), pk[kstep], oacc[db]);
            if constexpr (KCONV) {
                // chunk j's codes are read two steps before its first pair
#pragma unroll
                for (int j = 0; j < CV; ++j)
                    if (i == cv_read_step(j)) cw[j] = cv_read(kslot(PK2{}), j);
                if (i >= CU0 && i < CU0 + CUS) {
#pragma unroll
                    for (int u = ((i - CU0) * NCU) / CUS; u < ((i - CU0 + 1) * NCU) / CUS; ++u) {
                        const int j = u / 8, pr = u % 8;
                        if (pr < 4)
                            clo[j][pr] = cv_pair(cw[j], pr);
                        else
                            chi[j][pr - 4] = cv_pair(cw[j], pr);
                        if (pr == 7) cv_write(khslot(p), j, clo[j], chi[j]);
                    }
                }
            }
            if constexpr (SPREAD) {
                if (i % (NC / NL) == 1) DL::issue_one(sg.v, dl.voff, vslot(PV{}), wave, i / (NC / NL));
            }
            // row-maximum units
            if (i >= MX0 && i < MX0 + MXS) {
#pragma unroll
                for (int u = ((i - MX0) * NMX) / MXS; u < ((i - MX0 + 1) * NMX) / MXS; ++u) {
                    const int e = 2 * u;  // scores e, e+1 of the flattened NSB x 16 registers
                    if constexpr (F8) {
                        // keys 32kb + 8(r/4) + 4hlf + r%4 and the next: two consecutive scales
                        const int kb = e / 16, r = e % 16;
                        const float2 sc = *(const float2*)(kscl(PN{}) + wave * KT + 32 * kb + 8 * (r >> 2) +
                                                           4 * hlf + (r & 3));
                        sn[kb][r] *= sc.x;
                        sn[kb][r + 1] *= sc.y;
                    }
                    macc = vmax3(macc, sn[e / 16][e % 16], sn[(e + 1) / 16][(e + 1) % 16]);
                }
            }
            if (XCHG_EARLY && i == MX0 + MXS - 1) mfull = wave_half_max(macc);
            __builtin_amdgcn_sched_barrier(0);
        }
        raise_max((XCHG_EARLY ? mfull : wave_half_max(macc)) * crow);
        refill(p, it);
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb) scur[kb] = sn[kb];
    };

    // Any iteration, masked tiles and the last tile included.
    auto iteration_tail = [&](auto p, int it) {
        using PN = std::integral_constant<int, decltype(p)::value + 1>;
        if constexpr (SPREAD) {
            using PV = std::integral_constant<int, decltype(p)::value + R - 1>;
            const SpreadGroup sg = spread_group(it);
#pragma unroll
            for (int j = 0; j < DL::kLoads; ++j) {
                DL::issue_one(sg.k, dl.koff, kslot(p), wave, j);
                DL::issue_one(sg.v, dl.voff, vslot(PV{}), wave, j);
            }
        }
        // P and PV of this tile first, then the scores of the next: the scores
        // of the two tiles are never live together (fewer registers than the
        // pipelined iteration needs)
        h8 pk[KS];
        exp_tile(scur, pk);
        compute_pv(vslot(p), pk);
        f16x sn[NSB];
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb) sn[kb] = f16x{};
        if (it + 1 < n_tiles) {
            compute_s(ktile(PN{}), sn);
            kscale_tile(sn, kscl(PN{}) + wave * KT);
        }
        if constexpr (KCONV) {
            // K(it+2) into the FP16 tile K(it) vacated (past the last tile the
            // codes are the zeros of an empty load; they are never used)
            using PK2 = std::integral_constant<int, decltype(p)::value + 2>;
            convert_tile(kslot(PK2{}), khslot(p));
        }
        if (it + 1 < n_tiles) raise_max(row_max(sn, tile_key0(it + 1), true));
        refill(p, it);
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb) scur[kb] = sn[kb];
    };

    // tiles 0 .. n_plain-1 need no mask (a prefix of the tile sequence)
    int n_plain = n_tiles;
    if (CAUSAL) {
        const int64_t lim = min(a.offset + q0 + 1, (int64_t)key_end);  // keys every row of the tile sees
        n_plain = (int)max((int64_t)0, min((int64_t)n_tiles, (lim - key_begin) / KT));
    } else if (MODE == KEYS_DENSE) {
        n_plain = min(n_tiles, (key_end - key_begin) / KT);
    } else if (MODE == KEYS_BLOCKS && a.Lkv % kTileN != 0) {
        // a partial last block: a dense-prefix item's keys ascend, so only its
        // last tiles need the tail mask; a list may hold the partial block at
        // any position, so every one of its tiles is checked
        n_plain = blist ? 0 : (key_stop - key_begin) / KT;
    }
    int it = 0;
    for (; it + PH < n_plain; it += PH) {
        iteration_main(P0{}, it);
        iteration_main(P1{}, it + 1);
        if constexpr (PH > 2) iteration_main(P2{}, it + 2);
        if constexpr (PH > 3) iteration_main(P3{}, it + 3);
    }
    if constexpr (MODE == KEYS_DECODE) {
        // short items: every plain tile whose successor is plain takes the
        // pipelined path, not only those of whole unrolled rounds
        for (; it + 1 < n_plain; ++it) {
            const int ph = it % PH;
            if (ph == 0)
                iteration_main(P0{}, it);
            else if (ph == 1)
                iteration_main(P1{}, it);
            else if (ph == 2) {
                if constexpr (PH > 2) iteration_main(P2{}, it);
            } else {
                if constexpr (PH > 3) iteration_main(P3{}, it);
            }
        }
    }
    for (; it < n_tiles; ++it) {
        const int ph = it % PH;
        if (ph == 0)
            iteration_tail(P0{}, it);
        else if (ph == 1)
            iteration_tail(P1{}, it);
        else if (ph == 2) {
            if constexpr (PH > 2) iteration_tail(P2{}, it);
        } else {
            if constexpr (PH > 3) iteration_tail(P3{}, it);
        }
    }

    // no load into LDS may still be in flight when the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(kWaitVm0);

    // ---- epilogue ------------------------------------------------------------
    float l_tot = wave_half_sum(l_run);
    if constexpr (HALVES) {
        // the second half's waves leave O^T, the maximum and the row sum in the
        // first K slots (16 KB of O per wave, lane-major float4s) and the
        // first V slot; the first half's waves merge them into theirs:
        // M = max(m0, m1), O = O0 2^(m0 - M) + O1 2^(m1 - M), l likewise
        __syncthreads();  // every wave is done with the ring
        float4* xo = (float4*)((rwave < 2 ? kslot0 : kslot1) + (rwave & 1) * 16384);
        float2* xml = (float2*)vslot0 + rwave * 64;
        if (half == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    xo[(db * 4 + g4) * 64 + lane] = float4{oacc[db][4 * g4], oacc[db][4 * g4 + 1],
                                                           oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]};
            xml[lane] = float2{m_run, l_tot};
        }
        __syncthreads();
        if (half == 1) return;
        const float2 ml1 = xml[lane];
        const float mx = fmaxf(m_run, ml1.x);
        const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
        const float a1 = ml1.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml1.x - mx);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 o1 = xo[(db * 4 + g4) * 64 + lane];
                oacc[db][4 * g4] = oacc[db][4 * g4] * a0 + o1.x * a1;
                oacc[db][4 * g4 + 1] = oacc[db][4 * g4 + 1] * a0 + o1.y * a1;
                oacc[db][4 * g4 + 2] = oacc[db][4 * g4 + 2] * a0 + o1.z * a1;
                oacc[db][4 * g4 + 3] = oacc[db][4 * g4 + 3] * a0 + o1.w * a1;
            }
        l_tot = l_tot * a0 + ml1.y * a1;
        m_run = mx;
    }
    if (!row_ok) return;
    const int64_t bh = (int64_t)b * a.Hq + qh;
    // block lists split only the dense-prefix query blocks
    const bool to_part = SPLIT && (MODE != KEYS_BLOCKS || qt < a.dense_prefix);
    if (to_part) {
        float* op = a.o_part + (((int64_t)seg * a.B * a.Hq + bh) * a.part_lq + my_row) * D;
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
            *(float2*)(a.ml_part + (((int64_t)seg * a.B * a.Hq + bh) * a.part_lq + my_row) * 2) = ml;
        }
    } else {
        const float inv = a.oscale / l_tot;
        _Float16* op = a.o + (int64_t)b * a.o_sb + (int64_t)qh * a.o_sh + (int64_t)my_row * a.o_ss;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                int d = db * 32 + 8 * g4 + 4 * hlf;
                h4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = to_out<BF>(oacc[db][4 * g4 + e] * inv);
                *(h4*)(op + d) = v4;
            }
        if (a.lse && hlf == 0)
            a.lse[bh * a.Lq + my_row] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
    }
}

// ---------------------------------------------------------------------------
// Decode of 33..64 packed rows at D = 256 from the paged E4M3 cache: 16-row
// waves on v_mfma_f32_16x16x32_f16, NR = 4 of them per key half, two key
// halves per workgroup (eight waves, two per SIMD, where the four-wave kernel
// has one wave per SIMD and two 32-row waves of padding), the halves' states
// merged in LDS at the end. (Six row waves for 65..96 rows, three waves per
// SIMD, leave too few registers to read operands ahead and are not used.)
//
// MFMA layouts (16x16x32): A lane l holds row l % 16, k = 8 (l / 16) .. +7;
// B lane l holds column l % 16, the same k; D register r of lane l is row
// 4 (l / 16) + r, column l % 16. With lane (q, g) = (l % 16, l / 16):
//  - S^T = K Q^T per 16-key block kb: A = FP16 K rows 16 kb + q, dims
//    32 kk + 8 g .. +7 (eight k-steps over D); B = Q^T of query row q (the
//    wave's packed row 16 rw + q); lane (q, g) gets the scores of keys
//    16 kb + 4 g + r for its query q.
//  - P^T, the B operand of O^T += V^T P^T, takes them in that order: k-index
//    8 g + i stands for key pi(8 g + i) = 4 g + i (i < 4), 16 + 4 g + i - 4.
//  - V^T, the A operand (16 d x 32 k), lane (d, g): codes of keys pi(8 g .. +7)
//    at column 16 db + d, through ds_read_b64_tr_b8 (source lane 2 j + h of
//    group g points at key row pi(8 g + j), bytes 16 db + 8 h .. +7).
//  - O^T per 16-wide d block db: lane (q, g) holds d = 16 db + 4 g + r.
// Ring per iteration j: all waves convert K(j+1)'s codes into its FP16 tile
// (both halves), compute S(j) and PV(j), wait for every load issued before
// the previous barrier, pass the barrier, and issue K(j+3) and V(j+2) into
// the code slots just freed: two K code slots, two V code slots and two FP16
// K slots, each holding both halves' tiles (132 KB). Eight waves issue the
// loads, one 1 KB block of each 8 KB tile each.
// ---------------------------------------------------------------------------
template <int NR, bool SCALED>
__global__ __launch_bounds__(NR * 128, 1) void attn_decode16_kernel(const AttnArgs a)
{
    static_assert(NR >= 1 && NR <= 6, "row waves: the merge space holds six waves' states");
    constexpr int D = 256, KT = 32, NW = 2 * NR, NT = NW * 64;
    constexpr int TB = KT * D;      // code tile bytes
    constexpr int FROW = 2 * D + 16;  // FP16 tile row bytes, padded: the 16 rows of an operand read fall in
                                      // 16 distinct 16-byte bank groups, and k-steps are immediate offsets
    constexpr int TF = KT * FROW;     // FP16 tile bytes
    typedef float f4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(1024))) unsigned char kcs0[2 * TB];
    __shared__ __attribute__((aligned(1024))) unsigned char kcs1[2 * TB];
    __shared__ __attribute__((aligned(1024))) unsigned char vcs0[2 * TB];
    __shared__ __attribute__((aligned(1024))) unsigned char vcs1[2 * TB];
    __shared__ __attribute__((aligned(1024))) unsigned char kfs0[2 * TF];
    __shared__ __attribute__((aligned(1024))) unsigned char kfs1[2 * TF];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave / NR, rw = wave % NR;
    const int q = lane & 15, gq = lane >> 4;

    const int item = item_of_block(a, blockIdx.x);
    if (item < 0) return;
    const Item wi = decode_item(KEYS_DECODE, a, item, kDecodeRows);
    if (wi.empty) return;
    const int b = wi.b, h0 = wi.h, seg = wi.seg;
    const int g = h0 / a.group;
    // tiles of the segment, the first half's share first
    const int n_all = (wi.key_stop - wi.key_begin + KT - 1) / KT;
    const int n0 = (n_all + 1) / 2;
    const int n_my = half ? n_all - n0 : n0;
    const int key_begin = wi.key_begin + (half ? n0 * KT : 0);
    const int key_stop = wi.key_stop;

    // this lane's packed row: head h0 + r / Lq, position r % Lq
    const int r = 16 * rw + q, jh = r / a.Lq;
    const int pos = r - jh * a.Lq, qh = h0 + min(jh, a.group - 1);
    const bool row_ok = jh < a.group;
    h8 qf[8];
    {
        const _Float16* qp = a.q + (int64_t)b * a.q_sb + (int64_t)qh * a.q_sh + (int64_t)pos * a.q_ss;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qf[kk] = *(const h8*)(qp + 32 * kk + 8 * gq);
    }
    const float crow = a.c;
    const int64_t qlim = a.offset + pos;  // the last key this row sees

    // loads: waves 0-7, one 1 KB block of a tile each
    const int32_t* table = a.table + (int64_t)b * a.table_stride;
    ByteLoader<D, 8, KT> bl;
    if (wave < 8) bl.init(a.Hkv * D, wave, lane);
    auto issue_tile = [&](const uint8_t* cache, int hf, int t, unsigned char* slot) {
        const int nh = hf ? n_all - n0 : n0;
        const bool ok = t < nh;
        const int key0 = wi.key_begin + (hf ? n0 * KT : 0) + (ok ? t : 0) * KT;
        const int page = min(max(scalar_load(table, key0 >> 5), 0), a.num_pages - 1);
        const int rows = ok ? min(KT, key_stop - key0) : 0;
        bl.issue(cache + ((int64_t)page * 32 * a.Hkv + g) * D, rows * a.Hkv * D, slot + hf * TB, wave);
    };
    auto issue_k = [&](int t, unsigned char* slot) {
        if (wave < 8) {
            issue_tile(a.kc, 0, t, slot);
            issue_tile(a.kc, 1, t, slot);
        }
    };
    auto issue_v = [&](int t, unsigned char* slot) {
        if (wave < 8) {
            issue_tile(a.vc, 0, t, slot);
            issue_tile(a.vc, 1, t, slot);
        }
    };

    // K code tile -> FP16 tile (both halves): 1024 chunks of 16 codes
    const float kscale = a.kscale;
    auto conv2 = [&](f2 d) -> uint32_t {
        if constexpr (SCALED) {
            float x0 = d.x * kscale, x1 = d.y * kscale;
            asm volatile("" : "+v"(x0), "+v"(x1));
            return __builtin_bit_cast(uint32_t, h2{(_Float16)x0, (_Float16)x1});
        } else {
            return __builtin_bit_cast(uint32_t, h2{(_Float16)d.x, (_Float16)d.y});  // exact
        }
    };
    auto convert = [&](const unsigned char* cs, unsigned char* fs) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = tid + NT * j;
            if (c < 1024) {
                const int hf = c >> 9, cc = c & 511, row = cc >> 4, ch = cc & 15;
                const u4 w = *(const u4*)(cs + hf * TB + row * D + ((ch ^ bswz<D>(row)) << 4));
                u4 lo, hi;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t word = w[u];
                    const uint32_t p0 = conv2(__builtin_amdgcn_cvt_pk_f32_fp8(word, false));
                    const uint32_t p1 = conv2(__builtin_amdgcn_cvt_pk_f32_fp8(word, true));
                    if (u < 2) {
                        lo[2 * u] = p0;
                        lo[2 * u + 1] = p1;
                    } else {
                        hi[2 * (u - 2)] = p0;
                        hi[2 * (u - 2) + 1] = p1;
                    }
                }
                *(u4*)(fs + hf * TF + row * FROW + 32 * ch) = lo;
                *(u4*)(fs + hf * TF + row * FROW + 32 * ch + 16) = hi;
            }
        }
    };

    f4 oacc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[i] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const h2 ones = {(_Float16)1.f, (_Float16)1.f};

    // per-lane LDS offsets: K operand (row 16 kb + q, FP16 chunk 4 kk + gq: the
    // k-step and the block are immediate offsets) and the V tr8 source (key
    // row pi(8 gq + sl / 2), bytes 8 (sl % 2) .. +7 of the chunk of d block db)
    const int sl = lane & 15, vj = sl >> 1, vh = sl & 1;
    const int vrow = vj < 4 ? 4 * gq + vj : 16 + 4 * gq + vj - 4;
    const int koff = q * FROW + 16 * gq;
    const int vbase = vrow * D + 8 * vh, vx = (vrow & 15) << 4;  // chunk db sits at db ^ (row % 16)

    // one tile: scores, softmax, PV (the wave's half, tile t of it)
    auto tile = [&](const unsigned char* kf, const unsigned char* vc, int t) {
        const unsigned char* kt = kf + half * TF;
        const unsigned char* vt = vc + half * TB;
        f4 s[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const h8*)(kt + koff + kb * 16 * FROW + 64 * kk),
                                                               qf[kk], s[kb], 0, 0, 0);
        const int key0 = key_begin + t * KT;
        if ((int64_t)key0 + KT > a.offset + 1 || key0 + KT > key_stop) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key0 + 16 * kb + 4 * gq + i;
                    if (key >= key_stop || key > qlim) s[kb][i] = -INFINITY;
                }
        }
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        const float2 m16 = row_pair(mx);
        mx = wave_half_max(fmaxf(m16.x, m16.y));
        const float mc = mx * crow;
        const bool raise = mc > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mc) : 1.f;
            m_run = raise ? mc : m_run;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[i] *= alpha;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        h8 pk;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][i], crow, -m_use));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][i + 1], crow, -m_use));
                const h2 p = {(_Float16)e0, (_Float16)e1};
                l_run = __builtin_amdgcn_fdot2(p, ones, l_run, false);
                pk[4 * kb + i] = p.x;
                pk[4 * kb + i + 1] = p.y;
            }
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            const u2 c = __builtin_bit_cast(
                u2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_v2i_t*)(vt + vbase + ((db << 4) ^ vx))));
            const u2 lo = e4m3x4_to_f16(c.x), hi = e4m3x4_to_f16(c.y);
            const h8 vop = __builtin_bit_cast(h8, u4{lo.x, lo.y, hi.x, hi.y});
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pk, oacc[db], 0, 0, 0);
        }
    };

    // prologue: K(0), K(1), V(0), V(1); K(0) converted; then K(2)
    issue_k(0, kcs0);
    issue_k(1, kcs1);
    issue_v(0, vcs0);
    issue_v(1, vcs1);
    ring_barrier<kWaitAll>();  // vmcnt(0), lgkmcnt(0)
    convert(kcs0, kfs0);
    ring_barrier<kWaitAll>();
    issue_k(2, kcs0);

    // iteration j: convert K(j+1), tile j, then wait, barrier, K(j+3), V(j+2)
    auto iteration = [&](auto p, int j) {
        constexpr int P = decltype(p)::value;
        unsigned char* kc_next = P == 0 ? kcs1 : kcs0;  // K(j+1)'s codes
        unsigned char* kf_next = P == 0 ? kfs1 : kfs0;
        const unsigned char* kf_cur = P == 0 ? kfs0 : kfs1;
        unsigned char* vc_cur = P == 0 ? vcs0 : vcs1;
        convert(kc_next, kf_next);
        if (j < n_my) tile(kf_cur, vc_cur, j);
        ring_barrier<kWaitAll>();
        issue_k(j + 3, kc_next);
        issue_v(j + 2, vc_cur);
    };
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    int j = 0;
    for (; j + 1 < n0; j += 2) {
        iteration(Q0{}, j);
        iteration(Q1{}, j + 1);
    }
    if (j < n0) iteration(Q0{}, j);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no load into LDS in flight at the end

    // row sums over the four lanes of a query; then the halves' merge
    const float2 l16 = row_pair(l_run);
    l_run = wave_half_sum(l16.x + l16.y);
    __syncthreads();
    {
        // half 1 leaves O (16 KB per wave) and (m, l) in the ring's space
        unsigned char* xb = rw < 2 ? kfs0 : rw < 4 ? kfs1 : rw == 4 ? vcs0 : vcs1;
        f4* xo = (f4*)(xb + (rw < 4 ? (rw & 1) * 16384 : 0));
        f2* xml = (f2*)kcs0 + rw * 64;
        if (half == 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) xo[i * 64 + lane] = oacc[i];
            xml[lane] = f2{m_run, l_run};
        }
        __syncthreads();
        if (half == 1) return;
        const f2 ml1 = xml[lane];
        const float mx = fmaxf(m_run, ml1.x);
        const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
        const float a1 = ml1.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml1.x - mx);
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[i] = oacc[i] * a0 + xo[i * 64 + lane] * a1;
        l_run = l_run * a0 + ml1.y * a1;
        m_run = mx;
    }
    if (!row_ok) return;
    const int64_t bh = (int64_t)b * a.Hq + qh;
    float* op = a.o_part + (((int64_t)seg * a.B * a.Hq + bh) * a.part_lq + pos) * D;
#pragma unroll
    for (int db = 0; db < 16; ++db) *(f4*)(op + 16 * db + 4 * gq) = oacc[db];
    if (gq == 0) *(f2*)(a.ml_part + (((int64_t)seg * a.B * a.Hq + bh) * a.part_lq + pos) * 2) = f2{m_run, l_run};
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
    const int su = seg_units(nt, m.nseg);
    const int nseg = (nt + su - 1) / su;

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
    if (m.lse && lane == 0) m.lse[bh * m.lse_sh + i] = (mmax + __log2f(den)) * 0.69314718055994530942f;
}

// The same merge for splits with many segments (decode): one 256-thread
// workgroup per (query row, COLS columns), so that a decode of a few rows
// still spreads over the CUs (COLS = 16 then, else 64). Its threads split into
// streams of COLS / 4 threads, each thread one float4 of the columns, stream t
// summing segments t, t + S, t + 2S, ... (S streams) in that order. Each
// thread issues its first kPre partial loads before the segment weights
// 2^(m_s - M) are formed in LDS, so that the two latencies overlap; the S
// partial sums are added in stream order, so the result is fixed run to run.
constexpr int kWideMaxSeg = kMaxDecodeSeg;
constexpr int kWideThreads = 256;
template <int D, int COLS>
__global__ __launch_bounds__(kWideThreads) void attn_merge_wide_kernel(const MergeArgs m)
{
    constexpr int TPS = COLS / 4;               // threads per stream
    constexpr int S = kWideThreads / TPS;       // streams
    constexpr int W = kWideThreads / 64;        // waves
    constexpr int kPre = 1024 / S < 16 ? 1024 / S : 16;  // partial loads per thread and round
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row_id = blockIdx.x;
    const int col0 = blockIdx.y * COLS;
    const int i = (int)(row_id % m.Lq);
    const int64_t bh = row_id / m.Lq;
    const int b = (int)(bh / m.Hq), h = (int)(bh % m.Hq);
    const int qt = i / m.rows_per_tile;
    const int last_row = min((qt + 1) * m.rows_per_tile, m.Lq) - 1;
    const int key_end = (int)min((int64_t)m.Lkv, m.offset + last_row + 1);
    const int nt = (key_end + kTileN - 1) / kTileN;
    const int su = seg_units(nt, m.nseg);
    const int nseg = (nt + su - 1) / su;  // <= kWideMaxSeg (checked at launch)
    const int64_t seg_stride = (int64_t)m.B * m.Hq * m.Lq;

    const int st = tid / TPS, c = tid % TPS;
    const float4* op = (const float4*)(m.o_part + row_id * D + col0) + c;
    float4 v[kPre];
    auto load_round = [&](int base) {
#pragma unroll
        for (int j = 0; j < kPre; ++j) {
            const int sg = base + st + S * j;
            if (sg < nseg) v[j] = op[sg * seg_stride * (D / 4)];
        }
    };
    load_round(0);

    __shared__ float wgt[kWideMaxSeg];
    __shared__ float lsg[kWideMaxSeg];
    __shared__ float red[W];
    __shared__ float4 part[S][TPS];
    // M = max of the segment maxima
    float mx = -INFINITY;
    for (int sg = tid; sg < nseg; sg += kWideThreads) {
        const float2 ml = *(const float2*)(m.ml_part + (sg * seg_stride + row_id) * 2);
        wgt[sg] = ml.x;
        lsg[sg] = ml.y;
        mx = fmaxf(mx, ml.x);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float mmax = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) mmax = fmaxf(mmax, red[w]);
    __syncthreads();
    // weights, and sum w_s l_s (each thread its segments, then in wave order)
    float den = 0.f;
    for (int sg = tid; sg < nseg; sg += kWideThreads) {
        const float ls = lsg[sg];
        const float w = ls == 0.f ? 0.f : __builtin_amdgcn_exp2f(wgt[sg] - mmax);  // no visible key: no weight
        wgt[sg] = w;
        den += w * ls;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
    if (lane == 0) red[wave] = den;
    __syncthreads();
    float dsum = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) dsum += red[w];

    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int base = 0; base < nseg; base += S * kPre) {
        if (base > 0) load_round(base);
#pragma unroll
        for (int j = 0; j < kPre; ++j) {
            const int sg = base + st + S * j;
            if (sg < nseg) {
                const float w = wgt[sg];
                acc.x += w * v[j].x;
                acc.y += w * v[j].y;
                acc.z += w * v[j].z;
                acc.w += w * v[j].w;
            }
        }
    }
    part[st][c] = acc;
    __syncthreads();
    if (st != 0) return;
    float4 sum = part[0][c];
#pragma unroll
    for (int t = 1; t < S; ++t) {
        sum.x += part[t][c].x;
        sum.y += part[t][c].y;
        sum.z += part[t][c].z;
        sum.w += part[t][c].w;
    }
    const float inv = m.oscale / dsum;
    _Float16* o = m.o + (int64_t)b * m.o_sb + (int64_t)h * m.o_sh + (int64_t)i * m.o_ss + col0 + 4 * c;
    o[0] = (_Float16)(sum.x * inv);
    o[1] = (_Float16)(sum.y * inv);
    o[2] = (_Float16)(sum.z * inv);
    o[3] = (_Float16)(sum.w * inv);
    if (m.lse && blockIdx.y == 0 && c == 0) m.lse[bh * m.lse_sh + i] = (mmax + __log2f(dsum)) * 0.69314718055994530942f;
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

// Dense D = 128: the last partial round's items as 8-wave workgroups that
// split each item's keys between their two halves.
hipError_t launch_dense_halves(const AttnArgs& a, KvSource src, hipStream_t stream)
{
    int grid = a.per_xcd > 0 ? a.per_xcd * 8 : a.n_items;
    if (grid <= 0) return hipSuccess;
    if (src == KV_BF16)
        hipLaunchKernelGGL((attn_fwd_kernel<128, 8, KV_BF16, KEYS_DENSE, false, true>), dim3(grid), dim3(512), 0,
                           stream, a);
    else if (src == KV_FP16)
        hipLaunchKernelGGL((attn_fwd_kernel<128, 8, KV_FP16, KEYS_DENSE, false, true>), dim3(grid), dim3(512), 0,
                           stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, KvSource src, KeyMode mode, bool split,
                           hipStream_t stream)
{
    if (mode == KEYS_DENSE && src == KV_FP8QK) {
        if constexpr (D == 128)
            return launch_one<D, 4, KV_FP8QK, KEYS_DENSE, false>(a, stream);
        else
            return hipErrorInvalidValue;
    }
    if (mode == KEYS_DENSE)
        return src == KV_BF16 ? launch_one<D, 4, KV_BF16, KEYS_DENSE, false>(a, stream)
                              : launch_one<D, 4, KV_FP16, KEYS_DENSE, false>(a, stream);
    if (src == KV_BF16) return hipErrorInvalidValue;
    if (mode == KEYS_BLOCKS) return hipErrorInvalidValue;
    if (src == KV_FP16)
        return split ? launch_one<D, 4, KV_FP16, KEYS_CAUSAL, true>(a, stream)
                     : launch_one<D, 4, KV_FP16, KEYS_CAUSAL, false>(a, stream);
    if (src == KV_E4M3_PAGED_SCALED)
        return split ? launch_one<D, 4, KV_E4M3_PAGED_SCALED, KEYS_CAUSAL, true>(a, stream)
                     : launch_one<D, 4, KV_E4M3_PAGED_SCALED, KEYS_CAUSAL, false>(a, stream);
    return split ? launch_one<D, 4, KV_E4M3_PAGED, KEYS_CAUSAL, true>(a, stream)
                 : launch_one<D, 4, KV_E4M3_PAGED, KEYS_CAUSAL, false>(a, stream);
}

hipError_t launch_attn(const AttnArgs& a, int D, KvSource src, KeyMode mode, bool split,
                       hipStream_t stream)
{
    if (mode == KEYS_DECODE) {
        // always split: the merge writes the output
        if (!split) return hipErrorInvalidValue;
        // the workgroup holds the packed rows in as few waves as fit them; at
        // D = 256, 33..64 rows take the 16-row-wave kernel
        const int waves = decode_waves(a.group * a.Lq);
        const int rows = a.group * a.Lq;
        if (D == 256 && rows > 32 && rows <= 64 && (src == KV_E4M3_PAGED_SCALED || src == KV_E4M3_PAGED)) {
            const int grid = a.per_xcd > 0 ? a.per_xcd * 8 : a.n_items;
            if (grid <= 0) return hipSuccess;
            if (src == KV_E4M3_PAGED_SCALED)
                hipLaunchKernelGGL((attn_decode16_kernel<4, true>), dim3(grid), dim3(512), 0, stream, a);
            else
                hipLaunchKernelGGL((attn_decode16_kernel<4, false>), dim3(grid), dim3(512), 0, stream, a);
            return hipGetLastError();
        }
        if (src == KV_E4M3_PAGED_SCALED) {
            if (D == 128)
                return waves == 1 ? launch_one<128, 1, KV_E4M3_PAGED_SCALED, KEYS_DECODE, true>(a, stream)
                                  : launch_one<128, 4, KV_E4M3_PAGED_SCALED, KEYS_DECODE, true>(a, stream);
            if (D == 256)
                return waves == 1 ? launch_one<256, 1, KV_E4M3_PAGED_SCALED, KEYS_DECODE, true>(a, stream)
                                  : launch_one<256, 4, KV_E4M3_PAGED_SCALED, KEYS_DECODE, true>(a, stream);
            return hipErrorInvalidValue;
        }
        if (src != KV_E4M3_PAGED) return hipErrorInvalidValue;
        if (D == 128)
            return waves == 1 ? launch_one<128, 1, KV_E4M3_PAGED, KEYS_DECODE, true>(a, stream)
                              : launch_one<128, 4, KV_E4M3_PAGED, KEYS_DECODE, true>(a, stream);
        if (D == 256)
            return waves == 1 ? launch_one<256, 1, KV_E4M3_PAGED, KEYS_DECODE, true>(a, stream)
                              : launch_one<256, 4, KV_E4M3_PAGED, KEYS_DECODE, true>(a, stream);
        return hipErrorInvalidValue;
    }
    if (mode == KEYS_BLOCKS) {
        if (D != 128 || src != KV_FP16) return hipErrorInvalidValue;
        return split ? launch_one<128, 2, KV_FP16, KEYS_BLOCKS, true>(a, stream)
                     : launch_one<128, 2, KV_FP16, KEYS_BLOCKS, false>(a, stream);
    }
    if (D == 128) return launch_d<128>(a, src, mode, split, stream);
    if (D == 256) return launch_d<256>(a, src, mode, split, stream);
    return hipErrorInvalidValue;
}

// Every kernel the launchers use, instantiated explicitly: the host compiler
// otherwise left the launch stubs of the paged E4M3 kernels undefined (the
// shared library then fails to load), with no diagnostic.
template __global__ void attn_fwd_kernel<128, 4, KV_FP16, KEYS_DENSE, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 8, KV_FP16, KEYS_DENSE, false, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 8, KV_BF16, KEYS_DENSE, false, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_FP16, KEYS_DENSE, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_BF16, KEYS_DENSE, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_BF16, KEYS_DENSE, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_FP8QK, KEYS_DENSE, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_FP16, KEYS_CAUSAL, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_FP16, KEYS_CAUSAL, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_FP16, KEYS_CAUSAL, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_FP16, KEYS_CAUSAL, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_E4M3_PAGED, KEYS_CAUSAL, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_E4M3_PAGED, KEYS_CAUSAL, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_E4M3_PAGED, KEYS_CAUSAL, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_E4M3_PAGED, KEYS_CAUSAL, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 2, KV_FP16, KEYS_BLOCKS, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 2, KV_FP16, KEYS_BLOCKS, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_E4M3_PAGED, KEYS_DECODE, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_E4M3_PAGED, KEYS_DECODE, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_E4M3_PAGED_SCALED, KEYS_CAUSAL, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_E4M3_PAGED_SCALED, KEYS_CAUSAL, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_E4M3_PAGED_SCALED, KEYS_CAUSAL, false>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_E4M3_PAGED_SCALED, KEYS_CAUSAL, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, KV_E4M3_PAGED_SCALED, KEYS_DECODE, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 4, KV_E4M3_PAGED_SCALED, KEYS_DECODE, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 1, KV_E4M3_PAGED_SCALED, KEYS_DECODE, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 1, KV_E4M3_PAGED_SCALED, KEYS_DECODE, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<128, 1, KV_E4M3_PAGED, KEYS_DECODE, true>(const AttnArgs);
template __global__ void attn_fwd_kernel<256, 1, KV_E4M3_PAGED, KEYS_DECODE, true>(const AttnArgs);
template __global__ void attn_decode16_kernel<4, true>(const AttnArgs);
template __global__ void attn_decode16_kernel<4, false>(const AttnArgs);

hipError_t launch_merge(const MergeArgs& m, int D, hipStream_t stream)
{
    int64_t rows = (int64_t)m.B * m.Hq * m.Lq;
    if (m.nseg >= 16) {
        // many segments per row: a workgroup per (row, 64 columns), or per
        // (row, 16 columns) when that leaves fewer workgroups than CUs
        if (rows <= 0) return hipSuccess;
        if (m.nseg > kWideMaxSeg || rows > 0x7fffffff) return hipErrorInvalidValue;
        if (D != 128 && D != 256) return hipErrorInvalidValue;
        const bool narrow = rows * (D / 64) < kComputeUnits;
        const dim3 grid((unsigned)rows, (unsigned)(D / (narrow ? 16 : 64)));
        if (D == 128) {
            if (narrow)
                hipLaunchKernelGGL((attn_merge_wide_kernel<128, 16>), grid, dim3(kWideThreads), 0, stream, m);
            else
                hipLaunchKernelGGL((attn_merge_wide_kernel<128, 64>), grid, dim3(kWideThreads), 0, stream, m);
        } else {
            if (narrow)
                hipLaunchKernelGGL((attn_merge_wide_kernel<256, 16>), grid, dim3(kWideThreads), 0, stream, m);
            else
                hipLaunchKernelGGL((attn_merge_wide_kernel<256, 64>), grid, dim3(kWideThreads), 0, stream, m);
        }
        return hipGetLastError();
    }
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
