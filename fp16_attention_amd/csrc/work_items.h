// Work items of the attention launches: the split plans the host chooses and
// the decode of a workgroup's item into (batch, head, query tile, key
// segment, key range). The launcher (abi.cpp), the kernel (attn_fwd.hip) and
// the host-side checker of the test suite all include this one header, so
// the ranges the checker verifies are the ranges the kernel uses.
//
// Plain C++ with no HIP headers: under hipcc the functions are host and
// device functions; under a host compiler they are ordinary inline code.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

namespace fa {

// Keys per 64-key unit of the split plans (and per VSA block).
constexpr int kTileN = 64;
// Query rows per wave (one 32-wide MFMA column block).
constexpr int kRowsPerWave = 32;
// Query rows per workgroup of the dense and causal launches (4 waves).
constexpr int kRowsPerTile = 128;
// Packed (head, position) rows of a decode work item, at most.
constexpr int kDecodeRows = 128;
constexpr int kComputeUnits = 256;  // MI355X
constexpr int kMaxSeg = 16;         // key segments per query tile, at most
constexpr int kMinSegUnits = 16;    // at least 1024 keys per segment
constexpr int kMaxDecodeSeg = 1024; // key segments of a decode, at most

// Waves (32 packed rows each) of a decode workgroup for `rows` packed rows:
// one when they fit one wave, so that a few live rows do not carry a full
// 128-row tile and four such workgroups share a CU, else four.
FA_HD inline int decode_waves(int rows) { return rows <= 32 ? 1 : 4; }

// KEYS_DECODE: causal rows of a few query positions (Lq <= 16), with the
// rows of every query head of a kv-head group packed into one tile, so each
// K/V byte is read once per group.
enum KeyMode { KEYS_DENSE = 0, KEYS_CAUSAL = 1, KEYS_BLOCKS = 2, KEYS_DECODE = 3 };

// Length, in 64-key units, of the key segments of a query tile whose keys span
// nt units, when it is split into at most nseg segments; the last one may be
// shorter, and the number that exist is ceil(nt / seg_units).
FA_HD inline int seg_units(int nt, int nseg) { return (nt + nseg - 1) / nseg; }

// The shape of one launch as its work items see it.
struct Geometry {
    int B, Hq, Hkv, group;
    int Lq, Lkv;
    int64_t offset;    // causal: kv_len - q_real
    int n_qt;          // query tiles per (b, h)
    int nseg;          // key segments per query tile (1: no split)
    int part_lq;       // rows per (segment, b, h) of the partial-state workspace
    int dense_prefix;  // block lists: dense query blocks per (b, h)
    int nqb;           // block lists: query blocks per (b, h)
    int topk;          // block lists: selected blocks per query block
    int n_items;       // work items
    int per_xcd;       // work items per XCD slice (0: identity mapping)
    int item_base;     // added to each decoded item (a launch over a later range of a plan's items)
    int key_split;     // dense halves: keys [0, key_split) and [key_split, Lkv) per work item (0: none)
};

// The work item of workgroup `block` (the XCD-aware mapping gives each of the
// 8 XCDs a contiguous range of items); -1 for a workgroup past the last item.
FA_HD inline int item_of_block(const Geometry& g, int block)
{
    const int item = g.per_xcd > 0 ? (block & 7) * g.per_xcd + (block >> 3) : block;
    return item < g.n_items ? item : -1;
}

struct Item {
    int b, h, qt, seg;
    // keys [key_begin, key_stop) are streamed in tiles; key_end bounds every
    // row's keys (causal: the tile's last row's limit)
    int key_begin, key_stop, key_end;
    bool list;   // block lists: the keys are the item's selected blocks
    bool empty;  // a segment past the tile's key range: no work, no output
};

// Decode of item `item` of a launch in key mode `mode` whose workgroups own
// `rows` query rows (decode: packed rows).
FA_HD inline Item decode_item(int mode, const Geometry& g, int item, int rows)
{
    item += g.item_base;
    Item it;
    it.seg = 0;
    it.list = false;
    it.empty = false;
    if (mode == KEYS_DECODE) {
        // (b, kv head, key segment); h is the group's first query head
        it.seg = item % g.nseg;
        const int r = item / g.nseg;
        it.b = r / g.Hkv;
        it.h = (r % g.Hkv) * g.group;
        it.qt = 0;
    } else if (mode == KEYS_CAUSAL) {
        const int j = item % g.group;
        int r = item / g.group;
        it.qt = r % g.n_qt;
        r /= g.n_qt;
        it.seg = r % g.nseg;
        r /= g.nseg;
        const int kvh = r % g.Hkv;
        it.b = r / g.Hkv;
        it.h = kvh * g.group + j;
    } else if (mode == KEYS_BLOCKS) {
        // items of one (b, h) are consecutive: the dense-prefix query blocks,
        // each split into nseg key segments, then the sparse query blocks
        const int n_dense = g.dense_prefix * g.nseg;
        const int per_bh = n_dense + (g.nqb - g.dense_prefix);
        const int bh = item / per_bh;
        const int r = item % per_bh;
        if (r < n_dense) {
            it.qt = r / g.nseg;
            it.seg = r % g.nseg;
        } else {
            it.qt = g.dense_prefix + (r - n_dense);
        }
        it.h = bh % g.Hq;
        it.b = bh / g.Hq;
    } else {
        it.qt = item % g.n_qt;
        const int r = item / g.n_qt;
        it.h = r % g.Hq;
        it.b = r / g.Hq;
    }
    const int q0 = it.qt * rows;
    it.key_begin = 0;
    it.key_stop = g.Lkv;
    it.key_end = g.Lkv;
    if (mode == KEYS_CAUSAL || mode == KEYS_DECODE) {
        const int last_row = (q0 + rows < g.Lq ? q0 + rows : g.Lq) - 1;
        const int64_t lim = g.offset + last_row + 1;
        it.key_end = (int)(lim < g.Lkv ? lim : (int64_t)g.Lkv);
        const int len = seg_units((it.key_end + kTileN - 1) / kTileN, g.nseg) * kTileN;
        it.key_begin = it.seg * len;
        const int stop = (it.seg + 1) * len;
        it.key_stop = stop < it.key_end ? stop : it.key_end;
        it.empty = it.key_begin >= it.key_stop;  // the merge skips segments past the key range
    } else if (mode == KEYS_BLOCKS) {
        if (it.qt < g.dense_prefix) {
            const int len = seg_units((g.Lkv + kTileN - 1) / kTileN, g.nseg) * kTileN;
            it.key_begin = it.seg * len;
            const int stop = (it.seg + 1) * len;
            it.key_stop = stop < g.Lkv ? stop : g.Lkv;
            it.empty = it.key_begin >= it.key_stop;
        } else {
            it.list = true;
        }
    }
    return it;
}

// ---------------------------------------------------------------------------
// Split plans (host): pure functions of the shape, so the workspace query and
// the launch agree and results are reproducible.
// ---------------------------------------------------------------------------
struct SplitPlan {
    int n_qt, nseg;
    size_t workspace;
};

// Bytes of the partial states of `rows` (segment, b, h, row) rows: FP32
// unnormalised O [rows][D] (256-byte aligned), then (m, l) pairs [rows][2].
inline size_t partial_bytes(size_t rows, int D, size_t* o_bytes_out = nullptr)
{
    const size_t o_bytes = ((rows * (size_t)D * 4) + 255) & ~(size_t)255;
    if (o_bytes_out) *o_bytes_out = o_bytes;
    return o_bytes + rows * 2 * 4;
}

// Causal prefill: each query tile's key range is cut into nseg near-equal
// segments; nseg is the smallest count whose work items fill the resident
// workgroup slots of the chip (one per CU at D = 256, two at D = 128) in whole
// rounds best, since a last, partly filled round costs far more than its
// share of the work (about half a round's time at a quarter filled, with two
// slots per CU).
inline SplitPlan plan_split(int B, int Hq, int D, int q_rows, int kv_len)
{
    SplitPlan p;
    p.n_qt = (q_rows + kRowsPerTile - 1) / kRowsPerTile;
    const int max_units = (kv_len + kTileN - 1) / kTileN;
    const int64_t items = (int64_t)B * Hq * p.n_qt;
    const int64_t slots = (int64_t)kComputeUnits * (D == 128 ? 2 : 1);
    auto fill = [&](int n) {
        const int64_t work = items * n;
        const int64_t rounds = (work + slots - 1) / slots;
        return (double)work / (double)(rounds * slots);
    };
    p.nseg = 1;
    double best = fill(1);
    for (int n = 2; n <= kMaxSeg && seg_units(max_units, n) >= kMinSegUnits; ++n) {
        const double f = fill(n);
        if (f > best * 1.01) {
            best = f;
            p.nseg = n;
        }
    }
    p.workspace = p.nseg <= 1 ? 0 : partial_bytes((size_t)p.nseg * B * Hq * q_rows, D);
    return p;
}

// Decode: one work item per (b, kv head, segment), as many segments as it
// takes to give every workgroup slot of the GPU (4 / waves per CU, twice that
// at D = 128) its own stream of the cache, each segment at least
// 1024 * waves / 4 keys, and at most kMaxDecodeSeg segments.
inline SplitPlan plan_decode(int B, int Hq, int Hkv, int D, int q_rows, int kv_len)
{
    SplitPlan p;
    p.n_qt = 1;
    const int max_units = (kv_len + kTileN - 1) / kTileN;
    const int waves = decode_waves((Hq / Hkv) * q_rows);
    const int64_t slots = (int64_t)kComputeUnits * (D == 128 ? 2 : 1) * (4 / waves);
    const int64_t want = (slots + (int64_t)B * Hkv - 1) / ((int64_t)B * Hkv);
    int cap = max_units / (kMinSegUnits * waves / 4);
    if (cap > kMaxDecodeSeg) cap = kMaxDecodeSeg;
    if (cap < 1) cap = 1;
    int64_t n = want < 1 ? 1 : want;
    p.nseg = (int)(n < cap ? n : cap);
    p.workspace = partial_bytes((size_t)p.nseg * B * Hq * q_rows, D);
    return p;
}

// Block lists: the dense-prefix query blocks are split into key segments of
// max(topk, ceil(NB / 16)) blocks, so that no work item is much longer than a
// sparse query block's list.
inline SplitPlan plan_vsa(int B, int H, int D, int NB, int topk, int dense_prefix)
{
    SplitPlan p;
    p.n_qt = NB;
    const int len = topk > (NB + 15) / 16 ? topk : (NB + 15) / 16;
    p.nseg = (NB + len - 1) / len;
    if (dense_prefix == 0 || p.nseg <= 1) {
        p.nseg = 1;
        p.workspace = 0;
        return p;
    }
    p.workspace = partial_bytes((size_t)p.nseg * B * H * dense_prefix * kTileN, D);
    return p;
}

// Work-item count and XCD slice of a launch; false when out of range.
inline bool set_items(Geometry& g, int64_t items, bool xcd)
{
    if (items <= 0 || items > (int64_t)1 << 30) return false;
    g.n_items = (int)items;
    g.per_xcd = xcd ? (int)((items + 7) / 8) : 0;
    return true;
}

// ---------------------------------------------------------------------------
// Geometry of each launch (host), from the validated shape and its plan.
// Each returns false when the work-item count is out of range.
// ---------------------------------------------------------------------------
inline void clear_geometry(Geometry& g)
{
    g.B = g.Hq = g.Hkv = g.group = g.Lq = g.Lkv = 0;
    g.offset = 0;
    g.n_qt = g.nseg = g.part_lq = g.dense_prefix = g.nqb = g.topk = g.n_items = g.per_xcd = 0;
    g.item_base = g.key_split = 0;
}

// Dense non-causal: one item per (b, h, 128-row query tile).
inline bool dense_geometry(Geometry& g, int B, int H, int Lq, int Lkv)
{
    clear_geometry(g);
    g.B = B;
    g.Hq = g.Hkv = H;
    g.group = 1;
    g.Lq = Lq;
    g.Lkv = Lkv;
    g.n_qt = (Lq + kRowsPerTile - 1) / kRowsPerTile;
    g.nseg = 1;
    return set_items(g, (int64_t)B * H * g.n_qt, true);
}

// Dense D = 128, the last partial round (two workgroups per CU in the main
// rounds). When the items leave at most half a round after the whole ones,
// that rest runs as a launch of its own with 8-wave workgroups, each of whose
// two 4-wave halves streams half of the keys for the same 128 rows (the
// halves' states merge in LDS): two waves per SIMD again, each with half the
// work, instead of a lone 4-wave workgroup per CU streaming every key.
// `main` then covers the whole rounds and `tail` the rest; false (and `tail`
// with no items) when the split does not apply.
inline bool dense_tail_split(const Geometry& all, Geometry& main, Geometry& tail)
{
    tail = all;
    tail.n_items = 0;
    const int64_t slots = (int64_t)kComputeUnits * 2;
    const int64_t rest = all.n_items % slots;
    const int units = (all.Lkv + kTileN - 1) / kTileN;
    if (rest == 0 || rest > slots / 2 || units < 2) return false;
    main = all;
    if (!set_items(main, all.n_items - rest, true)) return false;
    if (!set_items(tail, rest, true)) return false;
    tail.item_base = (int)(all.n_items - rest);
    tail.key_split = seg_units(units, 2) * kTileN;
    return true;
}

// Causal prefill (decode = false: one item per (b, query head, query tile,
// segment)) or decode (one item per (b, kv head, segment), rows packed).
inline bool causal_geometry(Geometry& g, const SplitPlan& p, int B, int Hq, int Hkv, int q_rows, int q_real,
                            int kv_len, bool decode)
{
    clear_geometry(g);
    g.B = B;
    g.Hq = Hq;
    g.Hkv = Hkv;
    g.group = Hq / Hkv;
    g.Lq = q_rows;
    g.Lkv = kv_len;
    g.offset = (int64_t)kv_len - q_real;
    g.n_qt = p.n_qt;
    g.nseg = p.nseg;
    g.part_lq = q_rows;
    const int64_t items = decode ? (int64_t)B * Hkv * p.nseg : (int64_t)B * Hq * p.n_qt * p.nseg;
    return set_items(g, items, true);
}

// Block lists: per (b, h) the dense-prefix query blocks (each in nseg key
// segments), then the sparse query blocks; only the dense-prefix rows (those
// below L) have partial states.
inline bool vsa_geometry(Geometry& g, const SplitPlan& p, int B, int H, int L, int block, int topk,
                         int dense_prefix)
{
    clear_geometry(g);
    const int NB = (L + block - 1) / block;
    g.B = B;
    g.Hq = g.Hkv = H;
    g.group = 1;
    g.Lq = g.Lkv = L;
    g.topk = topk;
    g.dense_prefix = dense_prefix;
    g.nqb = NB;
    g.n_qt = NB;
    g.nseg = p.nseg;
    g.part_lq = dense_prefix * block < L ? dense_prefix * block : L;
    const int64_t per_bh = (int64_t)dense_prefix * p.nseg + (NB - dense_prefix);
    return set_items(g, (int64_t)B * H * per_bh, true);
}

}  // namespace fa
