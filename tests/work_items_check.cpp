// Host replay of the attention launchers' work items (test infrastructure).
//
// Builds each launch's plan and geometry with the functions the C-ABI layer
// calls, decodes every workgroup's item with the function the kernel calls
// (all from fp16_attention_amd/csrc/work_items.h), and checks that every
// index the kernel derives stays inside the tensors and the workspace, that
// the XCD-aware block -> item map is a bijection, and that the key segments
// of each query tile tile its key range exactly as the merge expects.
//
//   work_items_check dense  B H Lq Lkv D
//   work_items_check causal B Hq Hkv D q_rows q_real kv_len
//   work_items_check decode B Hq Hkv D q_rows q_real kv_len
//   work_items_check blocks B H L D block topk dense_prefix
//   work_items_check dense_tail B H Lq Lkv D   the whole rounds and the split rest
//   [--list]  also print one line per item: b h qt seg key_begin key_stop key_end list empty
//   [--decode-as MODE]  decode the items with another mode's decode (to show
//                       that the checks catch a launcher/kernel mismatch)
//
// Exit status 0 and "OK <items>" when every check passes; 1 and a message
// naming the first failing item otherwise; 2 on bad arguments.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "../fp16_attention_amd/csrc/work_items.h"

using namespace fa;

static int fail(const char* what, int item, const Item& it)
{
    printf("FAIL %s: item %d b=%d h=%d qt=%d seg=%d keys [%d, %d) end %d list=%d empty=%d\n", what, item, it.b,
           it.h, it.qt, it.seg, it.key_begin, it.key_stop, it.key_end, (int)it.list, (int)it.empty);
    return 1;
}

// Dense with the last partial round split: the whole-round launch and the
// rest launch together cover every item of the dense geometry once, each
// launch's block map is a bijection, and the rest's two key halves tile
// [0, Lkv) with the first no shorter than the second (both halves run the
// first's iterations).
static int check_dense_tail(const std::vector<long>& v)
{
    Geometry all, whole, rest;
    if (!dense_geometry(all, (int)v[0], (int)v[1], (int)v[2], (int)v[3])) return printf("FAIL geometry\n"), 1;
    if (!dense_tail_split(all, whole, rest)) return printf("FAIL no split\n"), 1;
    if (whole.n_items % (2 * kComputeUnits) != 0) return printf("FAIL whole rounds\n"), 1;
    std::vector<int> seen(all.n_items, 0);
    for (const Geometry* g : {&whole, &rest}) {
        const int grid = g->per_xcd > 0 ? g->per_xcd * 8 : g->n_items;
        std::vector<int> hit(g->n_items, 0);
        for (int blk = 0; blk < grid; ++blk) {
            const int item = item_of_block(*g, blk);
            if (item < 0) continue;
            if (item >= g->n_items || hit[item]++) return printf("FAIL block map at block %d\n", blk), 1;
            const Item it = decode_item(KEYS_DENSE, *g, item, kRowsPerTile);
            if (it.b < 0 || it.b >= all.B || it.h < 0 || it.h >= all.Hq || it.qt < 0 || it.qt >= all.n_qt)
                return fail("item out of range", item, it);
            if (it.key_begin != 0 || it.key_stop != all.Lkv || it.key_end != all.Lkv)
                return fail("key range", item, it);
            const int idx = (it.b * all.Hq + it.h) * all.n_qt + it.qt;
            if (seen[idx]++) return fail("item decoded twice", item, it);
        }
        for (int i = 0; i < g->n_items; ++i)
            if (!hit[i]) return printf("FAIL item %d has no workgroup\n", i), 1;
    }
    for (int i = 0; i < all.n_items; ++i)
        if (!seen[i]) return printf("FAIL dense item %d not covered\n", i), 1;
    const int ks = rest.key_split;
    if (ks <= 0 || ks >= all.Lkv || ks % kTileN) return printf("FAIL key split %d\n", ks), 1;
    if (all.Lkv - ks > ks) return printf("FAIL second half longer than the first\n"), 1;
    printf("OK %d + %d items, key split %d\n", whole.n_items, rest.n_items, ks);
    return 0;
}

int main(int argc, char** argv)
{
    if (argc < 2) return 2;
    const std::string mode_s = argv[1];
    bool list = false;
    std::string decode_as;
    std::vector<long> v;
    for (int i = 2; i < argc; ++i) {
        if (!strcmp(argv[i], "--list"))
            list = true;
        else if (!strcmp(argv[i], "--decode-as") && i + 1 < argc)
            decode_as = argv[++i];
        else
            v.push_back(atol(argv[i]));
    }
    if (mode_s == "dense_tail" && v.size() == 5) return check_dense_tail(v);
    Geometry g;
    SplitPlan p{0, 1, 0};
    int mode, rows, D;
    if (mode_s == "dense" && v.size() == 5) {
        mode = KEYS_DENSE;
        D = (int)v[4];
        rows = kRowsPerTile;
        if (!dense_geometry(g, (int)v[0], (int)v[1], (int)v[2], (int)v[3])) return printf("FAIL geometry\n"), 1;
    } else if ((mode_s == "causal" || mode_s == "decode") && v.size() == 7) {
        const bool decode = mode_s == "decode";
        mode = decode ? KEYS_DECODE : KEYS_CAUSAL;
        D = (int)v[3];
        // decode: the launcher's workgroup of 1 or 4 waves for the packed rows
        rows = decode ? kRowsPerWave * decode_waves((int)(v[1] / v[2]) * (int)v[4]) : kRowsPerTile;
        p = decode ? plan_decode((int)v[0], (int)v[1], (int)v[2], D, (int)v[4], (int)v[6])
                   : plan_split((int)v[0], (int)v[1], D, (int)v[4], (int)v[6]);
        if (!causal_geometry(g, p, (int)v[0], (int)v[1], (int)v[2], (int)v[4], (int)v[5], (int)v[6], decode))
            return printf("FAIL geometry\n"), 1;
    } else if (mode_s == "blocks" && v.size() == 7) {
        mode = KEYS_BLOCKS;
        D = (int)v[3];
        const int block = (int)v[4];
        rows = block;
        const int NB = ((int)v[2] + block - 1) / block;
        p = plan_vsa((int)v[0], (int)v[1], D, NB, (int)v[5], (int)v[6]);
        if (!vsa_geometry(g, p, (int)v[0], (int)v[1], (int)v[2], block, (int)v[5], (int)v[6]))
            return printf("FAIL geometry\n"), 1;
    } else {
        return 2;
    }
    const bool split = mode == KEYS_DECODE || g.nseg > 1;
    if (!decode_as.empty()) {
        const char* names[] = {"dense", "causal", "blocks", "decode"};
        int m = -1;
        for (int i = 0; i < 4; ++i)
            if (decode_as == names[i]) m = i;
        if (m < 0) return 2;
        mode = m;
    }
    // the workspace rows the launcher lays out: nseg * B * Hq * part_lq
    const size_t ws_rows = split ? (size_t)g.nseg * g.B * g.Hq * g.part_lq : 0;
    if (split && partial_bytes(ws_rows, D) != p.workspace) return printf("FAIL workspace size\n"), 1;

    // block -> item: a bijection onto [0, n_items)
    const int grid = g.per_xcd > 0 ? g.per_xcd * 8 : g.n_items;
    std::vector<int> seen(g.n_items, 0);
    for (int blk = 0; blk < grid; ++blk) {
        const int item = item_of_block(g, blk);
        if (item < 0) continue;
        if (item >= g.n_items || seen[item]++) return printf("FAIL block map at block %d\n", blk), 1;
    }
    for (int i = 0; i < g.n_items; ++i)
        if (!seen[i]) return printf("FAIL item %d has no workgroup\n", i), 1;

    // per query tile: the key ranges its non-empty segments stream
    std::map<long, std::vector<std::pair<int, int>>> ranges;
    std::map<long, int> tile_end;
    for (int item = 0; item < g.n_items; ++item) {
        const Item it = decode_item(mode, g, item, rows);
        if (list)
            printf("%d %d %d %d %d %d %d %d %d\n", it.b, it.h, it.qt, it.seg, it.key_begin, it.key_stop, it.key_end,
                   (int)it.list, (int)it.empty);
        if (it.b < 0 || it.b >= g.B) return fail("batch out of range", item, it);
        if (it.h < 0 || it.h >= g.Hq) return fail("head out of range", item, it);
        if (it.h / g.group >= g.Hkv) return fail("kv head out of range", item, it);
        if (mode == KEYS_DECODE && it.h + g.group > g.Hq) return fail("decode head group", item, it);
        if (it.seg < 0 || it.seg >= g.nseg) return fail("segment out of range", item, it);
        const int n_qt = mode == KEYS_BLOCKS ? g.nqb : g.n_qt;
        if (it.qt < 0 || it.qt >= n_qt) return fail("query tile out of range", item, it);
        const int q0 = it.qt * rows;
        if (q0 >= g.Lq) return fail("query tile past the rows", item, it);
        if (mode == KEYS_DECODE && (g.Lq * g.group > rows)) return fail("decode rows exceed the tile", item, it);
        if (it.list) {
            if (mode != KEYS_BLOCKS || it.qt < g.dense_prefix) return fail("list item", item, it);
            continue;  // keys come from the (clamped) block list
        }
        if (it.empty) continue;
        if (it.key_begin < 0 || it.key_begin >= it.key_stop || it.key_stop > it.key_end || it.key_end > g.Lkv)
            return fail("key range", item, it);
        if (it.key_begin % kTileN) return fail("segment start not unit aligned", item, it);
        // split items write partial rows (seg, b, h, row) for their real rows
        const bool to_part = split && (mode != KEYS_BLOCKS || it.qt < g.dense_prefix);
        if (to_part) {
            // decode rows are (head, position) pairs: positions < Lq of the group's heads
            const int last_row = mode == KEYS_DECODE ? g.Lq - 1 : std::min(q0 + rows, g.Lq) - 1;
            if (last_row >= g.part_lq) return fail("partial row past part_lq", item, it);
            const int bh_last = mode == KEYS_DECODE ? it.b * g.Hq + it.h + g.group - 1 : it.b * g.Hq + it.h;
            const size_t idx = ((size_t)it.seg * g.B * g.Hq + bh_last) * g.part_lq + last_row;
            if (idx >= ws_rows) return fail("partial row past the workspace", item, it);
        }
        const long key = ((long)it.b * g.Hq + it.h) * 100000 + it.qt;
        ranges[key].push_back({it.key_begin, it.key_stop});
        tile_end[key] = it.key_end;
    }
    // the non-empty segments of a tile cover [0, key_end) in order, and the
    // merge (which recomputes the segment count from the tile's key range)
    // reads exactly those
    for (auto& kv : ranges) {
        auto& r = kv.second;
        std::sort(r.begin(), r.end());
        int at = 0;
        for (auto& s : r) {
            if (s.first != at) return printf("FAIL tile %ld: gap or overlap at key %d\n", kv.first, at), 1;
            at = s.second;
        }
        if (at != tile_end[kv.first]) return printf("FAIL tile %ld: keys end at %d\n", kv.first, at), 1;
        if (split) {
            const int nt = (tile_end[kv.first] + kTileN - 1) / kTileN;
            const int su = seg_units(nt, g.nseg);
            const int merged = (nt + su - 1) / su;
            if (merged != (int)r.size())
                return printf("FAIL tile %ld: merge reads %d segments, %zu written\n", kv.first, merged, r.size()), 1;
        }
    }
    printf("OK %d items, %d segments, grid %d\n", g.n_items, g.nseg, grid);
    return 0;
}
