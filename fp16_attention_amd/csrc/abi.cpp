// C-ABI entry points of libfa16attn.so (declared in include/fa16attn.h).
//
// Each entry point validates every argument on the host before its first HIP
// call, so rejected calls have no side effects and the rejection paths can be
// exercised without a GPU. It then fills the kernel argument block, enqueues
// the kernels on the caller's stream and returns; nothing here allocates
// device memory or synchronises.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "../../include/fa16attn.h"
#include "fa_internal.h"

namespace {

using fa::AttnArgs;

using fa::kDecodeRows;
using fa::kRowsPerTile;
using fa::plan_decode;
using fa::plan_split;
using fa::plan_vsa;
using fa::SplitPlan;

struct Span {
    uintptr_t lo, hi;  // [lo, hi) in bytes
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Address range covered by a [B,H,S,D] strided view of elements of `esize` bytes.
Span span_of(const void* p, int64_t sb, int64_t sh, int64_t ss, int B, int H, int S, int D, int esize)
{
    int64_t last = (int64_t)(B - 1) * sb + (int64_t)(H - 1) * sh + (int64_t)(S - 1) * ss + (D - 1);
    return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)((last + 1) * esize)};
}

Span span_flat(const void* p, int64_t n, int esize)
{
    return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(n * esize)};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

int check_view(const fa_tensor& t)
{
    if (!t.data) return FA_ERR_NULL;
    if (!aligned16(t.data)) return FA_ERR_ALIGN;
    if (t.stride_b < 0 || t.stride_h < 0 || t.stride_s < 0) return FA_ERR_ALIGN;
    if ((t.stride_b % 8) || (t.stride_h % 8) || (t.stride_s % 8)) return FA_ERR_ALIGN;
    return FA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP + (int)e; }

void fill_view(const fa_tensor& t, const _Float16*& p, int64_t& sb, int64_t& sh, int64_t& ss)
{
    p = (const _Float16*)t.data;
    sb = t.stride_b;
    sh = t.stride_h;
    ss = t.stride_s;
}

int check_decode_domain(int B, int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len)
{
    if (D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
    if (B < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (q_rows < 1 || q_rows > 16 || (Hq / Hkv) * q_rows > kDecodeRows) return FA_ERR_SHAPE;
    if (q_real < 1 || q_real > q_rows) return FA_ERR_SHAPE;
    if (kv_len <= q_real || kv_len > 262144 || kv_len % 32 != 0) return FA_ERR_SHAPE;
    return FA_OK;
}

int check_vsa_domain(int B, int H, int L, int D, int block, int topk, int dense_prefix)
{
    if (D != 128 || block != 64) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || L < 1) return FA_ERR_SHAPE;
    const int NB = (L + block - 1) / block;  // the last block may be partial
    if (topk < 1 || topk > NB || dense_prefix < 0 || dense_prefix > NB) return FA_ERR_SHAPE;
    return FA_OK;
}

int check_causal_domain(int B, int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len)
{
    if (D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
    if (B < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (q_rows < 64 || q_rows > 8192 || q_rows % 64 != 0) return FA_ERR_SHAPE;
    if (q_real < 1 || q_real > q_rows) return FA_ERR_SHAPE;
    if (kv_len <= q_real || kv_len > 262144 || kv_len % 32 != 0) return FA_ERR_SHAPE;
    return FA_OK;
}


// Shared body of the causal entry points (prefill and decode).
int run_causal(AttnArgs& a, fa::KvSource src, fa::KeyMode mode, const SplitPlan& p, int D, int q_rows,
               void* workspace, size_t workspace_bytes, hipStream_t stream, const Span* inputs,
               int n_inputs, Span out_span, Span lse_span, const fa::WorkspaceSource* wsrc = nullptr)
{
    if (p.workspace > 0 && wsrc) {
        const int rc = wsrc->get(p.workspace, &workspace, &workspace_bytes);
        if (rc) return rc;
    }
    if (p.workspace > 0) {
        if (!workspace || workspace_bytes < p.workspace) return FA_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
        Span ws = span_flat(workspace, (int64_t)p.workspace, 1);
        for (int i = 0; i < n_inputs; ++i)
            if (overlap(ws, inputs[i])) return FA_ERR_ALIAS;
        if (overlap(ws, out_span) || (a.lse && overlap(ws, lse_span))) return FA_ERR_ALIAS;
    }
    const bool decode = mode == fa::KEYS_DECODE;
    if (!fa::causal_geometry(a, p, a.B, a.Hq, a.Hkv, q_rows, (int)(a.Lkv - a.offset), a.Lkv, decode))
        return FA_ERR_SHAPE;
    const bool split = p.nseg > 1 || decode;
    if (split) {
        size_t o_bytes;
        fa::partial_bytes((size_t)p.nseg * a.B * a.Hq * q_rows, D, &o_bytes);
        a.o_part = (float*)workspace;
        a.ml_part = (float*)((char*)workspace + o_bytes);
    }
    hipError_t e = fa::launch_attn(a, D, src, mode, split, stream);
    if (e != hipSuccess || !split) return hip_status(e);
    fa::MergeArgs m;
    memset(&m, 0, sizeof(m));
    m.o_part = a.o_part;
    m.ml_part = a.ml_part;
    m.o = a.o;
    m.o_sb = a.o_sb;
    m.o_sh = a.o_sh;
    m.o_ss = a.o_ss;
    m.lse = a.lse;
    m.lse_sh = a.Lq;
    m.B = a.B;
    m.Hq = a.Hq;
    m.Lq = a.Lq;
    m.nseg = p.nseg;
    m.n_qt = p.n_qt;
    m.rows_per_tile = decode ? q_rows : kRowsPerTile;
    m.offset = a.offset;
    m.Lkv = a.Lkv;
    m.oscale = a.oscale;
    return hip_status(fa::launch_merge(m, D, stream));
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA16ATTN_ABI_VERSION; }

const char* fa_error_string(int code)
{
    switch (code) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "fa16attn: a required pointer is NULL";
    case FA_ERR_SHAPE: return "fa16attn: a size is outside the supported domain";
    case FA_ERR_UNSUPPORTED: return "fa16attn: unsupported head dimension, page size or block size";
    case FA_ERR_ALIGN: return "fa16attn: bad alignment or stride (D stride 1, 16-byte base, strides multiple of 8)";
    case FA_ERR_WORKSPACE: return "fa16attn: workspace missing or too small";
    case FA_ERR_ALIAS: return "fa16attn: an output overlaps an input or another output";
    default: break;
    }
    if (code > FA_ERR_HIP) return "fa16attn: HIP error during launch (code - 1000 = hipError_t)";
    return "fa16attn: unknown error code";
}

}  // extern "C"

namespace {

// Shared body of the dense entry points (FP16 and BF16 operands).
int run_dense(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse, int B, int H, int Lq, int Lkv,
              int D, float scale, void* stream, fa::KvSource src)
{
    int rc;
    if ((rc = check_view(q)) || (rc = check_view(k)) || (rc = check_view(v)) || (rc = check_view(o)))
        return rc;
    if (D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || Lq < 0 || Lkv < 1) return FA_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SHAPE;
    if (Lq == 0) return FA_OK;
    Span sq = span_of(q.data, q.stride_b, q.stride_h, q.stride_s, B, H, Lq, D, 2);
    Span sk = span_of(k.data, k.stride_b, k.stride_h, k.stride_s, B, H, Lkv, D, 2);
    Span sv = span_of(v.data, v.stride_b, v.stride_h, v.stride_s, B, H, Lkv, D, 2);
    Span so = span_of(o.data, o.stride_b, o.stride_h, o.stride_s, B, H, Lq, D, 2);
    Span sl = lse ? span_flat(lse, (int64_t)B * H * Lq, 4) : Span{0, 0};
    if (overlap(so, sq) || overlap(so, sk) || overlap(so, sv)) return FA_ERR_ALIAS;
    if (lse && (overlap(sl, sq) || overlap(sl, sk) || overlap(sl, sv) || overlap(sl, so)))
        return FA_ERR_ALIAS;

    AttnArgs a;
    memset(&a, 0, sizeof(a));
    fill_view(q, a.q, a.q_sb, a.q_sh, a.q_ss);
    fill_view(k, a.k, a.k_sb, a.k_sh, a.k_ss);
    fill_view(v, a.v, a.v_sb, a.v_sh, a.v_ss);
    a.o = (_Float16*)o.data;
    a.o_sb = o.stride_b;
    a.o_sh = o.stride_h;
    a.o_ss = o.stride_s;
    a.lse = lse;
    if (!fa::dense_geometry(a, B, H, Lq, Lkv)) return FA_ERR_SHAPE;
    a.c = scale * 1.4426950408889634f;
    a.oscale = 1.f;
    AttnArgs whole = a, rest = a;
    if (D == 128 && fa::dense_tail_split(a, whole, rest)) {
        // the whole rounds, then the rest of the items with their keys split
        // between the halves of 8-wave workgroups
        const hipError_t e = fa::launch_attn(whole, D, src, fa::KEYS_DENSE, false, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e);
        return hip_status(fa::launch_dense_halves(rest, src, (hipStream_t)stream));
    }
    return hip_status(fa::launch_attn(a, D, src, fa::KEYS_DENSE, false, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int attn_fwd_dense(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse, int B, int H,
                   int Lq, int Lkv, int D, float scale, void* stream)
{
    return run_dense(q, k, v, o, lse, B, H, Lq, Lkv, D, scale, stream, fa::KV_FP16);
}

int attn_fwd_dense_bf16(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse, int B, int H,
                        int Lq, int Lkv, int D, float scale, void* stream)
{
    return run_dense(q, k, v, o, lse, B, H, Lq, Lkv, D, scale, stream, fa::KV_BF16);
}

size_t attn_fwd_prefix_causal_workspace(int B, int Hq, int Hkv, int D, int q_rows, int kv_len)
{
    if (check_causal_domain(B, Hq, Hkv, D, q_rows, 1, kv_len)) return 0;
    return plan_split(B, Hq, D, q_rows, kv_len).workspace;
}

int attn_fwd_prefix_causal(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse, int B,
                           int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len, float scale,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    int rc;
    if ((rc = check_view(q)) || (rc = check_view(k)) || (rc = check_view(v)) || (rc = check_view(o)))
        return rc;
    if ((rc = check_causal_domain(B, Hq, Hkv, D, q_rows, q_real, kv_len))) return rc;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SHAPE;
    Span in[3] = {span_of(q.data, q.stride_b, q.stride_h, q.stride_s, B, Hq, q_rows, D, 2),
                  span_of(k.data, k.stride_b, k.stride_h, k.stride_s, B, Hkv, kv_len, D, 2),
                  span_of(v.data, v.stride_b, v.stride_h, v.stride_s, B, Hkv, kv_len, D, 2)};
    Span so = span_of(o.data, o.stride_b, o.stride_h, o.stride_s, B, Hq, q_rows, D, 2);
    Span sl = lse ? span_flat(lse, (int64_t)B * Hq * q_rows, 4) : Span{0, 0};
    for (const Span& s : in) {
        if (overlap(so, s)) return FA_ERR_ALIAS;
        if (lse && overlap(sl, s)) return FA_ERR_ALIAS;
    }
    if (lse && overlap(sl, so)) return FA_ERR_ALIAS;

    AttnArgs a;
    memset(&a, 0, sizeof(a));
    fill_view(q, a.q, a.q_sb, a.q_sh, a.q_ss);
    fill_view(k, a.k, a.k_sb, a.k_sh, a.k_ss);
    fill_view(v, a.v, a.v_sb, a.v_sh, a.v_ss);
    a.o = (_Float16*)o.data;
    a.o_sb = o.stride_b;
    a.o_sh = o.stride_h;
    a.o_ss = o.stride_s;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.group = Hq / Hkv;
    a.Lq = q_rows;
    a.Lkv = kv_len;
    a.offset = (int64_t)kv_len - q_real;
    a.c = scale * 1.4426950408889634f;
    a.oscale = 1.f;
    return run_causal(a, fa::KV_FP16, fa::KEYS_CAUSAL, plan_split(B, Hq, D, q_rows, kv_len), D, q_rows,
                      workspace, workspace_bytes, (hipStream_t)stream, in, 3, so, sl);
}

size_t attn_fwd_paged_e4m3_workspace(int B, int Hq, int Hkv, int D, int q_rows, int kv_len)
{
    return attn_fwd_prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len);
}

}  // extern "C"

namespace {

// A k_scale for which every decode(code) * k_scale is an FP16 value: a power
// of two in [2^-15, 2^7].
bool pow2_scale(float k_scale)
{
    int e;
    return frexpf(k_scale, &e) == 0.5f && k_scale >= 0x1p-15f && k_scale <= 128.f;
}

// Bytes of the paged prefill's bridged plan: the split-KV partial states
// (rounded up to 256 bytes), then the FP16 K and V the bridge writes.
size_t bridged_bytes(int B, int Hq, int Hkv, int D, int q_rows, int kv_len, size_t* partial)
{
    *partial = (plan_split(B, Hq, D, q_rows, kv_len).workspace + 255) & ~(size_t)255;
    return *partial + 2 * (size_t)B * Hkv * kv_len * D * sizeof(uint16_t);
}

// Shared body of the paged E4M3 entry points (prefill and decode).
int run_paged(fa_tensor q, const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* page_table,
              int64_t table_stride, int num_phys_pages, int page_size, float k_scale, float v_scale,
              fa_tensor o, float* lse, int B, int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len,
              float scale, void* workspace, size_t workspace_bytes, void* stream, bool decode,
              const fa::WorkspaceSource* wsrc = nullptr)
{
    int rc;
    if ((rc = check_view(q)) || (rc = check_view(o))) return rc;
    if (!k_cache || !v_cache || !page_table) return FA_ERR_NULL;
    if (page_size != 32) return FA_ERR_UNSUPPORTED;
    rc = decode ? check_decode_domain(B, Hq, Hkv, D, q_rows, q_real, kv_len)
                : check_causal_domain(B, Hq, Hkv, D, q_rows, q_real, kv_len);
    if (rc) return rc;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SHAPE;
    if (!(k_scale > 0.f) || !isfinite(k_scale) || !(v_scale > 0.f) || !isfinite(v_scale))
        return FA_ERR_SHAPE;
    if (num_phys_pages < 1 || table_stride < (int64_t)(kv_len / 32)) return FA_ERR_SHAPE;
    if (((uintptr_t)k_cache & 15u) || ((uintptr_t)v_cache & 15u) || ((uintptr_t)page_table & 3u))
        return FA_ERR_ALIGN;
    const int64_t cache_bytes = (int64_t)num_phys_pages * 32 * Hkv * D;
    Span in[4] = {span_of(q.data, q.stride_b, q.stride_h, q.stride_s, B, Hq, q_rows, D, 2),
                  span_flat(k_cache, cache_bytes, 1), span_flat(v_cache, cache_bytes, 1),
                  span_flat(page_table, (int64_t)(B - 1) * table_stride + kv_len / 32, 4)};
    Span so = span_of(o.data, o.stride_b, o.stride_h, o.stride_s, B, Hq, q_rows, D, 2);
    Span sl = lse ? span_flat(lse, (int64_t)B * Hq * q_rows, 4) : Span{0, 0};
    for (const Span& s : in) {
        if (overlap(so, s)) return FA_ERR_ALIAS;
        if (lse && overlap(sl, s)) return FA_ERR_ALIAS;
    }
    if (lse && overlap(sl, so)) return FA_ERR_ALIAS;

    AttnArgs a;
    memset(&a, 0, sizeof(a));
    fill_view(q, a.q, a.q_sb, a.q_sh, a.q_ss);
    a.o = (_Float16*)o.data;
    a.o_sb = o.stride_b;
    a.o_sh = o.stride_h;
    a.o_ss = o.stride_s;
    a.lse = lse;
    a.kc = k_cache;
    a.vc = v_cache;
    a.table = page_table;
    a.table_stride = table_stride;
    a.num_pages = num_phys_pages;
    a.page_shift = 5;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.group = Hq / Hkv;
    a.Lq = q_rows;
    a.Lkv = kv_len;
    a.offset = (int64_t)kv_len - q_real;
    // K is attended as the converted cache's FP16 values RNE16(RNE32(decode *
    // k_scale)). A power-of-two k_scale in [2^-15, 2^7] keeps every such product
    // an exact FP16 value, so the exact decode is used and k_scale folds into the
    // softmax constant; any other k_scale converts each K code tile once per
    // workgroup into an FP16 tile in LDS.
    const bool k_pow2 = pow2_scale(k_scale);
    if (!decode && !k_pow2 && !wsrc) {
        // The bridged plan, when the caller's workspace holds it: the exact
        // bridge converts K and V into FP16 in the workspace, and the FP16
        // causal kernel attends to them (the order of [P4] Implementation;
        // faster than converting K in every workgroup's LDS).
        size_t partial;
        const size_t need = bridged_bytes(B, Hq, Hkv, D, q_rows, kv_len, &partial);
        if (workspace && workspace_bytes >= need && (int64_t)B * Hkv * 2 <= 65535) {
            if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
            Span ws = span_flat(workspace, (int64_t)need, 1);
            for (const Span& s : in)
                if (overlap(ws, s)) return FA_ERR_ALIAS;
            if (overlap(ws, so) || (lse && overlap(ws, sl))) return FA_ERR_ALIAS;
            const int64_t n = (int64_t)B * Hkv * kv_len * D;
            uint16_t* kf = (uint16_t*)((char*)workspace + partial);
            uint16_t* vf = kf + n;
            hipError_t e = fa::launch_e4m3_bridge(k_cache, v_cache, page_table, table_stride, num_phys_pages, B,
                                                  Hkv, D, kv_len, k_scale, v_scale, kf, vf, (hipStream_t)stream);
            if (e != hipSuccess) return hip_status(e);
            a.k = (const _Float16*)kf;
            a.v = (const _Float16*)vf;
            a.k_sb = a.v_sb = (int64_t)Hkv * kv_len * D;
            a.k_sh = a.v_sh = (int64_t)kv_len * D;
            a.k_ss = a.v_ss = D;
            a.c = scale * 1.4426950408889634f;
            a.oscale = 1.f;
            return run_causal(a, fa::KV_FP16, fa::KEYS_CAUSAL, plan_split(B, Hq, D, q_rows, kv_len), D, q_rows,
                              workspace, partial, (hipStream_t)stream, in, 4, so, sl);
        }
    }
    const fa::KvSource src = k_pow2 ? fa::KV_E4M3_PAGED : fa::KV_E4M3_PAGED_SCALED;
    a.c = scale * (k_pow2 ? k_scale : 1.f) * 1.4426950408889634f;
    a.kscale = k_scale;
    a.oscale = v_scale;
    const SplitPlan p = decode ? plan_decode(B, Hq, Hkv, D, q_rows, kv_len) : plan_split(B, Hq, D, q_rows, kv_len);
    return run_causal(a, src, decode ? fa::KEYS_DECODE : fa::KEYS_CAUSAL, p, D, q_rows,
                      workspace, workspace_bytes, (hipStream_t)stream, in, 4, so, sl, wsrc);
}

}  // namespace

int fa::paged_decode_from(const WorkspaceSource* wsrc, const void* q, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                          const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* page_table,
                          int64_t table_stride, int num_phys_pages, int page_size, float k_scale, float v_scale,
                          void* o, int64_t o_sb, int64_t o_sh, int64_t o_ss, float* lse, int B, int Hq, int Hkv,
                          int D, int q_rows, int q_real, int kv_len, float scale, void* stream)
{
    const fa_tensor qt = {(void*)q, q_sb, q_sh, q_ss}, ot = {o, o_sb, o_sh, o_ss};
    return run_paged(qt, k_cache, v_cache, page_table, table_stride, num_phys_pages, page_size, k_scale, v_scale,
                     ot, lse, B, Hq, Hkv, D, q_rows, q_real, kv_len, scale, nullptr, 0, stream, true, wsrc);
}

extern "C" {

int attn_fwd_paged_e4m3(fa_tensor q, const uint8_t* k_cache, const uint8_t* v_cache,
                        const int32_t* page_table, int64_t table_stride, int num_phys_pages,
                        int page_size, float k_scale, float v_scale, fa_tensor o, float* lse, int B,
                        int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len, float scale,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    return run_paged(q, k_cache, v_cache, page_table, table_stride, num_phys_pages, page_size, k_scale, v_scale,
                     o, lse, B, Hq, Hkv, D, q_rows, q_real, kv_len, scale, workspace, workspace_bytes, stream,
                     false);
}

size_t attn_fwd_paged_e4m3_bridged_workspace(int B, int Hq, int Hkv, int D, int q_rows, int kv_len, float k_scale)
{
    if (check_causal_domain(B, Hq, Hkv, D, q_rows, 1, kv_len)) return 0;
    if (!(k_scale > 0.f) || !isfinite(k_scale) || pow2_scale(k_scale))
        return attn_fwd_paged_e4m3_workspace(B, Hq, Hkv, D, q_rows, kv_len);
    size_t partial;
    return bridged_bytes(B, Hq, Hkv, D, q_rows, kv_len, &partial);
}

size_t attn_fwd_paged_e4m3_decode_workspace(int B, int Hq, int Hkv, int D, int q_rows, int kv_len)
{
    if (check_decode_domain(B, Hq, Hkv, D, q_rows, 1, kv_len)) return 0;
    return plan_decode(B, Hq, Hkv, D, q_rows, kv_len).workspace;
}

int attn_fwd_paged_e4m3_decode(fa_tensor q, const uint8_t* k_cache, const uint8_t* v_cache,
                               const int32_t* page_table, int64_t table_stride, int num_phys_pages,
                               int page_size, float k_scale, float v_scale, fa_tensor o, float* lse, int B,
                               int Hq, int Hkv, int D, int q_rows, int q_real, int kv_len, float scale,
                               void* workspace, size_t workspace_bytes, void* stream)
{
    return run_paged(q, k_cache, v_cache, page_table, table_stride, num_phys_pages, page_size, k_scale, v_scale,
                     o, lse, B, Hq, Hkv, D, q_rows, q_real, kv_len, scale, workspace, workspace_bytes, stream,
                     true);
}

int kv_e4m3_paged_to_fp16(const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* page_table,
                          int64_t table_stride, int num_phys_pages, int page_size, int B, int Hkv,
                          int D, int kv_len, float k_scale, float v_scale, uint16_t* k_out,
                          uint16_t* v_out, void* stream)
{
    if (!k_cache || !v_cache || !page_table || !k_out || !v_out) return FA_ERR_NULL;
    if (page_size != 32) return FA_ERR_UNSUPPORTED;
    if (D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
    if (B < 1 || Hkv < 1 || kv_len < 1 || num_phys_pages < 1) return FA_ERR_SHAPE;
    if ((int64_t)B * Hkv * 2 > 65535 || kv_len > (1 << 26)) return FA_ERR_SHAPE;
    if (table_stride < (int64_t)((kv_len + 31) / 32)) return FA_ERR_SHAPE;
    if (!isfinite(k_scale) || !isfinite(v_scale)) return FA_ERR_SHAPE;
    if (((uintptr_t)k_cache & 15u) || ((uintptr_t)v_cache & 15u) || ((uintptr_t)page_table & 3u) ||
        ((uintptr_t)k_out & 15u) || ((uintptr_t)v_out & 15u))
        return FA_ERR_ALIGN;
    const int64_t cache_bytes = (int64_t)num_phys_pages * 32 * Hkv * D;
    const int64_t out_elems = (int64_t)B * Hkv * kv_len * D;
    Span in[3] = {span_flat(k_cache, cache_bytes, 1), span_flat(v_cache, cache_bytes, 1),
                  span_flat(page_table, (int64_t)(B - 1) * table_stride + (kv_len + 31) / 32, 4)};
    Span ko = span_flat(k_out, out_elems, 2), vo = span_flat(v_out, out_elems, 2);
    if (overlap(ko, vo)) return FA_ERR_ALIAS;
    for (const Span& s : in)
        if (overlap(ko, s) || overlap(vo, s)) return FA_ERR_ALIAS;
    return hip_status(fa::launch_e4m3_bridge(k_cache, v_cache, page_table, table_stride,
                                             num_phys_pages, B, Hkv, D, kv_len, k_scale, v_scale,
                                             k_out, v_out, (hipStream_t)stream));
}

int kv_prefix_fp8_gather(const uint16_t* k, const uint16_t* v, int B, int N, int H, int D,
                         const int32_t* index, int rows, uint16_t* k_out, uint16_t* v_out, void* stream)
{
    if (!k || !v || !index || !k_out || !v_out) return FA_ERR_NULL;
    if (D != 128) return FA_ERR_UNSUPPORTED;
    if (B < 1 || N < 1 || H < 1 || rows < 0) return FA_ERR_SHAPE;
    if (rows == 0) return FA_OK;
    if (((uintptr_t)k & 15u) || ((uintptr_t)v & 15u) || ((uintptr_t)k_out & 15u) || ((uintptr_t)v_out & 15u) ||
        ((uintptr_t)index & 3u))
        return FA_ERR_ALIGN;
    const int64_t in_elems = (int64_t)B * N * H * D, out_elems = (int64_t)B * rows * H * D;
    Span in[3] = {span_flat(k, in_elems, 2), span_flat(v, in_elems, 2), span_flat(index, rows, 4)};
    Span out[2] = {span_flat(k_out, out_elems, 2), span_flat(v_out, out_elems, 2)};
    if (overlap(out[0], out[1])) return FA_ERR_ALIAS;
    for (const Span& o : out)
        for (const Span& s : in)
            if (overlap(o, s)) return FA_ERR_ALIAS;
    return hip_status(fa::launch_prefix_fp8_gather(k, v, B, N, H, index, rows, k_out, v_out, (hipStream_t)stream));
}

int vsa_topk_for_sparsity(int L, int block, double sparsity)
{
    if (block < 1 || L < 1 || !(sparsity >= 0.0) || !(sparsity < 1.0)) return -FA_ERR_SHAPE;
    const int NB = (L + block - 1) / block;
    // a product within 1e-9 of an integer is that integer: 1 - 0.7 is not 0.3 in binary
    const double x = (1.0 - sparsity) * NB;
    const double n = nearbyint(x);
    const int keep = fabs(x - n) <= 1e-9 * NB ? (int)n : (int)ceil(x);
    return keep < 1 ? 1 : keep;
}

// Workspace of vsa_block_select: the FP32 pooled means [2][B*H*NB][D], then
// (256-byte aligned) the FP64 block scores [B*H*NB][NB].
static size_t vsa_pooled_bytes(int B, int H, int L, int D)
{
    return (((size_t)2 * B * H * ((L + 63) / 64) * D * 4) + 255) & ~(size_t)255;
}

size_t vsa_block_select_workspace(int B, int H, int L, int D, int block)
{
    if (B < 1 || H < 1 || D != 128 || block != 64 || L < 1 || (L + 63) / 64 > 1024) return 0;
    const size_t nb = (size_t)((L + 63) / 64);
    return vsa_pooled_bytes(B, H, L, D) + (size_t)B * H * nb * nb * 8;
}

int vsa_block_select(const uint16_t* q, const uint16_t* k, int B, int H, int L, int D, int block,
                     int topk, int32_t* idx_out, double* score_out, void* workspace,
                     size_t workspace_bytes, void* stream)
{
    if (!q || !k || !idx_out) return FA_ERR_NULL;
    if (D != 128 || block != 64) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || L < 1) return FA_ERR_SHAPE;
    const int NB = (L + block - 1) / block;  // the last block may be partial
    if (NB > 1024 || topk < 1 || topk > NB) return FA_ERR_SHAPE;
    if (((uintptr_t)q & 15u) || ((uintptr_t)k & 15u) || ((uintptr_t)idx_out & 3u) ||
        ((uintptr_t)score_out & 7u))
        return FA_ERR_ALIGN;
    const size_t need = vsa_block_select_workspace(B, H, L, D, block);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255u) return FA_ERR_ALIGN;
    const int64_t elems = (int64_t)B * H * L * D;
    Span in[2] = {span_flat(q, elems, 2), span_flat(k, elems, 2)};
    Span outs[3] = {span_flat(idx_out, (int64_t)B * H * NB * topk, 4),
                    score_out ? span_flat(score_out, (int64_t)B * H * NB * NB, 8) : Span{0, 0},
                    span_flat(workspace, (int64_t)need, 1)};
    for (int i = 0; i < 3; ++i) {
        for (const Span& s : in)
            if (overlap(outs[i], s)) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_ALIAS;
    }
    double* scores = score_out ? score_out : (double*)((char*)workspace + vsa_pooled_bytes(B, H, L, D));
    return hip_status(fa::launch_vsa_select(q, k, B, H, L, D, topk, idx_out, scores, (float*)workspace,
                                            (hipStream_t)stream));
}

size_t vsa_block_sparse_attn_workspace(int B, int H, int L, int D, int block, int topk,
                                       int dense_prefix_qblocks)
{
    if (check_vsa_domain(B, H, L, D, block, topk, dense_prefix_qblocks)) return 0;
    return plan_vsa(B, H, D, (L + block - 1) / block, topk, dense_prefix_qblocks).workspace;
}

int vsa_block_sparse_attn(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, const int32_t* idx,
                          float* lse, int B, int H, int L, int D, int block, int topk,
                          int dense_prefix_qblocks, float scale, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    int rc;
    if ((rc = check_view(q)) || (rc = check_view(k)) || (rc = check_view(v)) || (rc = check_view(o)))
        return rc;
    if (!idx) return FA_ERR_NULL;
    if ((rc = check_vsa_domain(B, H, L, D, block, topk, dense_prefix_qblocks))) return rc;
    const int NB = (L + block - 1) / block;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SHAPE;
    if ((uintptr_t)idx & 3u) return FA_ERR_ALIGN;
    Span in[4] = {span_of(q.data, q.stride_b, q.stride_h, q.stride_s, B, H, L, D, 2),
                  span_of(k.data, k.stride_b, k.stride_h, k.stride_s, B, H, L, D, 2),
                  span_of(v.data, v.stride_b, v.stride_h, v.stride_s, B, H, L, D, 2),
                  span_flat(idx, (int64_t)B * H * NB * topk, 4)};
    Span so = span_of(o.data, o.stride_b, o.stride_h, o.stride_s, B, H, L, D, 2);
    Span sl = lse ? span_flat(lse, (int64_t)B * H * L, 4) : Span{0, 0};
    for (const Span& s : in) {
        if (overlap(so, s)) return FA_ERR_ALIAS;
        if (lse && overlap(sl, s)) return FA_ERR_ALIAS;
    }
    if (lse && overlap(sl, so)) return FA_ERR_ALIAS;
    const SplitPlan p = plan_vsa(B, H, D, NB, topk, dense_prefix_qblocks);
    if (p.workspace > 0) {
        if (!workspace || workspace_bytes < p.workspace) return FA_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
        Span ws = span_flat(workspace, (int64_t)p.workspace, 1);
        for (const Span& s : in)
            if (overlap(ws, s)) return FA_ERR_ALIAS;
        if (overlap(ws, so) || (lse && overlap(ws, sl))) return FA_ERR_ALIAS;
    }

    AttnArgs a;
    memset(&a, 0, sizeof(a));
    fill_view(q, a.q, a.q_sb, a.q_sh, a.q_ss);
    fill_view(k, a.k, a.k_sb, a.k_sh, a.k_ss);
    fill_view(v, a.v, a.v_sb, a.v_sh, a.v_ss);
    a.o = (_Float16*)o.data;
    a.o_sb = o.stride_b;
    a.o_sh = o.stride_h;
    a.o_ss = o.stride_s;
    a.lse = lse;
    a.idx = idx;
    if (!fa::vsa_geometry(a, p, B, H, L, block, topk, dense_prefix_qblocks)) return FA_ERR_SHAPE;
    a.c = scale * 1.4426950408889634f;
    a.oscale = 1.f;
    const bool split = p.nseg > 1;
    if (split) {
        size_t o_bytes;
        fa::partial_bytes((size_t)p.nseg * B * H * a.part_lq, D, &o_bytes);
        a.o_part = (float*)workspace;
        a.ml_part = (float*)((char*)workspace + o_bytes);
    }
    hipError_t e = fa::launch_attn(a, D, fa::KV_FP16, fa::KEYS_BLOCKS, split, (hipStream_t)stream);
    if (e != hipSuccess || !split) return hip_status(e);
    // the dense-prefix rows: merge the key segments (every key is visible, so
    // the causal offset is set past the last key)
    fa::MergeArgs m;
    memset(&m, 0, sizeof(m));
    m.o_part = a.o_part;
    m.ml_part = a.ml_part;
    m.o = a.o;
    m.o_sb = a.o_sb;
    m.o_sh = a.o_sh;
    m.o_ss = a.o_ss;
    m.lse = lse;
    m.lse_sh = L;
    m.B = B;
    m.Hq = H;
    m.Lq = a.part_lq;
    m.nseg = p.nseg;
    m.n_qt = dense_prefix_qblocks;
    m.rows_per_tile = block;
    m.offset = L;
    m.Lkv = L;
    m.oscale = 1.f;
    return hip_status(fa::launch_merge(m, D, (hipStream_t)stream));
}

int vsa_tile_means(const uint16_t* x, int B, int H, int L, int D, int block, float* out, void* stream)
{
    if (!x || !out) return FA_ERR_NULL;
    if (D != 128 || block != 64) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || L < 1) return FA_ERR_SHAPE;
    if (((uintptr_t)x & 15u) || ((uintptr_t)out & 15u)) return FA_ERR_ALIGN;
    const int64_t NB = (L + block - 1) / block;
    if (overlap(span_flat(x, (int64_t)B * H * L * D, 2), span_flat(out, (int64_t)B * H * NB * D, 4)))
        return FA_ERR_ALIAS;
    return hip_status(fa::launch_vsa_tile_means(x, B, H, L, D, out, (hipStream_t)stream));
}

int vsa_tile_mask_to_block_lists(const uint8_t* mask, const int32_t* valid, int B, int H, int T, int tile,
                                 int32_t* indices, int32_t* counts, int32_t* kv_valid, uint8_t* quadrants,
                                 void* stream)
{
    if (!mask || !valid || !indices || !counts || !kv_valid) return FA_ERR_NULL;
    if (tile != 64 && tile != 128) return FA_ERR_UNSUPPORTED;
    if (quadrants && tile != 64) return FA_ERR_UNSUPPORTED;  // quadrant masks belong to 64-token tiles
    if (B < 1 || H < 1 || T < 1 || T * (tile / 64) > 1024) return FA_ERR_SHAPE;
    if (((uintptr_t)valid & 3u) || ((uintptr_t)indices & 3u) || ((uintptr_t)counts & 3u) ||
        ((uintptr_t)kv_valid & 3u))
        return FA_ERR_ALIGN;
    const int64_t NB = (T * (tile / 64) + 1) / 2;
    const int64_t lists = (int64_t)B * H * NB * NB;
    Span in[2] = {span_flat(mask, (int64_t)B * H * T * T, 1), span_flat(valid, T, 4)};
    Span outs[4] = {span_flat(indices, lists, 4), span_flat(counts, (int64_t)B * H * NB, 4),
                    span_flat(kv_valid, 2 * NB, 4), quadrants ? span_flat(quadrants, lists, 1) : Span{0, 0}};
    for (int i = 0; i < 4; ++i) {
        for (const Span& s : in)
            if (overlap(outs[i], s)) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_ALIAS;
    }
    return hip_status(fa::launch_vsa_block_lists(mask, valid, B, H, T, tile, indices, counts, kv_valid, quadrants,
                                                 (hipStream_t)stream));
}

// Workspace of attn_fwd_prefix_fp8: the E4M3 codes of Q [B,H,Lq,D] and K
// [B,H,Lkv,D] (each 256-byte aligned), then their FP32 row scales.
static size_t fp8_codes_bytes(int64_t rows, int D) { return ((size_t)rows * D + 255) & ~(size_t)255; }
static size_t fp8_scales_bytes(int64_t rows) { return ((size_t)rows * 4 + 255) & ~(size_t)255; }

size_t attn_fwd_prefix_fp8_workspace(int B, int H, int Lq, int Lkv, int D)
{
    if (D != 128 || B < 1 || H < 1 || Lq < 1 || Lkv < 1) return 0;
    const int64_t bh = (int64_t)B * H;
    return fp8_codes_bytes(bh * Lq, D) + fp8_codes_bytes(bh * Lkv, D) + fp8_scales_bytes(bh * Lq) +
           fp8_scales_bytes(bh * Lkv);
}

int attn_fwd_prefix_fp8(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse, int B, int H, int Lq,
                        int Lkv, int D, float scale, void* workspace, size_t workspace_bytes, void* stream)
{
    int rc;
    if ((rc = check_view(q)) || (rc = check_view(k)) || (rc = check_view(v)) || (rc = check_view(o)))
        return rc;
    if (D != 128) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || Lq < 0 || Lkv < 1) return FA_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SHAPE;
    if (Lq == 0) return FA_OK;
    Span in[3] = {span_of(q.data, q.stride_b, q.stride_h, q.stride_s, B, H, Lq, D, 2),
                  span_of(k.data, k.stride_b, k.stride_h, k.stride_s, B, H, Lkv, D, 2),
                  span_of(v.data, v.stride_b, v.stride_h, v.stride_s, B, H, Lkv, D, 2)};
    Span so = span_of(o.data, o.stride_b, o.stride_h, o.stride_s, B, H, Lq, D, 2);
    Span sl = lse ? span_flat(lse, (int64_t)B * H * Lq, 4) : Span{0, 0};
    for (const Span& s : in) {
        if (overlap(so, s)) return FA_ERR_ALIAS;
        if (lse && overlap(sl, s)) return FA_ERR_ALIAS;
    }
    if (lse && overlap(sl, so)) return FA_ERR_ALIAS;
    const size_t need = attn_fwd_prefix_fp8_workspace(B, H, Lq, Lkv, D);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255u) return FA_ERR_ALIGN;
    Span ws = span_flat(workspace, (int64_t)need, 1);
    for (const Span& s : in)
        if (overlap(ws, s)) return FA_ERR_ALIAS;
    if (overlap(ws, so) || (lse && overlap(ws, sl))) return FA_ERR_ALIAS;

    const int64_t bh = (int64_t)B * H;
    uint8_t* qc = (uint8_t*)workspace;
    uint8_t* kc = qc + fp8_codes_bytes(bh * Lq, D);
    float* qsc = (float*)(kc + fp8_codes_bytes(bh * Lkv, D));
    float* ksc = (float*)((char*)qsc + fp8_scales_bytes(bh * Lq));
    hipError_t e = fa::launch_fp8_rows_quantize((const uint16_t*)q.data, q.stride_b, q.stride_h, q.stride_s, B, H, Lq,
                                                qc, qsc, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    e = fa::launch_fp8_rows_quantize((const uint16_t*)k.data, k.stride_b, k.stride_h, k.stride_s, B, H, Lkv, kc, ksc,
                                     (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);

    AttnArgs a;
    memset(&a, 0, sizeof(a));
    fill_view(q, a.q, a.q_sb, a.q_sh, a.q_ss);
    fill_view(k, a.k, a.k_sb, a.k_sh, a.k_ss);
    fill_view(v, a.v, a.v_sb, a.v_sh, a.v_ss);
    a.o = (_Float16*)o.data;
    a.o_sb = o.stride_b;
    a.o_sh = o.stride_h;
    a.o_ss = o.stride_s;
    a.lse = lse;
    a.qc = qc;
    a.qsc = qsc;
    a.kc = kc;
    a.ksc = ksc;
    if (!fa::dense_geometry(a, B, H, Lq, Lkv)) return FA_ERR_SHAPE;
    a.c = scale * 1.4426950408889634f;
    a.oscale = 1.f;
    return hip_status(fa::launch_attn(a, D, fa::KV_FP8QK, fa::KEYS_DENSE, false, (hipStream_t)stream));
}

}  // extern "C"
