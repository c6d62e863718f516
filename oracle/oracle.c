/*
 * Plain FP64 CPU oracle for the FP16 attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code, header or table with the HIP library.
 *
 * Every function computes the plain definition of its result, one output at a
 * time, in double precision, with no blocking, fusion or reordering beyond what
 * the definition states. Sources (page titles as published):
 *   [P1] "[Kernel] Share SM70 projection, attention and row reduction paths"
 *   [P3] "[Video] Integrate H3 SM70 execution, metrics and VSA diagnostics"
 *   [P4] "[Kernel][SM70] Integrate FP32 v37 prefill and exact E4M3 bridge"
 *   [P5] "[perf] FastH3 two-Spark: gather packed FP4 inputs before head
 *        projections" (a diff; files named where used)
 *
 * Every function here is pinned by tests that do not re-type its formula:
 * closed forms, invariants, library special cases and brute force (see the
 * tests/test_oracle_*.py files).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 (FP16), from the format definition: 1 sign bit, 5        */
/* exponent bits with bias 15, 10 fraction bits, subnormals below 2^-14.      */
/* ------------------------------------------------------------------------ */

double or_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double mag;
    if (e == 31)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, -24);
    else
        mag = ldexp(1024.0 + f, e - 25);
    return s ? -mag : mag;
}

/* bfloat16, from its definition: the upper 16 bits of an IEEE binary32 (1    */
/* sign bit, 8 exponent bits with bias 127, 7 fraction bits). [P5] uses it    */
/* for the BF16 dense attention of the GB10 shape.                            */
double or_bf16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 7) & 255;
    int f = h & 127;
    double mag;
    if (e == 255)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, -133);
    else
        mag = ldexp(128.0 + f, e - 134);
    return s ? -mag : mag;
}

/* Round a double to the nearest FP16 value, ties to even; overflow to inf. */
uint16_t or_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return sign | 0x7E00;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7C00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; rint() rounds half to even */
        double m = rint(ldexp(a, 24));
        return sign | (uint16_t)m; /* m == 1024 gives the smallest normal */
    }
    int E;
    frexp(a, &E);          /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;         /* a in [2^e, 2^(e+1)) */
    double m = rint(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e > 15)
        return sign | 0x7C00;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0);
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN ("float8_e4m3fn", the dtype the [P5] diff stores its FP8    */
/* tensors in): 1 sign bit, 4 exponent bits with bias 7, 3 fraction bits, no  */
/* infinities, NaN only at S.1111.111, largest finite 448. Exponent field 0   */
/* holds subnormals m * 2^-9, the construction the [P5] diff uses in         */
/* minimax_h3_swiglu_quant.cuh (scale_float).                                 */
/* ------------------------------------------------------------------------ */

static double g_e4m3[256];
static pthread_once_t g_e4m3_once = PTHREAD_ONCE_INIT;

static void e4m3_table_init(void)
{
    for (int c = 0; c < 256; ++c) {
        int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
        double v;
        if (e == 15 && m == 7)
            v = NAN;
        else if (e == 0)
            v = ldexp((double)m, -9);
        else
            v = ldexp(1.0 + m / 8.0, e - 7);
        g_e4m3[c] = s ? -v : v;
    }
}

double or_e4m3_decode(uint8_t c)
{
    pthread_once(&g_e4m3_once, e4m3_table_init);
    return g_e4m3[c];
}

/*
 * [P4] "Implementation": exact E4M3 byte conversion to FP16 with unit and
 * non-unit scales. Reading: out = RNE_fp16(RNE_fp32(decode(c) * scale)),
 * i.e. one FP32 multiply then one FP16 conversion, both round-to-nearest-even;
 * FP16 subnormals kept. A NaN code keeps its sign and becomes the FP16 quiet
 * NaN 0x7E00.
 */
uint16_t or_e4m3_to_f16(uint8_t c, float scale)
{
    double d = or_e4m3_decode(c);
    if (isnan(d))
        return (uint16_t)(((c & 0x80) << 8) | 0x7E00);
    volatile float p = (float)d * scale; /* decode(c) is exact in FP32 */
    return or_f64_to_f16((double)p);
}

void or_e4m3_to_f16_array(const uint8_t* c, int64_t n, float scale, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_e4m3_to_f16(c[i], scale);
}

/*
 * The E4M3FN code nearest to a finite float x in [-448, 448], ties to the code
 * with an even mantissa (round to nearest even); the sign of x is kept (a
 * negative value that rounds to zero gives -0). Plain search over the codes of
 * x's sign.
 */
uint8_t or_f32_to_e4m3(float x)
{
    pthread_once(&g_e4m3_once, e4m3_table_init);
    int base = signbit(x) ? 0x80 : 0x00;
    int best = base;
    double err = INFINITY;
    for (int m = 0; m < 127; ++m) { /* 0x7F / 0xFF are NaN */
        double e = fabs(g_e4m3[base + m] - (double)x);
        if (e < err || (e == err && ((base + m) & 1) == 0 && (best & 1) == 1)) {
            best = base + m;
            err = e;
        }
    }
    return (uint8_t)best;
}

/* bfloat16 bits of the value nearest to a finite float, ties to even: the two
   candidates are the truncation and the next bfloat16 away from zero. */
uint16_t or_f32_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t lo = (uint16_t)(u >> 16), hi = (uint16_t)(lo + 1);
    double dlo = or_bf16_to_f64(lo), dhi = or_bf16_to_f64(hi);
    double elo = fabs((double)x - dlo), ehi = isfinite(dhi) ? fabs(dhi - (double)x) : INFINITY;
    if (elo < ehi || (elo == ehi && (lo & 1) == 0))
        return lo;
    return hi;
}

/*
 * FP8 round trip of prefix keys with the valid-row gather ([P5]
 * prefix_quant.py, quantize_gather_prefix_kv). k, v: bfloat16 [B, N, H, D]
 * contiguous; index: the `rows` source tokens. For every (b, r, h), with x
 * the FP32 values of K's row index[r], head h:
 *   scale = max |x| / 448 (FP32), inv = scale == 0 ? 0 : 1 / scale,
 *   ko = RNE_bf16( decode( RNE_e4m3( clamp(x * inv, +-448) ) ) * scale ),
 * each operation rounding once in FP32; vo is V's row copied. Outputs are
 * [B, rows, H, D] bfloat16.
 */
/* The per-row E4M3 quantization of the round trip: x holds D bfloat16 values;
 * scale = max |x| / 448 (FP32), inv = scale == 0 ? 0 : 1 / scale,
 * codes[d] = RNE_e4m3(clamp(x[d] * inv, +-448)), each step rounding once in
 * FP32. Returns scale. */
static float or_fp8_row(const uint16_t* x, int D, uint8_t* codes)
{
    volatile float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
        float a = fabsf((float)or_bf16_to_f64(x[d]));
        if (a > amax)
            amax = a;
    }
    volatile float scale = amax / 448.0f;
    volatile float inv = scale == 0.0f ? 0.0f : 1.0f / scale;
    for (int d = 0; d < D; ++d) {
        volatile float y = (float)or_bf16_to_f64(x[d]) * inv;
        float c = y < -448.0f ? -448.0f : (y > 448.0f ? 448.0f : y);
        codes[d] = or_f32_to_e4m3(c);
    }
    return scale;
}

void or_prefix_fp8_gather(const uint16_t* k, const uint16_t* v, int B, int N, int H, int D,
                          const int32_t* index, int rows, uint16_t* ko, uint16_t* vo)
{
    uint8_t* codes = (uint8_t*)malloc((size_t)D);
    for (int b = 0; b < B; ++b)
        for (int r = 0; r < rows; ++r)
            for (int h = 0; h < H; ++h) {
                const int64_t src = (((int64_t)b * N + index[r]) * H + h) * D;
                const int64_t dst = (((int64_t)b * rows + r) * H + h) * D;
                const float scale = or_fp8_row(k + src, D, codes);
                for (int d = 0; d < D; ++d) {
                    volatile float y = (float)or_e4m3_decode(codes[d]) * scale;
                    ko[dst + d] = or_f32_to_bf16(y);
                    vo[dst + d] = v[src + d];
                }
            }
    free(codes);
}

/*
 * E4M3 quantization of rows of D bfloat16 values with a per-row amax / 448
 * scale ([P5] query_pool.py, the PREFIX_FP8 round trip of the prefix
 * queries; prefix_quant.py, the same for the prefix keys): codes [rows][D]
 * and scales [rows], the steps of or_fp8_row.
 */
void or_fp8_quantize_rows(const uint16_t* x, int64_t rows, int D, uint8_t* codes, float* scales)
{
    for (int64_t r = 0; r < rows; ++r)
        scales[r] = or_fp8_row(x + r * D, D, codes + r * D);
}

/*
 * Paged cache gather (reading of [P4] "Implementation", paged E4M3 KV):
 * cache [num_pages, page_size, Hkv, D] bytes, table [B, pages_per_seq] int32,
 * logical token t of sequence b lives in page table[b][t / page_size], slot
 * t % page_size. Output is the contiguous [B, Hkv, kv_len, D] byte tensor.
 * Returns -1 on an out-of-range page id.
 */
int or_paged_gather(const uint8_t* cache, int64_t num_pages, int page_size, const int32_t* table,
                    int64_t table_stride, int B, int Hkv, int D, int64_t kv_len, uint8_t* out)
{
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g)
            for (int64_t t = 0; t < kv_len; ++t) {
                int32_t page = table[(int64_t)b * table_stride + t / page_size];
                if (page < 0 || page >= num_pages)
                    return -1;
                const uint8_t* src =
                    cache + (((int64_t)page * page_size + t % page_size) * Hkv + g) * D;
                memcpy(out + (((int64_t)b * Hkv + g) * kv_len + t) * D, src, (size_t)D);
            }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Scaled dot-product attention, FP64, one query row at a time.              */
/*                                                                            */
/*   s_j  = scale * sum_d q_d k_jd        over the keys j the row may see     */
/*   m    = max_j s_j                                                         */
/*   o    = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m)                       */
/*   lse  = m + ln sum_j exp(s_j - m)                                         */
/*                                                                            */
/* Key sets ([P4] "Implementation" for the causal prefill, [P3] "Purpose"     */
/* for the VSA top-k with prefix-dense queries):                              */
/*   mode 0  dense: all j < Lkv                                               */
/*   mode 1  causal with offset: j <= offset + i, offset = kv_len - q_real,   */
/*           the same rule for padded rows i >= q_real                        */
/*   mode 2  block list: query block bq = i / block; bq < dense_prefix sees   */
/*           all keys, otherwise the keys (below Lkv: the last block may be   */
/*           partial) of blocks idx[b][h][bq][0..topk)                        */
/* GQA: query head h reads kv head h / (Hq / Hkv).                            */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void* q;
    const void* k;
    const void* v;
    int64_t qs[3], ks[3], vs[3]; /* element strides (batch, head, row); D stride 1 */
    int B, Hq, Hkv, Lq, Lkv, D;
    double scale;
    int mode;
    int64_t offset;
    const int32_t* idx; /* [B, Hq, Lq/block, topk] */
    int block, topk, dense_prefix;
    const int32_t* rows; /* n_rows triples (b, h, i) */
    int64_t n_rows;
    double* out; /* [n_rows, D] */
    double* lse; /* [n_rows] */
    int fmt; /* q, k, v element format: 0 FP16, 1 BF16, 2 FP64 */
    int64_t next;
    pthread_mutex_t lock;
} attn_job;

/* element i (an element offset) of an operand in the job's format */
static double elem(const attn_job* J, const void* base, int64_t i)
{
    if (J->fmt == 2)
        return ((const double*)base)[i];
    const uint16_t h = ((const uint16_t*)base)[i];
    return J->fmt == 1 ? or_bf16_to_f64(h) : or_f16_to_f64(h);
}

static int64_t claim(attn_job* J)
{
    pthread_mutex_lock(&J->lock);
    int64_t r = J->next++;
    pthread_mutex_unlock(&J->lock);
    return r;
}

static int64_t keys_of_row(const attn_job* J, int b, int h, int i, int64_t* keys)
{
    int64_t n = 0;
    if (J->mode == 0) {
        for (int64_t j = 0; j < J->Lkv; ++j)
            keys[n++] = j;
    } else if (J->mode == 1) {
        int64_t last = J->offset + i;
        for (int64_t j = 0; j < J->Lkv && j <= last; ++j)
            keys[n++] = j;
    } else {
        int bq = i / J->block;
        if (bq < J->dense_prefix) {
            for (int64_t j = 0; j < J->Lkv; ++j)
                keys[n++] = j;
        } else {
            int nqb = (J->Lq + J->block - 1) / J->block;
            const int32_t* list = J->idx + (((int64_t)b * J->Hq + h) * nqb + bq) * J->topk;
            for (int t = 0; t < J->topk; ++t)
                for (int u = 0; u < J->block; ++u) {
                    int64_t j = (int64_t)list[t] * J->block + u;
                    if (j < J->Lkv) /* the last block may be partial */
                        keys[n++] = j;
                }
        }
    }
    return n;
}

static void* attn_worker(void* arg)
{
    attn_job* J = (attn_job*)arg;
    int D = J->D;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(J->Lkv > 0 ? J->Lkv : 1));
    double* s = (double*)malloc(sizeof(double) * (size_t)(J->Lkv > 0 ? J->Lkv : 1));
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    int group = J->Hq / J->Hkv;
    for (;;) {
        int64_t r = claim(J);
        if (r >= J->n_rows)
            break;
        int b = J->rows[3 * r], h = J->rows[3 * r + 1], i = J->rows[3 * r + 2];
        int g = h / group;
        const int64_t qrow = b * J->qs[0] + h * J->qs[1] + (int64_t)i * J->qs[2];
        for (int d = 0; d < D; ++d)
            qd[d] = elem(J, J->q, qrow + d);
        int64_t n = keys_of_row(J, b, h, i, keys);
        double m = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
            const int64_t krow = b * J->ks[0] + g * J->ks[1] + keys[t] * J->ks[2];
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += qd[d] * elem(J, J->k, krow + d);
            s[t] = J->scale * dot;
            if (s[t] > m)
                m = s[t];
        }
        double denom = 0.0;
        for (int d = 0; d < D; ++d)
            acc[d] = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            double p = exp(s[t] - m);
            denom += p;
            const int64_t vrow = b * J->vs[0] + g * J->vs[1] + keys[t] * J->vs[2];
            for (int d = 0; d < D; ++d)
                acc[d] += p * elem(J, J->v, vrow + d);
        }
        for (int d = 0; d < D; ++d)
            J->out[r * D + d] = acc[d] / denom;
        J->lse[r] = m + log(denom);
    }
    free(keys);
    free(s);
    free(qd);
    free(acc);
    return NULL;
}

/* Returns 0, or -1 for an invalid argument. fmt: the element format of q, k
   and v: 0 FP16, 1 bfloat16 (both as 16-bit patterns), 2 FP64 values. */
int or_attention(const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                 const void* v, const int64_t* vs, int B, int Hq, int Hkv, int Lq, int Lkv,
                 int D, double scale, int mode, int64_t offset, const int32_t* idx, int block,
                 int topk, int dense_prefix, const int32_t* rows, int64_t n_rows, double* out,
                 double* lse, int threads, int fmt)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || (mode == 2 && (block <= 0 || !idx)))
        return -1;
    attn_job J;
    memset(&J, 0, sizeof(J));
    J.q = q;
    J.k = k;
    J.v = v;
    memcpy(J.qs, qs, sizeof(J.qs));
    memcpy(J.ks, ks, sizeof(J.ks));
    memcpy(J.vs, vs, sizeof(J.vs));
    J.B = B;
    J.Hq = Hq;
    J.Hkv = Hkv;
    J.Lq = Lq;
    J.Lkv = Lkv;
    J.D = D;
    J.scale = scale;
    J.mode = mode;
    J.offset = offset;
    J.idx = idx;
    J.block = block;
    J.topk = topk;
    J.dense_prefix = dense_prefix;
    J.rows = rows;
    J.n_rows = n_rows;
    J.out = out;
    J.lse = lse;
    if (fmt < 0 || fmt > 2)
        return -1;
    J.fmt = fmt;
    J.next = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (threads < 1)
        threads = 1;
    pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
    for (int t = 0; t < threads; ++t)
        pthread_create(&tid[t], NULL, attn_worker, &J);
    for (int t = 0; t < threads; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    pthread_mutex_destroy(&J.lock);
    return 0;
}

/*
 * Merge of partial softmax states over disjoint key segments ([P4]
 * "Implementation": FP32 prefix/tail state and a final merge). Segment s holds
 * (m_s, l_s, o_s) with o_s already normalised by l_s. With M = max m_s:
 *   o = sum_s e^(m_s - M) l_s o_s / sum_s e^(m_s - M) l_s,
 *   lse = M + ln sum_s e^(m_s - M) l_s.
 */
void or_merge(int nseg, int D, const double* m, const double* l, const double* o, double* out,
              double* lse)
{
    double M = -INFINITY;
    for (int s = 0; s < nseg; ++s)
        if (m[s] > M)
            M = m[s];
    double denom = 0.0;
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    for (int s = 0; s < nseg; ++s) {
        double w = exp(m[s] - M) * l[s];
        denom += w;
        for (int d = 0; d < D; ++d)
            out[d] += w * o[(int64_t)s * D + d];
    }
    for (int d = 0; d < D; ++d)
        out[d] /= denom;
    *lse = M + log(denom);
}

/* ------------------------------------------------------------------------ */
/* VSA block selection ([P3] "Purpose": top-k = 64 KV blocks per query block, */
/* prefix-dense queries; [P5] key_quant.py / query_pool.py: tile means are    */
/* the tile sum divided by the valid count with one rounding, stored FP32).   */
/* ------------------------------------------------------------------------ */

/* The FP32 value nearest to sum / count (ties to even), for an exact FP64 sum
 * of FP16 values and 1 <= count <= 1024: the FP64 quotient is within one FP32
 * step of it, and each neighbour's distance |c * count - sum| is computed
 * exactly (24-bit c times an 11-bit count fits in 53 bits). */
static float or_div_rn_f32(double sum, int count)
{
    float best = (float)(sum / count);
    double err = fabs((double)best * count - sum);
    float nb[2] = {nextafterf(best, -INFINITY), nextafterf(best, INFINITY)};
    for (int i = 0; i < 2; ++i) {
        double e = fabs((double)nb[i] * count - sum);
        uint32_t u;
        memcpy(&u, &nb[i], 4);
        if (e < err || (e == err && (u & 1u) == 0)) {
            best = nb[i];
            err = e;
        }
    }
    return best;
}

/* x [B,H,L,D] FP16 contiguous -> out [B,H,ceil(L/block),D] FP32: the sum of the
 * block's valid rows (the last block may be partial) divided by their count,
 * rounded once. The FP64 sum of <= 2^10 FP16 values is exact (all are multiples
 * of 2^-24 below 2^16), so the order of the sum does not matter. */
void or_vsa_pool(const uint16_t* x, int B, int H, int L, int D, int block, float* out)
{
    int nb = (L + block - 1) / block;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < nb; ++t) {
                int count = L - t * block < block ? L - t * block : block;
                for (int d = 0; d < D; ++d) {
                    double sum = 0.0;
                    for (int u = 0; u < count; ++u)
                        sum += or_f16_to_f64(
                            x[(((int64_t)b * H + h) * L + (int64_t)t * block + u) * D + d]);
                    out[(((int64_t)b * H + h) * nb + t) * D + d] = or_div_rn_f32(sum, count);
                }
            }
}

/* s[b,h,i,j] = sum_{d ascending} qbar[b,h,i,d] * kbar[b,h,j,d] in FP64. Each
 * product of two FP32 values is exact in FP64; the sums round in this order. */
void or_vsa_scores(const float* qbar, const float* kbar, int B, int H, int NB, int D, double* s)
{
    for (int bh = 0; bh < B * H; ++bh)
        for (int i = 0; i < NB; ++i)
            for (int j = 0; j < NB; ++j) {
                const float* a = qbar + ((int64_t)bh * NB + i) * D;
                const float* c = kbar + ((int64_t)bh * NB + j) * D;
                double acc = 0.0;
                for (int d = 0; d < D; ++d)
                    acc += (double)a[d] * (double)c[d];
                s[((int64_t)bh * NB + i) * NB + j] = acc;
            }
}

/* Per row: the topk blocks with the largest score, equal scores ranked by the
 * lower block index; the kept indices are written in ascending order. Plain
 * selection: repeatedly take the best block not yet taken. */
void or_vsa_topk(const double* s, int B, int H, int NB, int topk, int32_t* idx)
{
    char* taken = (char*)malloc((size_t)NB);
    for (int64_t row = 0; row < (int64_t)B * H * NB; ++row) {
        const double* sr = s + row * NB;
        memset(taken, 0, (size_t)NB);
        for (int t = 0; t < topk; ++t) {
            int best = -1;
            for (int j = 0; j < NB; ++j) {
                if (taken[j])
                    continue;
                if (best < 0 || sr[j] > sr[best])
                    best = j; /* strict '>' keeps the lower index on ties */
            }
            taken[best] = 1;
        }
        int n = 0;
        for (int j = 0; j < NB; ++j)
            if (taken[j])
                idx[row * topk + n++] = j;
    }
    free(taken);
}

/* ------------------------------------------------------------------------ */
/* VSA block lists of 128-token blocks ([P5] block_lists.py,                */
/* tile_mask_to_fp4_blocks: the native kernel's descending block lists).     */
/*                                                                            */
/* Inputs: a square tile mask mask[b][h][i][j] (1 byte per entry; nonzero =   */
/* query tile i attends to key tile j) over T tiles of `tile` = 64 * HT      */
/* tokens, and valid[t], the valid tokens of tile t. The sequence is cut into */
/* 64-token halves (HT per tile, T * HT in all), and two consecutive halves   */
/* form one of NB = ceil(T * HT / 2) blocks. For query block r (halves        */
/* q0 = 2r, q1 = 2r + 1) and key block c (halves a = 2c, e = 2c + 1):         */
/*   va = clamp(valid[a / HT] - (a % HT) * 64, 0, 64), ve likewise, and 0     */
/*        for a half past the sequence;                                       */
/*   m(q, k) = mask[q / HT][k / HT] for halves inside the sequence, else 0;   */
/*   a query half q1 past the sequence (an odd count of halves) sees key     */
/*   half 0 only: m(q1, k) = (k == 0);                                        */
/*   quad = [m(q0,a) & va>0] + 2 [m(q0,e) & ve>0] + 4 [m(q1,a) & va>0]        */
/*          + 8 [m(q1,e) & ve>0].                                             */
/* Outputs per (b, h, r): idx[..][0..n) = the key blocks c with quad != 0 in */
/* descending order, idx[..][n..NB) = 0; quad_out likewise (its quad values); */
/* counts = n. kv_valid[2c], kv_valid[2c+1] = va, ve (one vector for all     */
/* (b, h)). quad_out may be NULL.                                             */
/* ------------------------------------------------------------------------ */
static int or_half_valid(const int32_t* valid, int T, int HT, int half)
{
    if (half >= T * HT)
        return 0;
    int v = valid[half / HT] - (half % HT) * 64;
    return v < 0 ? 0 : (v > 64 ? 64 : v);
}

static int or_half_mask(const uint8_t* m, int T, int HT, int qh, int kh)
{
    if (qh >= T * HT)
        return kh == 0; /* the padded odd query half sees key half 0 only */
    if (kh >= T * HT)
        return 0;
    return m[(int64_t)(qh / HT) * T + kh / HT] != 0;
}

void or_block_lists(const uint8_t* mask, const int32_t* valid, int B, int H, int T, int tile, int32_t* idx,
                    int32_t* counts, int32_t* kv_valid, uint8_t* quad_out)
{
    const int HT = tile / 64;
    const int NB = (T * HT + 1) / 2;
    for (int c = 0; c < NB; ++c) {
        kv_valid[2 * c] = or_half_valid(valid, T, HT, 2 * c);
        kv_valid[2 * c + 1] = or_half_valid(valid, T, HT, 2 * c + 1);
    }
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const uint8_t* m = mask + ((int64_t)b * H + h) * T * T;
            for (int r = 0; r < NB; ++r) {
                int32_t* list = idx + (((int64_t)b * H + h) * NB + r) * NB;
                uint8_t* ql = quad_out ? quad_out + (((int64_t)b * H + h) * NB + r) * NB : NULL;
                int n = 0;
                for (int c = NB - 1; c >= 0; --c) {
                    const int a = 2 * c, e = 2 * c + 1;
                    const int va = kv_valid[a] > 0, ve = kv_valid[e] > 0;
                    const int q0 = 2 * r, q1 = 2 * r + 1;
                    const int bits = (or_half_mask(m, T, HT, q0, a) && va) + 2 * (or_half_mask(m, T, HT, q0, e) && ve) +
                                     4 * (or_half_mask(m, T, HT, q1, a) && va) +
                                     8 * (or_half_mask(m, T, HT, q1, e) && ve);
                    if (bits) {
                        list[n] = c;
                        if (ql)
                            ql[n] = (uint8_t)bits;
                        ++n;
                    }
                }
                for (int t = n; t < NB; ++t) {
                    list[t] = 0;
                    if (ql)
                        ql[t] = 0;
                }
                counts[((int64_t)b * H + h) * NB + r] = n;
            }
        }
}
