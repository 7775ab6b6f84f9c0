/*
 * oracle.c -- the exact-attention ORACLE: a plain, slow, obviously correct
 * CPU implementation in fp64 of what the GPU path computes.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the package's smoke
 * check and the benchmark's CPU-baseline leg may load or call it.  The GPU
 * library shares no code with it: no header, helper, table or constant
 * generator is common to the two, and neither includes the other.
 *
 * Sources (web pages, cited by title and section):
 *   [SD]  "FlashAttention CUDA 커널 한 줄씩 살펴보기" (Korean translation of
 *         Stephen Diehl's line-by-line FlashAttention kernel walkthrough,
 *         yeokja.moreal.dev)
 *   [SU]  "Flash Attention" (suniverse77.github.io), sections "Standard
 *         Attention" and "Online Softmax", Eq. (1)-(4)
 *   [FX]  "FlashAttention原理与CUDA实现" (fxlin0261.github.io), the
 *         FlashAttention-2-order kernel listing
 *   [YJ]  "FlashAttention: GPU 메모리 계층을 활용한 어텐션 최적화 분석"
 *         (youngju.dev), sections 2.1, 5.1-5.2, 6.1-6.3, 7.2, 8.1-8.3, 11.3
 *   [PA]  "PagedAttention" (data-sketchers.com wiki, vLLM kernel
 *         walkthrough), sections "Concepts", "Key", "Softmax", "Value",
 *         "Output"
 *
 * Conventions fixed here (the pages leave them open):
 *   - Inputs are read from their storage type (fp32, bf16, fp16, fp64) and
 *     widened exactly to fp64 by decoding the bit patterns from the IEEE 754
 *     binary16 / bfloat16 definitions.
 *   - Every sum runs in ascending index order; libm exp/log in fp64.
 *   - lse is the natural log-sum-exp of the scaled, masked scores:
 *     lse_i = m_i + ln(l_i).
 *   - Causal mask: query row i sees keys j <= i (top-left aligned square
 *     mask, the "is_causal" / lower-triangular mask of [YJ] 11.3).
 *   - A row with no admissible key (cannot happen for the masks above) gets
 *     O = 0 and lse = -inf.
 *
 * Build (no -ffast-math, so sums stay sequential and exp/log stay libm):
 *   gcc -O2 -std=c11 -fPIC -shared -pthread oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2, OR_F64 = 3 };

/* ------------------------------------------------------------------ */
/* exact widening of storage types to fp64                              */
/* ------------------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Normal: (1 + f/1024) * 2^(e-15); subnormal: f/1024 * 2^-14. */
static double or_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25);
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32 bit pattern. */
static double or_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double or_load(const void *base, int dtype, int64_t i)
{
    switch (dtype) {
    case OR_F32: return (double)((const float *)base)[i];
    case OR_BF16: return or_bf16_to_double(((const uint16_t *)base)[i]);
    case OR_F16: return or_half_to_double(((const uint16_t *)base)[i]);
    default: return ((const double *)base)[i];
    }
}

static int or_elem_bytes(int dtype)
{
    switch (dtype) {
    case OR_F32: return 4;
    case OR_BF16: case OR_F16: return 2;
    case OR_F64: return 8;
    default: return 0;
    }
}

/* Exported so that tests can pin the decoders against library conversions. */
int oracle_widen(const void *src, int dtype, int64_t n, double *dst)
{
    if (or_elem_bytes(dtype) == 0) return -1;
    for (int64_t i = 0; i < n; ++i) dst[i] = or_load(src, dtype, i);
    return 0;
}

/* ------------------------------------------------------------------ */
/* thread pool helper: static partition of [0, n) over T threads        */
/* ------------------------------------------------------------------ */

typedef void (*or_item_fn)(void *ctx, int64_t item, double *scratch);

typedef struct {
    or_item_fn fn;
    void *ctx;
    int64_t begin, end;
    int64_t scratch_len;
    int status;
} or_job;

static void *or_run_job(void *arg)
{
    or_job *job = (or_job *)arg;
    double *scratch = NULL;
    if (job->scratch_len > 0) {
        scratch = (double *)malloc((size_t)job->scratch_len * sizeof(double));
        if (!scratch) { job->status = -1; return NULL; }
    }
    for (int64_t it = job->begin; it < job->end; ++it) job->fn(job->ctx, it, scratch);
    free(scratch);
    job->status = 0;
    return NULL;
}

static int or_parallel(or_item_fn fn, void *ctx, int64_t n, int64_t scratch_len, int nthreads)
{
    if (n <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)n;
    or_job jobs[256];
    pthread_t tids[256];
    int64_t chunk = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = (int64_t)t * chunk < n ? (int64_t)t * chunk : n;
        jobs[t].end = (int64_t)(t + 1) * chunk < n ? (int64_t)(t + 1) * chunk : n;
        jobs[t].scratch_len = scratch_len;
        jobs[t].status = -1;
    }
    if (nthreads == 1) {
        or_run_job(&jobs[0]);
        return jobs[0].status;
    }
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, or_run_job, &jobs[t]) != 0) break;
        ++started;
    }
    for (int t = 0; t < started; ++t) pthread_join(tids[t], NULL);
    if (started < nthreads) {
        for (int t = started; t < nthreads; ++t) or_run_job(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status != 0) return -1;
    return 0;
}

/* ------------------------------------------------------------------ */
/* One softmax row, the plain definition                                */
/* ------------------------------------------------------------------ */

/*
 * Given n scores s[0..n) (already scaled and restricted to admissible keys),
 * value rows v_of(j)[0..d) and output o[0..d):
 *     m = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j,
 *     o_c = (sum_j p_j v_jc) / l,  return lse = m + ln l.
 * This is the safe softmax of [SU] Eq. (1) ([YJ] 6.1, [PA] "Softmax")
 * followed by O = PV ([SU] "Standard Attention", [YJ] 2.1).
 * s is overwritten with p.
 */
typedef double (*or_value_fn)(const void *ctx, int64_t j, int c);

static double or_softmax_row(double *s, int64_t n, int d, or_value_fn vfn, const void *vctx,
                             double *o)
{
    if (n <= 0) {
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        return -INFINITY;
    }
    double m = s[0];
    for (int64_t j = 1; j < n; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j) acc += s[j] * vfn(vctx, j, c);
        o[c] = acc / l;
    }
    return m + log(l);
}

/* ------------------------------------------------------------------ */
/* Dense attention forward                                              */
/* ------------------------------------------------------------------ */

typedef struct {
    const void *q, *k, *v;
    int dtype;
    int B, H, Hkv, N, d;
    double scale;
    int causal;
    const int64_t *rows;
    int64_t nrows;
    double *o, *lse;
    /* per-item value accessor context */
} or_fwd_ctx;

typedef struct {
    const void *v;
    int dtype;
    int64_t base; /* element offset of V[b,h,0,0] */
    int d;
} or_dense_v;

static double or_dense_value(const void *ctx, int64_t j, int c)
{
    const or_dense_v *dv = (const or_dense_v *)ctx;
    return or_load(dv->v, dv->dtype, dv->base + j * dv->d + c);
}

static void or_fwd_item(void *vctx, int64_t item, double *s)
{
    const or_fwd_ctx *x = (const or_fwd_ctx *)vctx;
    int64_t r = item % x->nrows;
    int64_t bh = item / x->nrows;
    int64_t i = x->rows ? x->rows[r] : r;
    int64_t base = bh * (int64_t)x->N * x->d; /* Q: [B,H,N,d] contiguous */
    /* K, V: [B,Hkv,N,d]; query head h reads kv head h / (H / Hkv) */
    int64_t b = bh / x->H, h = bh % x->H;
    int64_t kvbase = (b * x->Hkv + h / (x->H / x->Hkv)) * (int64_t)x->N * x->d;
    /* admissible keys A_i = { j < N : not causal or j <= i } */
    int64_t n = x->causal ? (i + 1 < x->N ? i + 1 : x->N) : x->N;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int c = 0; c < x->d; ++c)
            dot += or_load(x->q, x->dtype, base + i * x->d + c) *
                   or_load(x->k, x->dtype, kvbase + j * x->d + c);
        s[j] = x->scale * dot;
    }
    or_dense_v dv = { x->v, x->dtype, kvbase, x->d };
    double *o = x->o + item * x->d;
    x->lse[item] = or_softmax_row(s, n, x->d, or_dense_value, &dv, o);
}

/*
 * O = softmax(scale * Q K^T [+ causal mask]) V for every (b, h) and every
 * selected query row, with Q laid out [B, H, N, d] and K, V [B, Hkv, N, d]
 * contiguous; query head h attends with kv head h / (H / Hkv) (Hkv = H:
 * multi-head attention; grouped query heads as in the num_kv_heads of
 * [PA] "Concepts").
 *   rows  : query indices to evaluate (the same for every (b, h)); NULL
 *           means all N rows, in order.
 *   o     : [B, H, nrows, d] fp64;  lse : [B, H, nrows] fp64.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attention(const void *q, const void *k, const void *v, int dtype, int B, int H, int Hkv,
                     int N, int d, double scale, int causal, const int64_t *rows, int64_t nrows,
                     double *o, double *lse, int nthreads)
{
    if (!q || !k || !v || !o || !lse || B < 1 || H < 1 || N < 1 || d < 1) return -1;
    if (Hkv < 1 || H % Hkv != 0) return -1;
    if (or_elem_bytes(dtype) == 0) return -1;
    if (!rows) nrows = N;
    if (nrows < 1) return -1;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return -1;
    or_fwd_ctx ctx = { q, k, v, dtype, B, H, Hkv, N, d, scale, causal, rows, nrows, o, lse };
    return or_parallel(or_fwd_item, &ctx, (int64_t)B * H * nrows, N, nthreads);
}

/*
 * The full probability matrix P = softmax(scale * Q K^T [+ mask]) for tiny
 * inputs: P [B, H, N, N] fp64, masked entries exactly 0.
 */
int oracle_probs(const void *q, const void *k, int dtype, int B, int H, int N, int d, double scale,
                 int causal, double *P)
{
    if (!q || !k || !P || B < 1 || H < 1 || N < 1 || d < 1) return -1;
    if (or_elem_bytes(dtype) == 0) return -1;
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        int64_t base = bh * (int64_t)N * d;
        for (int64_t i = 0; i < N; ++i) {
            double *row = P + (bh * N + i) * N;
            int64_t n = causal ? i + 1 : N;
            for (int64_t j = 0; j < N; ++j) row[j] = 0.0;
            if (n <= 0) continue;
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int c = 0; c < d; ++c)
                    dot += or_load(q, dtype, base + i * d + c) * or_load(k, dtype, base + j * d + c);
                row[j] = scale * dot;
            }
            double m = row[0];
            for (int64_t j = 1; j < n; ++j)
                if (row[j] > m) m = row[j];
            double l = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                row[j] = exp(row[j] - m);
                l += row[j];
            }
            for (int64_t j = 0; j < n; ++j) row[j] /= l;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* The tiled online recurrence, in both loop orders (one head)          */
/* ------------------------------------------------------------------ */

/* score of query i against key j, -inf where the mask excludes it */
static double or_score(const double *q, const double *k, int N, int d, double scale, int causal,
                       int64_t i, int64_t j)
{
    if (j >= N || i >= N) return -INFINITY;
    if (causal && j > i) return -INFINITY;
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += q[i * d + c] * k[j * d + c];
    return scale * dot;
}

/*
 * [SU] Eq. (4): two partial results of one row over disjoint sets of keys,
 * each normalised by its own sum, (m1, l1, o1) and (m2, l2, o2), combine into
 * the result over the union:
 *     m = max(m1, m2),  w1 = l1 e^(m1 - m),  w2 = l2 e^(m2 - m),
 *     l = w1 + w2,      o = (w1 o1 + w2 o2) / l.
 * A part with l = 0 (no admissible key) has weight 0.  Part 1 is
 * overwritten with the result.
 */
static void or_merge_partial(double *m1, double *l1, double *o1, double m2, double l2,
                             const double *o2, int d)
{
    if (!(l2 > 0.0)) return;
    if (!(*l1 > 0.0)) {
        *m1 = m2;
        *l1 = l2;
        for (int c = 0; c < d; ++c) o1[c] = o2[c];
        return;
    }
    double m = *m1 > m2 ? *m1 : m2;
    double w1 = *l1 * exp(*m1 - m), w2 = l2 * exp(m2 - m);
    double l = w1 + w2;
    for (int c = 0; c < d; ++c) o1[c] = (w1 * o1[c] + w2 * o2[c]) / l;
    *m1 = m;
    *l1 = l;
}

/*
 * The partial result of query row i over the keys of one key tile,
 * [j0, j0 + Bc) ([SU] Eq. (1) restricted to those keys): its max m~, sum
 * l~ = sum_j exp(s_ij - m~) and normalised output o~ = sum_j exp(s_ij - m~)
 * v_j / l~.  Returns l~ (0 when no key of the tile is admissible); s is
 * scratch of Bc doubles.
 */
static double or_tile_partial(const double *q, const double *k, const double *v, int N, int d,
                              double scale, int causal, int64_t i, int64_t j0, int Bc, double *s,
                              double *mt, double *ot)
{
    double m = -INFINITY;
    for (int cc = 0; cc < Bc; ++cc) {
        s[cc] = or_score(q, k, N, d, scale, causal, i, j0 + cc);
        if (s[cc] > m) m = s[cc];
    }
    *mt = m;
    if (m == -INFINITY) return 0.0;
    double l = 0.0;
    for (int cc = 0; cc < Bc; ++cc) l += exp(s[cc] - m); /* exp(-inf) = 0: masked keys */
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int cc = 0; cc < Bc; ++cc)
            if (j0 + cc < N) acc += exp(s[cc] - m) * v[(j0 + cc) * d + c];
        ot[c] = acc / l;
    }
    return l;
}

/*
 * FlashAttention-1 loop order ([YJ] 5.2): the outer loop runs over the K/V
 * tiles j, the inner loops over the Q tiles of Br rows and their rows; the
 * running state (m, l, O) of every row lives outside the loops (in HBM, on
 * the page) and absorbs each tile's partial result through the merge of
 * [SU] Eq. (4).  (The [YJ] 5.2 pseudocode writes an inverse on the
 * exponential factors of that update; Eq. (4) and [YJ] 6.2 have none, so it
 * is read as a typesetting slip.)  Outputs o [N, d] and lse [N] (lse =
 * m + ln l).
 */
int oracle_tiled_fa1(const double *q, const double *k, const double *v, int N, int d, double scale,
                     int causal, int Br, int Bc, double *o, double *lse)
{
    if (!q || !k || !v || !o || !lse || N < 1 || d < 1 || Br < 1 || Bc < 1) return -1;
    double *m = (double *)malloc(sizeof(double) * N);
    double *l = (double *)malloc(sizeof(double) * N);
    double *s = (double *)malloc(sizeof(double) * Bc);
    double *ot = (double *)malloc(sizeof(double) * d);
    if (!m || !l || !s || !ot) { free(m); free(l); free(s); free(ot); return -1; }
    for (int64_t i = 0; i < N; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.0;
        for (int c = 0; c < d; ++c) o[i * d + c] = 0.0;
    }
    int Tr = (N + Br - 1) / Br, Tc = (N + Bc - 1) / Bc;
    for (int j = 0; j < Tc; ++j)
        for (int it = 0; it < Tr; ++it)
            for (int r = 0; r < Br && (int64_t)it * Br + r < N; ++r) {
                int64_t i = (int64_t)it * Br + r;
                double mt;
                double lt = or_tile_partial(q, k, v, N, d, scale, causal, i, (int64_t)j * Bc, Bc, s, &mt, ot);
                or_merge_partial(&m[i], &l[i], o + i * d, mt, lt, ot, d);
            }
    for (int64_t i = 0; i < N; ++i) lse[i] = l[i] > 0.0 ? m[i] + log(l[i]) : -INFINITY;
    free(m); free(l); free(s); free(ot);
    return 0;
}

/*
 * FlashAttention-2 loop order ([FX] kernel listing; [YJ] 8.1-8.2): outer
 * loop over Q tiles, inner loop over K/V tiles, running (m, l) per row and an
 * UNNORMALISED accumulator divided by l once at the end:
 *     m_new = max(m, rowmax(S_ij))                  [SU] Eq. (2)
 *     P~    = exp(S_ij - m_new)
 *     l     = e^(m - m_new) l + rowsum(P~)          [SU] Eq. (3)
 *     Oacc  = e^(m - m_new) Oacc + P~ V_j
 *     O     = Oacc / l,  lse = m + ln l             (after the last tile)
 */
int oracle_tiled_fa2(const double *q, const double *k, const double *v, int N, int d, double scale,
                     int causal, int Br, int Bc, double *o, double *lse)
{
    if (!q || !k || !v || !o || !lse || N < 1 || d < 1 || Br < 1 || Bc < 1) return -1;
    double *pt = (double *)malloc(sizeof(double) * Bc);
    if (!pt) return -1;
    int Tr = (N + Br - 1) / Br, Tc = (N + Bc - 1) / Bc;
    for (int it = 0; it < Tr; ++it) {
        for (int r = 0; r < Br; ++r) {
            int64_t i = (int64_t)it * Br + r;
            if (i >= N) break;
            double m = -INFINITY, l = 0.0;
            double *acc = o + i * d;
            for (int c = 0; c < d; ++c) acc[c] = 0.0;
            for (int j = 0; j < Tc; ++j) {
                double mt = -INFINITY;
                for (int cc = 0; cc < Bc; ++cc) {
                    pt[cc] = or_score(q, k, N, d, scale, causal, i, (int64_t)j * Bc + cc);
                    if (pt[cc] > mt) mt = pt[cc];
                }
                double mnew = m > mt ? m : mt;
                if (mnew == -INFINITY) continue; /* no admissible key seen yet */
                double alpha = exp(m - mnew);
                double rs = 0.0;
                for (int cc = 0; cc < Bc; ++cc) {
                    pt[cc] = exp(pt[cc] - mnew);
                    rs += pt[cc];
                }
                l = alpha * l + rs;
                for (int c = 0; c < d; ++c) {
                    double pv = 0.0;
                    for (int cc = 0; cc < Bc; ++cc) {
                        int64_t jj = (int64_t)j * Bc + cc;
                        if (jj < N) pv += pt[cc] * v[jj * d + c];
                    }
                    acc[c] = alpha * acc[c] + pv;
                }
                m = mnew;
            }
            if (l > 0.0) {
                for (int c = 0; c < d; ++c) acc[c] /= l;
                lse[i] = m + log(l);
            } else {
                lse[i] = -INFINITY;
            }
        }
    }
    free(pt);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Paged single-query decode                                            */
/* ------------------------------------------------------------------ */

/*
 * Cache layouts ([PA] "Inputs", "Concepts", "Key", "Value"):
 *   k_cache [num_blocks, num_kv_heads, head_size/x, block_size, x]
 *   v_cache [num_blocks, num_kv_heads, head_size, block_size]
 * where x is the number of elements in one 16-byte vector (8 for fp16).
 * Token t of sequence s lives in physical block block_tables[s][t / BS] at
 * offset t % BS; query head h reads kv head h / (num_heads / num_kv_heads).
 */
typedef struct {
    const void *q, *kc, *vc;
    int dtype;
    const int32_t *bt, *ctx_lens;
    int S, H, Hkv, D, BS, MB, x;
    double scale;
    int part_tokens; /* 0: no partitioning */
    double *out, *lse;
    double *part_m, *part_l, *part_o; /* optional partition partials */
    int P;                            /* partitions per (s, h) in part_* */
} or_dec_ctx;

static int64_t or_k_index(const or_dec_ctx *x, int64_t blk, int kvh, int e, int off)
{
    return ((((blk * x->Hkv + kvh) * (x->D / x->x) + e / x->x) * x->BS + off) * x->x) + e % x->x;
}

static int64_t or_v_index(const or_dec_ctx *x, int64_t blk, int kvh, int e, int off)
{
    return ((blk * x->Hkv + kvh) * (int64_t)x->D + e) * x->BS + off;
}

typedef struct {
    const or_dec_ctx *x;
    int s, kvh;
    int64_t t0; /* first context token of the range */
} or_paged_v;

static double or_paged_value(const void *ctx, int64_t j, int e)
{
    const or_paged_v *pv = (const or_paged_v *)ctx;
    const or_dec_ctx *x = pv->x;
    int64_t t = pv->t0 + j;
    int64_t blk = x->bt[(int64_t)pv->s * x->MB + t / x->BS];
    return or_load(x->vc, x->dtype, or_v_index(x, blk, pv->kvh, e, (int)(t % x->BS)));
}

/* logits scale * q . K_t for t in [t0, t1) into s[0 .. t1-t0) */
static void or_paged_logits(const or_dec_ctx *x, int s, int h, int64_t t0, int64_t t1, double *lg)
{
    int kvh = h / (x->H / x->Hkv);
    int64_t qbase = ((int64_t)s * x->H + h) * x->D;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t blk = x->bt[(int64_t)s * x->MB + t / x->BS];
        int off = (int)(t % x->BS);
        double dot = 0.0;
        for (int e = 0; e < x->D; ++e)
            dot += or_load(x->q, x->dtype, qbase + e) *
                   or_load(x->kc, x->dtype, or_k_index(x, blk, kvh, e, off));
        lg[t - t0] = x->scale * dot;
    }
}

static void or_dec_item(void *vctx, int64_t item, double *scratch)
{
    const or_dec_ctx *x = (const or_dec_ctx *)vctx;
    int s = (int)(item / x->H), h = (int)(item % x->H);
    int kvh = h / (x->H / x->Hkv);
    int64_t n = x->ctx_lens[s];
    double *out = x->out + item * x->D;
    if (x->part_tokens <= 0) {
        or_paged_logits(x, s, h, 0, n, scratch);
        or_paged_v pv = { x, s, kvh, 0 };
        double l = or_softmax_row(scratch, n, x->D, or_paged_value, &pv, out);
        if (x->lse) x->lse[item] = l;
        return;
    }
    /*
     * Partitioned form ([PA] grid axis max_num_partitions, "Softmax",
     * "exp_sum", "Value", "Output"): each partition of part_tokens context
     * tokens gets its own max m_p, exp-sum l_p and NORMALISED partial O_p;
     * the partials are then merged with [SU] Eq. (4) generalised to P parts:
     *     m = max_p m_p,  w_p = l_p e^(m_p - m),
     *     O = sum_p w_p O_p / sum_p w_p,  lse = m + ln(sum_p w_p).
     * An empty partition (m_p = -inf, l_p = 0) has weight 0.
     */
    double *op = scratch + x->part_tokens; /* D doubles for one partial */
    int64_t nparts = (n + x->part_tokens - 1) / x->part_tokens;
    double m_all = -INFINITY;
    for (int64_t p = 0; p < nparts; ++p) {
        double *pm = x->part_m + item * x->P + p;
        double *pl = x->part_l + item * x->P + p;
        int64_t t0 = p * x->part_tokens;
        int64_t t1 = t0 + x->part_tokens < n ? t0 + x->part_tokens : n;
        or_paged_logits(x, s, h, t0, t1, scratch);
        double mp = scratch[0];
        for (int64_t t = 1; t < t1 - t0; ++t)
            if (scratch[t] > mp) mp = scratch[t];
        double lp = 0.0;
        for (int64_t t = 0; t < t1 - t0; ++t) {
            scratch[t] = exp(scratch[t] - mp);
            lp += scratch[t];
        }
        for (int64_t t = 0; t < t1 - t0; ++t) scratch[t] /= lp; /* normalised partition */
        or_paged_v pv = { x, s, kvh, t0 };
        for (int e = 0; e < x->D; ++e) {
            double acc = 0.0;
            for (int64_t t = 0; t < t1 - t0; ++t) acc += scratch[t] * or_paged_value(&pv, t, e);
            op[e] = acc;
        }
        *pm = mp;
        *pl = lp;
        for (int e = 0; e < x->D; ++e) x->part_o[(item * x->P + p) * x->D + e] = op[e];
        if (mp > m_all) m_all = mp;
    }
    for (int64_t p = nparts; p < x->P; ++p) {
        x->part_m[item * x->P + p] = -INFINITY;
        x->part_l[item * x->P + p] = 0.0;
        for (int e = 0; e < x->D; ++e) x->part_o[(item * x->P + p) * x->D + e] = 0.0;
    }
    double wsum = 0.0;
    for (int e = 0; e < x->D; ++e) out[e] = 0.0;
    for (int64_t p = 0; p < nparts; ++p) {
        double w = x->part_l[item * x->P + p] * exp(x->part_m[item * x->P + p] - m_all);
        wsum += w;
        for (int e = 0; e < x->D; ++e) out[e] += w * x->part_o[(item * x->P + p) * x->D + e];
    }
    if (wsum > 0.0) {
        for (int e = 0; e < x->D; ++e) out[e] /= wsum;
        if (x->lse) x->lse[item] = m_all + log(wsum);
    } else if (x->lse) {
        x->lse[item] = -INFINITY;
    }
}

static int or_dec_check(const void *q, const void *kc, const void *vc, int dtype,
                        const int32_t *bt, const int32_t *cl, int S, int H, int Hkv, int D,
                        int BS, int MB)
{
    if (!q || !kc || !vc || !bt || !cl) return -1;
    int es = or_elem_bytes(dtype);
    if (es == 0 || es > 16 || 16 % es) return -1;
    if (S < 1 || H < 1 || Hkv < 1 || H % Hkv || D < 1 || BS < 1 || MB < 1) return -1;
    if (D % (16 / es)) return -1;
    for (int s = 0; s < S; ++s)
        if (cl[s] < 0 || (int64_t)cl[s] > (int64_t)MB * BS) return -1;
    return 0;
}

/*
 * Single-query paged decode, unsplit: for every sequence s and head h,
 * out[s,h,:] = softmax over t < context_lens[s] of scale * q[s,h] . K_t,
 * applied to V_t (no causal mask).  out [S, H, D] fp64, lse [S, H] (may be
 * NULL).  Context length 0 gives out = 0, lse = -inf.
 */
int oracle_paged_decode(const void *q, const void *k_cache, const void *v_cache, int dtype,
                        const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                        int num_heads, int num_kv_heads, int head_size, int block_size,
                        int max_blocks_per_seq, double scale, double *out, double *lse,
                        int nthreads)
{
    if (or_dec_check(q, k_cache, v_cache, dtype, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_size, block_size, max_blocks_per_seq) || !out)
        return -1;
    or_dec_ctx x = { q, k_cache, v_cache, dtype, block_tables, context_lens,
                     num_seqs, num_heads, num_kv_heads, head_size, block_size,
                     max_blocks_per_seq, 16 / or_elem_bytes(dtype), scale, 0,
                     out, lse, NULL, NULL, NULL, 0 };
    int64_t maxctx = (int64_t)max_blocks_per_seq * block_size;
    return or_parallel(or_dec_item, &x, (int64_t)num_seqs * num_heads, maxctx, nthreads);
}

/*
 * The same decode computed per context partition of part_tokens tokens and
 * merged (see or_dec_item).  Also returns the partials:
 *   part_m, part_l [S, H, P];  part_o [S, H, P, D]  with
 *   P = ceil(max_blocks_per_seq * block_size / part_tokens).
 */
int oracle_paged_decode_partitioned(const void *q, const void *k_cache, const void *v_cache,
                                    int dtype, const int32_t *block_tables,
                                    const int32_t *context_lens, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_size, int block_size,
                                    int max_blocks_per_seq, double scale, int part_tokens,
                                    double *out, double *lse, double *part_m, double *part_l,
                                    double *part_o, int nthreads)
{
    if (or_dec_check(q, k_cache, v_cache, dtype, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_size, block_size, max_blocks_per_seq) || !out)
        return -1;
    if (part_tokens < 1 || !part_m || !part_l || !part_o) return -1;
    int64_t maxctx = (int64_t)max_blocks_per_seq * block_size;
    int P = (int)((maxctx + part_tokens - 1) / part_tokens);
    or_dec_ctx x = { q, k_cache, v_cache, dtype, block_tables, context_lens,
                     num_seqs, num_heads, num_kv_heads, head_size, block_size,
                     max_blocks_per_seq, 16 / or_elem_bytes(dtype), scale, part_tokens,
                     out, lse, part_m, part_l, part_o, P };
    return or_parallel(or_dec_item, &x, (int64_t)num_seqs * num_heads,
                       (int64_t)part_tokens + head_size, nthreads);
}

/* ------------------------------------------------------------------ */
/* Dense attention backward                                             */
/* ------------------------------------------------------------------ */

/*
 * Gradients of O = softmax(scale * Q K^T [+ causal mask]) V given the
 * upstream gradient dO = dL/dO.  The pages fix the method ([YJ] 7.1-7.2:
 * the backward pass needs P, and FlashAttention recomputes it from Q, K, V
 * and the saved row statistics instead of storing it); the gradients
 * themselves are the chain rule applied to the forward definition:
 *     P_ij  = exp(s_ij - m_i) / l_i               (row i of the forward)
 *     dV_j  = sum_i P_ij dO_i
 *     dP_ij = dO_i . V_j
 *     D_i   = sum_j P_ij dP_ij                     (= dO_i . O_i)
 *     dS_ij = P_ij (dP_ij - D_i)                   (softmax Jacobian)
 *     dQ_i  = scale sum_j dS_ij K_j
 *     dK_j  = scale sum_i dS_ij Q_i
 * sums over admissible pairs only.  With grouped kv heads, dK and dV of kv
 * head g collect the terms of every query head that reads g, query heads in
 * ascending order.
 *
 * Two passes, each summing in ascending index order (so the result does not
 * depend on the thread count):
 *   1. per query row (b, h, i): m_i, l_i, D_i and, for selected rows, dQ_i;
 *   2. per key row (b, g, j): dV_j and dK_j over query heads h of group g,
 *      then rows i, recomputing P_ij and dP_ij with pass 1's m_i, l_i, D_i.
 */
typedef struct {
    const void *q, *k, *v, *dout;
    int dtype;
    int B, H, Hkv, N, d;
    double scale;
    int causal;
    const int64_t *rows, *keys;
    int64_t nrows, nkeys;
    const unsigned char *need_row; /* [N]: row i is needed by pass 1 */
    double *m, *l, *D;             /* [B, H, N] row statistics */
    double *dq, *dk, *dv;
} or_bwd_ctx;

static int64_t or_bwd_qbase(const or_bwd_ctx *x, int64_t b, int64_t h)
{
    return (b * x->H + h) * (int64_t)x->N * x->d;
}

static int64_t or_bwd_kvbase(const or_bwd_ctx *x, int64_t b, int64_t h)
{
    return (b * x->Hkv + h / (x->H / x->Hkv)) * (int64_t)x->N * x->d;
}

static double or_dot(const void *a, int64_t ia, const void *b, int64_t ib, int dtype, int d)
{
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += or_load(a, dtype, ia + c) * or_load(b, dtype, ib + c);
    return acc;
}

/* pass 1, item = (b, h, r): r indexes all N rows */
static void or_bwd_row_item(void *vctx, int64_t item, double *s)
{
    const or_bwd_ctx *x = (const or_bwd_ctx *)vctx;
    const int64_t N = x->N, d = x->d;
    int64_t i = item % N, bh = item / N;
    int64_t b = bh / x->H, h = bh % x->H;
    if (!x->need_row[i]) return;
    int64_t qb = or_bwd_qbase(x, b, h), kb = or_bwd_kvbase(x, b, h);
    int64_t n = x->causal ? i + 1 : N;
    double *dp = s + N;
    for (int64_t j = 0; j < n; ++j) s[j] = x->scale * or_dot(x->q, qb + i * d, x->k, kb + j * d, x->dtype, x->d);
    double m = s[0];
    for (int64_t j = 1; j < n; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) l += exp(s[j] - m);
    double D = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m) / l; /* P_ij */
        dp[j] = or_dot(x->dout, qb + i * d, x->v, kb + j * d, x->dtype, x->d);
        D += s[j] * dp[j];
    }
    x->m[item] = m;
    x->l[item] = l;
    x->D[item] = D;
    if (!x->dq) return;
    int64_t r = -1;
    if (!x->rows) r = i;
    else
        for (int64_t t = 0; t < x->nrows; ++t)
            if (x->rows[t] == i) { r = t; break; }
    if (r < 0) return;
    double *dq = x->dq + (bh * x->nrows + r) * d;
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j)
            acc += s[j] * (dp[j] - D) * or_load(x->k, x->dtype, kb + j * d + c);
        dq[c] = x->scale * acc;
    }
}

/* pass 2, item = (b, g, t): t indexes the selected keys */
static void or_bwd_key_item(void *vctx, int64_t item, double *scratch)
{
    const or_bwd_ctx *x = (const or_bwd_ctx *)vctx;
    const int64_t N = x->N, d = x->d;
    int64_t t = item % x->nkeys, bg = item / x->nkeys;
    int64_t b = bg / x->Hkv, g = bg % x->Hkv;
    int64_t j = x->keys ? x->keys[t] : t;
    int group = x->H / x->Hkv;
    double *dk = x->dk + item * d, *dv = x->dv + item * d;
    (void)scratch;
    for (int c = 0; c < d; ++c) dk[c] = dv[c] = 0.0;
    for (int64_t h = g * group; h < (g + 1) * group; ++h) {
        int64_t qb = or_bwd_qbase(x, b, h), kb = or_bwd_kvbase(x, b, h);
        int64_t st = (b * x->H + h) * N;
        for (int64_t i = x->causal ? j : 0; i < N; ++i) {
            double sij = x->scale * or_dot(x->q, qb + i * d, x->k, kb + j * d, x->dtype, x->d);
            double p = exp(sij - x->m[st + i]) / x->l[st + i];
            double dp = or_dot(x->dout, qb + i * d, x->v, kb + j * d, x->dtype, x->d);
            double ds = p * (dp - x->D[st + i]);
            for (int c = 0; c < d; ++c) {
                dv[c] += p * or_load(x->dout, x->dtype, qb + i * d + c);
                dk[c] += ds * or_load(x->q, x->dtype, qb + i * d + c);
            }
        }
    }
    for (int c = 0; c < d; ++c) dk[c] *= x->scale;
}

/*
 * q, dout [B, H, N, d]; k, v [B, Hkv, N, d] (contiguous, storage dtype).
 *   rows  : query rows whose dQ is wanted (NULL: all N, in order; nrows may
 *           be 0 with dq NULL to skip dQ);  dq [B, H, nrows, d] fp64.
 *   keys  : key rows whose dK, dV are wanted (NULL: all N; nkeys 0 with
 *           dk, dv NULL skips them);  dk, dv [B, Hkv, nkeys, d] fp64.
 *   D     : optional [B, H, N] fp64 output of D_i (computed for every row
 *           that pass 2 or dQ needs; other entries untouched).
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attention_bwd(const void *q, const void *k, const void *v, const void *dout, int dtype,
                         int B, int H, int Hkv, int N, int d, double scale, int causal,
                         const int64_t *rows, int64_t nrows, const int64_t *keys, int64_t nkeys,
                         double *dq, double *dk, double *dv, double *D_out, int nthreads)
{
    if (!q || !k || !v || !dout || B < 1 || H < 1 || N < 1 || d < 1) return -1;
    if (Hkv < 1 || H % Hkv != 0) return -1;
    if (or_elem_bytes(dtype) == 0) return -1;
    if (!rows) nrows = N;
    if (!keys) nkeys = N;
    if (nrows < 0 || nkeys < 0) return -1;
    if ((nrows > 0 && !dq) || (nkeys > 0 && (!dk || !dv))) return -1;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return -1;
    for (int64_t t = 0; keys && t < nkeys; ++t)
        if (keys[t] < 0 || keys[t] >= N) return -1;
    int64_t nst = (int64_t)B * H * N;
    unsigned char *need = (unsigned char *)calloc((size_t)N, 1);
    double *m = (double *)malloc(sizeof(double) * nst);
    double *l = (double *)malloc(sizeof(double) * nst);
    double *D = (double *)malloc(sizeof(double) * nst);
    int rc = -1;
    if (!need || !m || !l || !D) goto out;
    /* pass 2 needs every row that sees a selected key; dQ needs its rows */
    if (nkeys > 0) {
        int64_t jmin = N;
        for (int64_t t = 0; t < nkeys; ++t) {
            int64_t j = keys ? keys[t] : t;
            if (j < jmin) jmin = j;
        }
        for (int64_t i = causal ? jmin : 0; i < N; ++i) need[i] = 1;
    }
    for (int64_t r = 0; r < nrows; ++r) need[rows ? rows[r] : r] = 1;
    {
        or_bwd_ctx x = { q, k, v, dout, dtype, B, H, Hkv, N, d, scale, causal,
                         rows, keys, nrows, nkeys, need, m, l, D,
                         nrows > 0 ? dq : NULL, dk, dv };
        rc = or_parallel(or_bwd_row_item, &x, nst, 2 * (int64_t)N, nthreads);
        if (rc == 0 && nkeys > 0)
            rc = or_parallel(or_bwd_key_item, &x, (int64_t)B * Hkv * nkeys, 0, nthreads);
        if (rc == 0 && D_out)
            for (int64_t it = 0; it < nst; ++it)
                if (need[it % N]) D_out[it] = D[it];
    }
out:
    free(need); free(m); free(l); free(D);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Block-scaled FP8 (E4M3) quantisation                                 */
/* ------------------------------------------------------------------ */

/*
 * [YJ] 9.2 item 3: FP8 attention keeps a separate scale factor for each
 * block of the inputs so that each block uses the FP8 range.  Readings fixed
 * here (the pages name the technique only):
 *   - the FP8 format is E4M3 as defined by the OCP 8-bit floating point
 *     specification ("E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 *     subnormals, no infinities, S.1111.111 = NaN, largest finite 448;
 *   - a block is 128 consecutive rows of one (b, h) with all d columns;
 *   - the block's scale is the power of two 2^e with e = floor(log2 amax) - 7
 *     (amax = largest magnitude in the block; e = 0 for an all-zero block),
 *     so that every scaled value is below 256 and the scaling is exact;
 *   - code = E4M3 rounding (to nearest, ties to even) of x * 2^-e;
 *     dequantised value = value(code) * 2^e.
 */

/* E4M3 code of a finite double, round to nearest even, saturating at 448 */
static uint8_t or_e4m3_encode_one(double x)
{
    uint8_t s = (x < 0 || (x == 0 && signbit(x))) ? 0x80 : 0;
    double a = fabs(x);
    if (isnan(x)) return (uint8_t)(s | 0x7f);
    if (a < ldexp(1.0, -6)) {
        /* subnormal: a multiple of 2^-9 with a 3-bit mantissa */
        double m = nearbyint(ldexp(a, 9)); /* 0 .. 8; 8 is the smallest normal */
        return (uint8_t)(s | (uint8_t)m);
    }
    int ex;
    frexp(a, &ex); /* a = f 2^ex, f in [0.5, 1) */
    int E = ex - 1;  /* a in [2^E, 2^(E+1)) */
    double m = nearbyint((ldexp(a, -E) - 1.0) * 8.0); /* 0 .. 8 */
    if (m == 8.0) { m = 0.0; E += 1; }
    if (E > 8 || (E == 8 && m > 6.0)) return (uint8_t)(s | 0x7e); /* saturate to 448 */
    return (uint8_t)(s | (uint8_t)((E + 7) << 3) | (uint8_t)m);
}

static double or_e4m3_decode_one(uint8_t c)
{
    int s = c >> 7, ef = (c >> 3) & 15, m = c & 7;
    double v;
    if (ef == 15 && m == 7) return NAN;
    if (ef == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, ef - 7);
    return s ? -v : v;
}

int oracle_e4m3_encode(const double *x, int64_t n, uint8_t *codes)
{
    if ((!x || !codes) && n > 0) return -1;
    for (int64_t i = 0; i < n; ++i) codes[i] = or_e4m3_encode_one(x[i]);
    return 0;
}

int oracle_e4m3_decode(const uint8_t *codes, int64_t n, double *x)
{
    if ((!x || !codes) && n > 0) return -1;
    for (int64_t i = 0; i < n; ++i) x[i] = or_e4m3_decode_one(codes[i]);
    return 0;
}

/*
 * Code layouts:
 *   layout 0 (Q, K): codes [B, H, N, d], row-major like the input;
 *   layout 1 (V):    codes [B, H, T, d, 64] with T = ceil(N / 64): each tile
 *                    of 64 keys is stored d-major (element (key, c) of tile t
 *                    at [t][c][key - 64 t]); keys >= N hold code 0.
 * exps: [B, H, ceil(N / 128)] int32, the block exponents e.
 */
static int64_t or_fp8_code_index(int layout, int64_t bh, int64_t N, int d, int64_t i, int c)
{
    if (layout == 0) return (bh * N + i) * d + c;
    int64_t T = (N + 63) / 64;
    return ((bh * T + i / 64) * d + c) * 64 + (i % 64);
}

int64_t oracle_fp8_codes_len(int layout, int B, int H, int N, int d)
{
    if (layout == 0) return (int64_t)B * H * N * d;
    return (int64_t)B * H * ((N + 63) / 64) * d * 64;
}

int oracle_quant_fp8(const void *x, int dtype, int B, int H, int N, int d, int layout,
                     uint8_t *codes, int32_t *exps)
{
    if (!x || !codes || !exps || B < 1 || H < 1 || N < 1 || d < 1) return -1;
    if (or_elem_bytes(dtype) == 0 || (layout != 0 && layout != 1)) return -1;
    int64_t nblk = (N + 127) / 128;
    memset(codes, 0, (size_t)oracle_fp8_codes_len(layout, B, H, N, d));
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        for (int64_t blk = 0; blk < nblk; ++blk) {
            int64_t r0 = blk * 128, r1 = r0 + 128 < N ? r0 + 128 : N;
            double amax = 0.0;
            for (int64_t i = r0; i < r1; ++i)
                for (int c = 0; c < d; ++c) {
                    double a = fabs(or_load(x, dtype, (bh * N + i) * d + c));
                    if (a > amax) amax = a;
                }
            int e = 0;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);
                e = (ex - 1) - 7;
            }
            exps[bh * nblk + blk] = e;
            for (int64_t i = r0; i < r1; ++i)
                for (int c = 0; c < d; ++c)
                    codes[or_fp8_code_index(layout, bh, N, d, i, c)] =
                        or_e4m3_encode_one(ldexp(or_load(x, dtype, (bh * N + i) * d + c), -e));
        }
    }
    return 0;
}

/* dequantised values in the natural layout: out [B, H, N, d] fp64 */
int oracle_dequant_fp8(const uint8_t *codes, const int32_t *exps, int B, int H, int N, int d,
                       int layout, double *out)
{
    if (!codes || !exps || !out || B < 1 || H < 1 || N < 1 || d < 1) return -1;
    if (layout != 0 && layout != 1) return -1;
    int64_t nblk = (N + 127) / 128;
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh)
        for (int64_t i = 0; i < N; ++i)
            for (int c = 0; c < d; ++c)
                out[(bh * N + i) * d + c] =
                    ldexp(or_e4m3_decode_one(codes[or_fp8_code_index(layout, bh, N, d, i, c)]),
                          exps[bh * nblk + i / 128]);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Attention with general masks                                         */
/* ------------------------------------------------------------------ */

/*
 * [YJ] 11.3 passes either is_causal or an explicit boolean attn_mask (True =
 * the pair takes part); [YJ] 11.6 names sliding-window attention.  The
 * admissible keys of query row i (0 <= i < Nq) over Nk keys are
 *     A_i = { j < Nk : (!causal  or j <= i + off)
 *                     and (wl < 0 or j >= i + off - wl)
 *                     and (wr < 0 or j <= i + off + wr)
 *                     and (!mask or mask[i][j] != 0) },   off = Nk - Nq,
 * i.e. a causal mask aligned to the bottom-right corner when Nq != Nk (the
 * last query is the last key, as for new tokens appended to a context), and
 * a window of wl keys to the left and wr keys to the right of that
 * diagonal (a negative bound is unbounded).  mask is uint8 [.., Nq, Nk] at
 * element offset b * mask_sb + h * mask_sh (a zero stride broadcasts).
 * O_i = softmax over A_i of scale q_i . k_j applied to V; an empty A_i gives
 * O_i = 0 and lse_i = -inf.
 */
typedef struct {
    const void *q, *k, *v;
    int dtype;
    int B, H, Hkv, Nq, Nk, d;
    double scale;
    int causal, wl, wr;
    const uint8_t *mask;
    int64_t msb, msh;
    const int64_t *rows;
    int64_t nrows;
    double *o, *lse;
} or_ext_ctx;

static int or_ext_admissible(const or_ext_ctx *x, int64_t b, int64_t h, int64_t i, int64_t j)
{
    int64_t off = (int64_t)x->Nk - x->Nq;
    if (x->causal && j > i + off) return 0;
    if (x->wl >= 0 && j < i + off - x->wl) return 0;
    if (x->wr >= 0 && j > i + off + x->wr) return 0;
    if (x->mask && !x->mask[b * x->msb + h * x->msh + i * x->Nk + j]) return 0;
    return 1;
}

typedef struct {
    const void *v;
    int dtype;
    int64_t base;
    int d;
    const int64_t *idx; /* admissible key of each position */
} or_ext_v;

static double or_ext_value(const void *ctx, int64_t j, int c)
{
    const or_ext_v *ev = (const or_ext_v *)ctx;
    return or_load(ev->v, ev->dtype, ev->base + ev->idx[j] * ev->d + c);
}

static void or_ext_item(void *vctx, int64_t item, double *scratch)
{
    const or_ext_ctx *x = (const or_ext_ctx *)vctx;
    int64_t r = item % x->nrows, bh = item / x->nrows;
    int64_t i = x->rows ? x->rows[r] : r;
    int64_t b = bh / x->H, h = bh % x->H;
    int64_t qb = bh * (int64_t)x->Nq * x->d;
    int64_t kb = (b * x->Hkv + h / (x->H / x->Hkv)) * (int64_t)x->Nk * x->d;
    double *s = scratch;
    int64_t *idx = (int64_t *)(scratch + x->Nk);
    int64_t n = 0;
    for (int64_t j = 0; j < x->Nk; ++j) {
        if (!or_ext_admissible(x, b, h, i, j)) continue;
        double dot = 0.0;
        for (int c = 0; c < x->d; ++c)
            dot += or_load(x->q, x->dtype, qb + i * x->d + c) * or_load(x->k, x->dtype, kb + j * x->d + c);
        s[n] = x->scale * dot;
        idx[n] = j;
        ++n;
    }
    or_ext_v ev = { x->v, x->dtype, kb, x->d, idx };
    x->lse[item] = or_softmax_row(s, n, x->d, or_ext_value, &ev, x->o + item * x->d);
}

/*
 * q [B, H, Nq, d]; k, v [B, Hkv, Nk, d]; mask may be NULL.  rows selects the
 * query rows to evaluate (NULL: all Nq); o [B, H, nrows, d] and
 * lse [B, H, nrows] fp64.
 */
int oracle_attention_ext(const void *q, const void *k, const void *v, int dtype, int B, int H,
                         int Hkv, int Nq, int Nk, int d, double scale, int causal, int wl, int wr,
                         const uint8_t *mask, int64_t mask_sb, int64_t mask_sh,
                         const int64_t *rows, int64_t nrows, double *o, double *lse, int nthreads)
{
    if (!q || !k || !v || !o || !lse || B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return -1;
    if (Hkv < 1 || H % Hkv != 0 || or_elem_bytes(dtype) == 0) return -1;
    if (mask && (mask_sb < 0 || mask_sh < 0)) return -1;
    if (!rows) nrows = Nq;
    if (nrows < 1) return -1;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= Nq) return -1;
    or_ext_ctx x = { q, k, v, dtype, B, H, Hkv, Nq, Nk, d, scale, causal ? 1 : 0,
                     wl, wr, mask, mask_sb, mask_sh, rows, nrows, o, lse };
    /* scratch: Nk scores + Nk key indices (int64 stored in doubles' space) */
    return or_parallel(or_ext_item, &x, (int64_t)B * H * nrows, 2 * (int64_t)Nk, nthreads);
}

/* ------------------------------------------------------------------ */
/* Block map of a boolean mask                                          */
/* ------------------------------------------------------------------ */

/*
 * The boolean attn_mask of "FlashAttention: GPU 메모리 계층을 활용한 어텐션
 * 최적화 분석" (youngju.dev), section 11.3, summarised per block of 128 query
 * rows x 64 keys: which blocks hold a pair that takes part, and which hold no
 * masked pair.  The pages define the mask only; the map is the forward's
 * own acceleration structure, and this is its plain definition, block by
 * block and byte by byte.
 *
 * mask: Bs x Hs slices, slice (b, h) at byte b * mask_sb + h * mask_sh, Nq
 * rows mask_ld bytes apart, of which the first Nk count.  out: uint32 words
 * [Bs][Hs][ceil(Nq/128)][2][nkw], nkw = ceil(ceil(Nk/64) / 32), written in
 * full: bit i of word w of the first half is set iff key block 32 w + i has
 * a nonzero byte among its rows below Nq and keys below Nk; of the second
 * half, iff it has no zero byte there.  Blocks past Nk keep both bits 0.
 */
int oracle_mask_blocks(const uint8_t *mask, int Bs, int Hs, int Nq, int Nk, int64_t mask_sb,
                       int64_t mask_sh, int64_t mask_ld, uint32_t *out)
{
    if (!mask || !out || Bs < 1 || Hs < 1 || Nq < 1 || Nk < 1 || mask_ld < Nk) return -1;
    if (mask_sb < 0 || mask_sh < 0) return -1;
    const int nqb = (Nq + 127) / 128, nkb = (Nk + 63) / 64, nkw = (nkb + 31) / 32;
    for (int b = 0; b < Bs; ++b)
        for (int h = 0; h < Hs; ++h)
            for (int qb = 0; qb < nqb; ++qb) {
                uint32_t *words = out + (((int64_t)b * Hs + h) * nqb + qb) * 2 * nkw;
                for (int w = 0; w < 2 * nkw; ++w) words[w] = 0;
                for (int kb = 0; kb < nkb; ++kb) {
                    int any = 0, all = 1;
                    for (int i = qb * 128; i < qb * 128 + 128 && i < Nq; ++i)
                        for (int j = kb * 64; j < kb * 64 + 64 && j < Nk; ++j) {
                            if (mask[b * mask_sb + h * mask_sh + (int64_t)i * mask_ld + j] != 0)
                                any = 1;
                            else
                                all = 0;
                        }
                    if (any) words[kb / 32] |= 1u << (kb % 32);
                    if (all) words[nkw + kb / 32] |= 1u << (kb % 32);
                }
            }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Chunked prefill over the paged cache                                 */
/* ------------------------------------------------------------------ */

/*
 * Nq new query tokens per sequence attend to the sequence's context in the
 * paged cache (the cache layouts of [PA] "Inputs", "Concepts", "Key",
 * "Value"; one query token per sequence there, Nq here).  The queries are
 * the context's last Nq tokens: query row i of sequence s is context token
 * ctx_s - Nq + i, so the causal mask is aligned to the bottom-right corner
 * ([YJ] 11.3's is_causal on a rectangle; reading 30).  Row i sees the
 * context tokens t < ctx_s with (causal == 0 or t <= i + ctx_s - Nq), then
 * the dense softmax over them ([SU] Eq. (1)); a row that sees no token gets
 * O = 0 and lse = -inf.
 *
 * q [S, H, Nq, D]; caches as for the decode; o [S, H, Nq, D] and
 * lse [S, H, Nq] fp64.
 */
typedef struct {
    or_dec_ctx d;
    int Nq, causal;
    double *o, *lse;
} or_pre_ctx;

static void or_pre_item(void *vctx, int64_t item, double *scratch)
{
    const or_pre_ctx *x = (const or_pre_ctx *)vctx;
    const or_dec_ctx *dx = &x->d;
    int64_t i = item % x->Nq, sh = item / x->Nq;
    int s = (int)(sh / dx->H), h = (int)(sh % dx->H);
    int kvh = h / (dx->H / dx->Hkv);
    int64_t ctx = dx->ctx_lens[s];
    int64_t n = ctx;
    if (x->causal) {
        int64_t last = i + ctx - x->Nq; /* the row's own context position */
        n = last + 1 < ctx ? last + 1 : ctx;
        if (n < 0) n = 0;
    }
    int64_t qbase = item * dx->D;
    for (int64_t t = 0; t < n; ++t) {
        int64_t blk = dx->bt[(int64_t)s * dx->MB + t / dx->BS];
        int off = (int)(t % dx->BS);
        double dot = 0.0;
        for (int e = 0; e < dx->D; ++e)
            dot += or_load(dx->q, dx->dtype, qbase + e) *
                   or_load(dx->kc, dx->dtype, or_k_index(dx, blk, kvh, e, off));
        scratch[t] = dx->scale * dot;
    }
    or_paged_v pv = { dx, s, kvh, 0 };
    x->lse[item] = or_softmax_row(scratch, n, dx->D, or_paged_value, &pv, x->o + item * dx->D);
}

int oracle_paged_prefill(const void *q, const void *k_cache, const void *v_cache, int dtype,
                         const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                         int num_heads, int num_kv_heads, int Nq, int head_size, int block_size,
                         int max_blocks_per_seq, double scale, int causal, double *o, double *lse,
                         int nthreads)
{
    if (or_dec_check(q, k_cache, v_cache, dtype, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_size, block_size, max_blocks_per_seq) || !o || !lse || Nq < 1)
        return -1;
    or_pre_ctx x = { { q, k_cache, v_cache, dtype, block_tables, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_size, block_size,
                       max_blocks_per_seq, 16 / or_elem_bytes(dtype), scale, 0,
                       NULL, NULL, NULL, NULL, NULL, 0 },
                     Nq, causal ? 1 : 0, o, lse };
    int64_t maxctx = (int64_t)max_blocks_per_seq * block_size;
    return or_parallel(or_pre_item, &x, (int64_t)num_seqs * num_heads * Nq, maxctx, nthreads);
}
