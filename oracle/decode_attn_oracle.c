/*
 * decode_attn_oracle.c -- fp64 CPU oracle for small-q GQA decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * package smoke check and the CPU-baseline leg of the benchmark may build,
 * load or call it; the product path never does.  It shares no code, header,
 * table or constant with the HIP kernels.
 *
 * What it computes (FlashRT pull request #185, "feat(structures): ggml host
 * adapter -- llama.cpp distribution for pi0.5 on Thor (SM110)", the commit
 * message that introduces the decomposed decode attention): FLASH_ATTN_EXT
 * for at most 16 query tokens over ONE padded f16 KV head that every query
 * head shares, i.e. for each token t and head h
 *
 *     s_j  = scale * <q_{t,h}, K_j> + mask[t][j]        j < n_kv
 *     p_j  = exp(s_j - max_i s_i)                        (p_j = 0 when s_j = -inf)
 *     out  = sum_j p_j V_j / sum_j p_j
 *
 * The same pull request's GQA-collapse commit says the query rows are ordered
 * t-major, row r = t*n_head + h, and that the output lands in the
 * flash-attention node's [hd, n_head, n_tok] destination (ggml order, fastest
 * index first), i.e. out[(t*n_head + h)*hd + d].  Q is read in the same
 * t-major [n_tok][n_head][hd] order (the qkv_post handoff commit describes
 * Q's [M, Nq] layout as exactly that gather order).
 *
 * Readings where the pages are silent (listed again in the design notes):
 *   - a row whose every key is masked (-inf) yields an all-zero output row;
 *   - scale multiplies the dot product before the additive mask is added;
 *   - mask == NULL means an all-zero mask.
 *
 * Everything is fp64.  f16 inputs are widened exactly (binary16 -> binary64
 * is exact), f32 Q is widened exactly.  The only rounding of inputs is the
 * optional f32 -> f16 round-to-nearest-even of Q that reproduces the pages'
 * f16 gather (q_kind = ORACLE_Q_F32_ROUND_F16).  Sums run in index order.
 * Parallelism is over independent (t, h) rows only, so results do not depend
 * on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_Q_F32 = 0, ORACLE_Q_F16 = 1, ORACLE_Q_F32_ROUND_F16 = 2 };

/* IEEE 754 binary16 -> binary64, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 -> subnormal fraction * 2^-24; exponent 31 -> inf / NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even, from the definition:
 * the result is the representable binary16 value nearest to x (ties choose
 * the even significand); magnitudes at or above 65520 (half-way between the
 * largest finite 65504 and 2^16) overflow to infinity.  All arithmetic is in
 * double, where every step below is exact except the deliberate rint(). */
uint16_t oracle_f32_to_f16_rne(float xf)
{
    double x = (double)xf;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: multiples of 2^-24 (rint: ties to even) */
        double n = rint(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)n); /* n == 1024 encodes 2^-14 */
    }
    int ex;
    frexp(a, &ex);          /* a = m * 2^ex, m in [0.5, 1) -> a in [2^(ex-1), 2^ex) */
    int E = ex - 1;         /* unbiased exponent, -14 .. 15 */
    double n = rint(a * ldexp(1.0, 10 - E)); /* significand in units of 2^(E-10): 1024..2048 */
    if (n >= 2048.0) { n = 1024.0; E += 1; }
    if (E > 15)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)n - 1024));
}

/* A batched f32 -> f16 row copy (FlashRT PR #185, the commit batching the
 * persistent-KV tail copies): every element rounded on its own, nearest even,
 * exactly as one copy per row would. */
void oracle_f32_to_f16_rne_rows(const float *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_f32_to_f16_rne(src[i]);
}

/*
 * The query/KV producer ahead of the window (FlashRT PR #185: the prefix QKV
 * window fuses the q/k/v projections' epilogue -- RoPE, the query scale and
 * the f16 materialisations -- into "qkv_post", whose f16 Q rows in t-major
 * order are what the decode window reads).  RoPE in its NeoX form, written
 * from its definition: head vector x (length hd), position p, for i < hd/2
 *     a_i      = p * base^(-2i/hd)
 *     y_i      = x_i cos a_i - x_{i+hd/2} sin a_i
 *     y_{i+hd/2} = x_{i+hd/2} cos a_i + x_i sin a_i
 * qkv  : [n_tok][(n_head + 2*n_kv_head) * hd] f32 (query heads, key heads,
 *        value heads of each token)
 * pos  : [n_tok] positions
 * q    : [n_tok][n_head][hd]      rope(q) * q_scale       (fp64)
 * k, v : [n_kv_head][n_tok][hd]   rope(k), v unchanged    (fp64)
 */
void oracle_qkv_post_f64(const float *qkv, const int32_t *pos, int n_head, int n_kv_head,
                         int n_tok, int hd, double base, double q_scale,
                         double *q, double *k, double *v)
{
    const int half = hd / 2;
    const int width = (n_head + 2 * n_kv_head) * hd;
    for (int t = 0; t < n_tok; ++t) {
        const float *row = qkv + (size_t)t * width;
        for (int h = 0; h < n_head + 2 * n_kv_head; ++h) {
            const float *x = row + (size_t)h * hd;
            double *y;
            if (h < n_head)
                y = q + ((size_t)t * n_head + h) * hd;
            else if (h < n_head + n_kv_head)
                y = k + ((size_t)(h - n_head) * n_tok + t) * hd;
            else
                y = v + ((size_t)(h - n_head - n_kv_head) * n_tok + t) * hd;
            if (h >= n_head + n_kv_head) { /* values: no rotation */
                for (int d = 0; d < hd; ++d)
                    y[d] = (double)x[d];
                continue;
            }
            const double s = h < n_head ? q_scale : 1.0;
            for (int i = 0; i < half; ++i) {
                const double a = (double)pos[t] * pow(base, -2.0 * i / hd);
                const double c = cos(a), sn = sin(a);
                y[i] = ((double)x[i] * c - (double)x[i + half] * sn) * s;
                y[i + half] = ((double)x[i + half] * c + (double)x[i] * sn) * s;
            }
        }
    }
}

/* Element q[i] of the query tensor as fp64, for the three query kinds. */
static double q_at(const void *q, int q_kind, size_t i)
{
    if (q_kind == ORACLE_Q_F16)
        return oracle_f16_to_f64(((const uint16_t *)q)[i]);
    if (q_kind == ORACLE_Q_F32_ROUND_F16)
        return oracle_f16_to_f64(oracle_f32_to_f16_rne(((const float *)q)[i]));
    return (double)((const float *)q)[i];
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One attention instance with n_kv_head KV heads (grouped-query attention).
 *   q    : [n_tok][n_head][hd]       f32 (q_kind 0/2) or f16 bits (q_kind 1)
 *   k, v : [n_kv_head][n_kv][hd]     f16 bits
 *   mask : [n_tok][n_kv]             f16 bits, additive, shared by all heads;
 *                                    NULL = all zero
 *   out  : [n_tok][n_head][hd]       fp64
 * Query head h attends over KV head h / (n_head / n_kv_head): consecutive
 * query heads form a group sharing one KV head (the flash-attention node's
 * broadcast of KV heads over query heads).  n_kv_head = 1 is the pages' case,
 * one KV head shared by every query head.
 * Returns the number of threads used, or -1 on bad arguments / no memory.
 */
int oracle_decode_attn_gqa_f64(const void *q, int q_kind,
                               const uint16_t *k, const uint16_t *v, const uint16_t *mask,
                               double *out, int n_head, int n_kv_head, int n_tok, int n_kv,
                               int hd, double scale, int n_threads)
{
    if (!q || !k || !v || !out || n_head < 1 || n_tok < 1 || n_kv < 1 || hd < 1)
        return -1;
    if (n_kv_head < 1 || n_head % n_kv_head != 0)
        return -1;
    if (q_kind < ORACLE_Q_F32 || q_kind > ORACLE_Q_F32_ROUND_F16)
        return -1;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    const int group = n_head / n_kv_head; /* query heads per KV head */
    const size_t kv_elems = (size_t)n_kv_head * (size_t)n_kv * (size_t)hd;
    double *K = (double *)malloc(kv_elems * sizeof(double));
    double *V = (double *)malloc(kv_elems * sizeof(double));
    if (!K || !V) {
        free(K);
        free(V);
        return -1;
    }
    /* Widen K and V once (exact). */
    for (size_t i = 0; i < kv_elems; ++i) {
        K[i] = oracle_f16_to_f64(k[i]);
        V[i] = oracle_f16_to_f64(v[i]);
    }
    const int n_rows = n_head * n_tok;
    int used = 1;
    int failed = 0;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < n_rows; ++r) {
            /* per-row scratch: every thread reaches the worksharing loop */
            double *s = (double *)malloc((size_t)n_kv * sizeof(double));
            double *qr = (double *)malloc((size_t)hd * sizeof(double));
            double *acc = (double *)malloc((size_t)hd * sizeof(double));
            if (!s || !qr || !acc) {
#pragma omp atomic write
                failed = 1;
                free(s);
                free(qr);
                free(acc);
                continue;
            }
            const int t = r / n_head; /* row r = t*n_head + h (t-major) */
            const int h = r % n_head;
            /* this row's KV head */
            const double *Kh = K + (size_t)(h / group) * (size_t)n_kv * (size_t)hd;
            const double *Vh = V + (size_t)(h / group) * (size_t)n_kv * (size_t)hd;
            for (int e = 0; e < hd; ++e)
                qr[e] = q_at(q, q_kind, (size_t)r * hd + e);
            /* logits: scale * <q, K_j> + mask[t][j] */
            double m = -INFINITY;
            for (int j = 0; j < n_kv; ++j) {
                const double *kj = Kh + (size_t)j * hd;
                double dot = 0.0;
                for (int e = 0; e < hd; ++e)
                    dot += qr[e] * kj[e];
                double sj = scale * dot;
                if (mask)
                    sj += oracle_f16_to_f64(mask[(size_t)t * n_kv + j]);
                s[j] = sj;
                if (sj > m)
                    m = sj;
            }
            double *o = out + (size_t)r * hd;
            if (m == -INFINITY) { /* every key masked: zero row */
                for (int d = 0; d < hd; ++d)
                    o[d] = 0.0;
            } else {
                /* p_j = exp(s_j - m), l = sum p_j, acc = sum p_j V_j */
                double l = 0.0;
                for (int d = 0; d < hd; ++d)
                    acc[d] = 0.0;
                for (int j = 0; j < n_kv; ++j) {
                    if (s[j] == -INFINITY)
                        continue; /* exactly zero weight */
                    const double p = exp(s[j] - m);
                    l += p;
                    const double *vj = Vh + (size_t)j * hd;
                    for (int d = 0; d < hd; ++d)
                        acc[d] += p * vj[d];
                }
                for (int d = 0; d < hd; ++d)
                    o[d] = acc[d] / l;
            }
            free(s);
            free(qr);
            free(acc);
        }
    }
    free(K);
    free(V);
    return failed ? -1 : used;
}

/* The pages' case: one KV head shared by every query head. */
int oracle_decode_attn_f64(const void *q, int q_kind,
                           const uint16_t *k, const uint16_t *v, const uint16_t *mask,
                           double *out, int n_head, int n_tok, int n_kv, int hd,
                           double scale, int n_threads)
{
    return oracle_decode_attn_gqa_f64(q, q_kind, k, v, mask, out, n_head, 1, n_tok, n_kv, hd,
                                      scale, n_threads);
}
