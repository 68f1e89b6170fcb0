/*
 * Plain CPU oracle for query-aware sparse attention over a paged KV cache.
 * TEST INFRASTRUCTURE ONLY (see oracle.h): slow, fp64, written for reading.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC oracle.c -lm
 * (no -ffast-math, no FMA contraction: every fp64 operation is the IEEE one).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* bf16 values                                                               */
/* ------------------------------------------------------------------------ */

/* A bf16 pattern is the top half of an fp32 pattern; the value is exact in
 * fp64. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Total order used for the page summaries: numeric order, with -0 below +0
 * so that the min and the max of a set of patterns are unique patterns. */
static int bf16_below(uint16_t a, uint16_t b)
{
    double va = bf16_value(a), vb = bf16_value(b);
    if (va < vb) return 1;
    if (va > vb) return 0;
    return signbit(va) && !signbit(vb);
}

/* ------------------------------------------------------------------------ */
/* Exact summation                                                           */
/*                                                                           */
/* A fixed-point accumulator wide enough for any finite double: digit i has  */
/* weight 2^(32 i + XA_LO).  Each double is an integer M (|M| < 2^53) times  */
/* 2^e; its integer is added into the digits, so the accumulated value is    */
/* exact.  The result is rounded once, to nearest with ties to even.         */
/* ------------------------------------------------------------------------ */

#define XA_DIGITS 76
#define XA_LO (-1152)

typedef struct {
    int64_t d[XA_DIGITS];
} xacc;

/* floor(y / 2^32), written without relying on the shift of a negative. */
static int64_t floor_div_2p32(int64_t y)
{
    int64_t low = y & 0xffffffffLL; /* y mod 2^32, in [0, 2^32) */
    return (y - low) / ((int64_t)1 << 32);
}

/* Adds y * 2^(32 i) for |y| < 2^63. */
static void xa_add_at(xacc *a, int i, int64_t y)
{
    a->d[i] += y & 0xffffffffLL;
    a->d[i + 1] += floor_div_2p32(y);
}

static void xa_add(xacc *a, double x)
{
    if (x == 0.0) return;
    int e;
    double m = frexp(x, &e);                /* x = m 2^e, 1/2 <= |m| < 1 */
    int64_t M = (int64_t)ldexp(m, 53);      /* exact integer              */
    int off = (e - 53) - XA_LO;             /* x = M 2^(off + XA_LO)      */
    int di = off / 32, sh = off % 32;
    int64_t lo = M & 0xffffffffLL;          /* M = hi 2^32 + lo           */
    int64_t hi = floor_div_2p32(M);
    xa_add_at(a, di, lo * ((int64_t)1 << sh));
    xa_add_at(a, di + 1, hi * ((int64_t)1 << sh));
}

/* Brings every digit into [0, 2^32) except the top one, which keeps the
 * sign of the whole value. */
static void xa_normalize(xacc *a)
{
    for (int i = 0; i + 1 < XA_DIGITS; i++) {
        int64_t c = floor_div_2p32(a->d[i]);
        a->d[i] -= c * ((int64_t)1 << 32);
        a->d[i + 1] += c;
    }
}

static int xa_bit(const xacc *a, long i)
{
    if (i < 0) return 0;
    return (int)((a->d[i / 32] >> (i % 32)) & 1);
}

static double xa_round(xacc *a, int32_t *status)
{
    int neg = 0;
    xa_normalize(a);
    if (a->d[XA_DIGITS - 1] < 0) {
        neg = 1;
        for (int i = 0; i < XA_DIGITS; i++) a->d[i] = -a->d[i];
        xa_normalize(a);
    }
    int t = XA_DIGITS - 1;
    while (t >= 0 && a->d[t] == 0) t--;
    if (t < 0) return 0.0;
    int b = 31;
    while (((a->d[t] >> b) & 1) == 0) b--;
    long lead = 32L * t + b;               /* bit index of the leading one */

    uint64_t M = 0;                        /* the 53 bits from the leading one */
    for (long i = lead; i > lead - 53; i--) M = (M << 1) | (uint64_t)xa_bit(a, i);
    int round_bit = xa_bit(a, lead - 53);
    int sticky = 0;                        /* any one below the round bit */
    long p = lead - 54;
    if (p >= 0) {
        long q = p / 32;
        uint64_t mask = (2ULL << (p % 32)) - 1ULL;
        if (((uint64_t)a->d[q] & mask) != 0) sticky = 1;
        for (long i = 0; i < q && !sticky; i++)
            if (a->d[i] != 0) sticky = 1;
    }
    if (round_bit && (sticky || (M & 1ULL))) {
        M += 1;
        if (M == (1ULL << 53)) {
            M >>= 1;
            lead += 1;
        }
    }
    long e_lead = lead + XA_LO;            /* the value is in [2^e_lead, 2^(e_lead+1)) */
    if (e_lead < -1022 || e_lead > 1023) {
        if (status) *status = ORC_ERR_RANGE;
        return NAN;
    }
    double r = ldexp((double)M, (int)(e_lead - 52));
    return neg ? -r : r;
}

double orc_exact_sum(const double *x, int64_t n, int32_t *status)
{
    xacc a;
    memset(&a, 0, sizeof a);
    if (status) *status = ORC_OK;
    for (int64_t i = 0; i < n; i++) {
        if (!isfinite(x[i])) {
            if (status) *status = ORC_ERR_ARG;
            return NAN;
        }
        xa_add(&a, x[i]);
    }
    return xa_round(&a, status);
}

/* ------------------------------------------------------------------------ */
/* Geometry helpers                                                          */
/* ------------------------------------------------------------------------ */

static int64_t num_pages(int32_t L, int32_t ps)
{
    return L <= 0 ? 0 : ((int64_t)L + ps - 1) / ps;
}

static int check_layout(const orc_layout *lay)
{
    if (!lay) return 0;
    if (lay->num_pool_pages <= 0 || lay->page_size <= 0 || lay->num_kv_heads <= 0 ||
        lay->head_dim_k <= 0 || lay->head_dim_v <= 0)
        return 0;
    if (lay->v_from_k && lay->head_dim_v > lay->head_dim_k) return 0;
    return 1;
}

static int check_batch(const orc_layout *lay, const orc_batch *bat)
{
    if (!bat || bat->batch < 0) return 0;
    if (bat->batch == 0) return 1;
    if (!bat->page_table || !bat->seq_lens) return 0;
    if (bat->num_q_heads <= 0 || bat->num_q_heads % lay->num_kv_heads != 0) return 0;
    for (int32_t b = 0; b < bat->batch; b++) {
        int32_t L = bat->seq_lens[b];
        if (L < 0) return 0;
        int64_t P = num_pages(L, lay->page_size);
        if (P > bat->pt_stride) return 0;
        for (int64_t j = 0; j < P; j++) {
            int32_t phys = bat->page_table[(int64_t)b * bat->pt_stride + j];
            if (phys < 0 || phys >= lay->num_pool_pages) return 0;
        }
    }
    return 1;
}

static int is_static(const orc_policy *pol, int32_t g)
{
    return pol->static_heads != NULL && pol->static_heads[g] != 0;
}

/* Address of element (token t, channel d) of the key of page-head (phys, g). */
static const uint16_t *key_at(const orc_layout *lay, const uint16_t *k_pool,
                              int32_t phys, int32_t g, int32_t t)
{
    int64_t ph = (int64_t)phys * lay->num_kv_heads + g;
    return k_pool + (ph * lay->page_size + t) * lay->head_dim_k;
}

static double value_at(const orc_layout *lay, const uint16_t *k_pool,
                       const uint16_t *v_pool, int32_t phys, int32_t g,
                       int32_t t, int32_t dv)
{
    int64_t ph = (int64_t)phys * lay->num_kv_heads + g;
    if (lay->v_from_k) return bf16_value(key_at(lay, k_pool, phys, g, t)[dv]);
    return bf16_value(v_pool[(ph * lay->head_dim_v + dv) * lay->page_size + t]);
}

/* ------------------------------------------------------------------------ */
/* 2-bit quantised pages                                                     */
/*                                                                           */
/* 2-bit codes in groups of 32 (SCBench notes, the method table: KIVI with   */
/* 2 bits and group size 32; SparseEngine article, decode-hook paragraph:    */
/* KIVI keeps a quantised region and a full-precision residual region).      */
/* Readings: a group is 32 consecutive channels of one token (keys and       */
/* values alike); zero point m = the group minimum, step s = (max - min) / 3,*/
/* both stored as IEEE binary16; code = round-half-even((x - m) / s) clamped */
/* to 0..3 (s = 0: code 0), every step in IEEE binary32 with m and s as      */
/* stored; the value read back is m + code * s.  The last residual_pages     */
/* logical pages of a sequence stay full precision.                          */
/* ------------------------------------------------------------------------ */

/* IEEE binary16 pattern nearest to x (ties to even), from the format's
 * definition: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static uint16_t half_bits(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00;     /* past the largest finite (65504) by half a step or more */
    if (a < ldexp(1.0, -14)) {                  /* subnormal: a = n * 2^-24 */
        double n = nearbyint(a * ldexp(1.0, 24));
        return sign | (uint16_t)n;              /* n = 1024 is the smallest normal */
    }
    int e;
    frexp(a, &e);                               /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    double n = nearbyint(ldexp(a, 10 - E));     /* significand in [1024, 2048] */
    if (n == 2048.0) {
        n = 1024.0;
        E += 1;
    }
    if (E > 15) return sign | 0x7c00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0);
}

static double half_value(uint16_t h)
{
    int E = (h >> 10) & 0x1f, f = h & 0x3ff;
    double v;
    if (E == 0) v = ldexp((double)f, -24);
    else if (E == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), E - 25);
    return (h & 0x8000) ? -v : v;
}

/* One group of n values (bf16 values as binary32): its zero point, step and
 * codes. */
static void quant_group(const float *x, int n, uint16_t *m_out, uint16_t *s_out, uint8_t *codes)
{
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; i++) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    float d = mx - mn;
    float st = d / 3.0f;
    uint16_t m16 = half_bits(mn), s16 = half_bits(st);
    float m = (float)half_value(m16), sc = (float)half_value(s16);
    for (int i = 0; i < n; i++) {
        float c = 0.0f;
        if (sc != 0.0f) {
            float r = (x[i] - m) / sc;
            c = nearbyintf(r);
            if (c < 0.0f) c = 0.0f;
            if (c > 3.0f) c = 3.0f;
        }
        codes[i] = (uint8_t)c;
    }
    *m_out = m16;
    *s_out = s16;
}

/* Value read back from a quantised page: element i of a row of codes with
 * its group's (zero point, step) pair in meta (one pair per 32 elements). */
static double dequant(const uint8_t *codes, const uint16_t *meta, int32_t i)
{
    const uint16_t *ms = meta + 2 * (i / 32);
    return half_value(ms[0]) + (double)codes[i] * half_value(ms[1]);
}

/* ------------------------------------------------------------------------ */
/* Summaries and append                                                      */
/* ------------------------------------------------------------------------ */

int32_t orc_summaries(const orc_layout *lay, const orc_batch *bat,
                      const uint16_t *k_pool, uint16_t *summ_pool)
{
    if (!check_layout(lay) || !check_batch(lay, bat)) return ORC_ERR_ARG;
    if (bat->batch > 0 && (!k_pool || !summ_pool)) return ORC_ERR_ARG;
    const int32_t ps = lay->page_size, D = lay->head_dim_k;
    for (int32_t b = 0; b < bat->batch; b++) {
        int32_t L = bat->seq_lens[b];
        int64_t P = num_pages(L, ps);
        for (int64_t j = 0; j < P; j++) {
            int32_t phys = bat->page_table[(int64_t)b * bat->pt_stride + j];
            int32_t valid = (int32_t)((L - j * ps) < ps ? (L - j * ps) : ps);
            for (int32_t g = 0; g < lay->num_kv_heads; g++) {
                uint16_t *lo = summ_pool + ((int64_t)phys * lay->num_kv_heads + g) * 2 * D;
                uint16_t *hi = lo + D;
                for (int32_t d = 0; d < D; d++) {
                    uint16_t mn = key_at(lay, k_pool, phys, g, 0)[d];
                    uint16_t mx = mn;
                    for (int32_t t = 1; t < valid; t++) {
                        uint16_t v = key_at(lay, k_pool, phys, g, t)[d];
                        if (bf16_below(v, mn)) mn = v;
                        if (bf16_below(mx, v)) mx = v;
                    }
                    lo[d] = mn;
                    hi[d] = mx;
                }
            }
        }
    }
    return ORC_OK;
}

int32_t orc_append(const orc_layout *lay, const orc_batch *bat_before,
                   const uint16_t *k_new, const uint16_t *v_new,
                   uint16_t *k_pool, uint16_t *v_pool)
{
    if (!check_layout(lay) || !bat_before || bat_before->batch < 0) return ORC_ERR_ARG;
    const int32_t ps = lay->page_size, H = lay->num_kv_heads;
    for (int32_t b = 0; b < bat_before->batch; b++) {
        int32_t pos = bat_before->seq_lens[b];
        if (pos < 0 || pos / ps >= bat_before->pt_stride) return ORC_ERR_ARG;
        int32_t phys = bat_before->page_table[(int64_t)b * bat_before->pt_stride + pos / ps];
        if (phys < 0 || phys >= lay->num_pool_pages) return ORC_ERR_ARG;
        int32_t t = pos % ps;
        for (int32_t g = 0; g < H; g++) {
            uint16_t *kd = (uint16_t *)key_at(lay, k_pool, phys, g, t);
            for (int32_t d = 0; d < lay->head_dim_k; d++)
                kd[d] = k_new[((int64_t)b * H + g) * lay->head_dim_k + d];
            if (!lay->v_from_k) {
                int64_t ph = (int64_t)phys * H + g;
                for (int32_t dv = 0; dv < lay->head_dim_v; dv++)
                    v_pool[(ph * lay->head_dim_v + dv) * ps + t] =
                        v_new[((int64_t)b * H + g) * lay->head_dim_v + dv];
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Per-unit steps: one unit = (sequence b, KV head g)                        */
/* ------------------------------------------------------------------------ */

/* Group score of every page of the unit: row[j] for j < max_pages.
 * q holds nq query rows per head: q[b][i][h][:] for i < nq (nq = 1 for a
 * one-token step); the score is the maximum over every (i, h) of the group.
 * terms: scratch of head_dim_k doubles. */
static int unit_scores(const orc_layout *lay, const orc_batch *bat,
                       const orc_policy *pol, const uint16_t *q, int32_t nq,
                       const uint16_t *summ_pool, int32_t b, int32_t g,
                       double *row, int32_t max_pages, double *terms)
{
    const int32_t D = lay->head_dim_k;
    const int32_t G = bat->num_q_heads / lay->num_kv_heads;
    int32_t L = bat->seq_lens[b];
    int64_t P = num_pages(L, lay->page_size);
    for (int32_t j = 0; j < max_pages; j++) row[j] = -INFINITY;
    if (is_static(pol, g)) return ORC_OK;
    int64_t first = pol->n_sink_pages;          /* candidates: [first, last) */
    int64_t last = P - pol->n_local_pages;
    for (int64_t j = first; j < last; j++) {
        int32_t phys = bat->page_table[(int64_t)b * bat->pt_stride + j];
        const uint16_t *lo = summ_pool + ((int64_t)phys * lay->num_kv_heads + g) * 2 * D;
        const uint16_t *hi = lo + D;
        double best = -INFINITY;
        for (int32_t r = 0; r < nq * G; r++) {
            int32_t i = r / G, h = g * G + r % G;
            const uint16_t *qh = q + (((int64_t)b * nq + i) * bat->num_q_heads + h) * D;
            for (int32_t d = 0; d < D; d++) {
                double qd = bf16_value(qh[d]);
                double a = qd * bf16_value(lo[d]);   /* exact: 8-bit x 8-bit significands */
                double c = qd * bf16_value(hi[d]);
                terms[d] = a > c ? a : c;
            }
            int32_t st;
            double u = orc_exact_sum(terms, D, &st);
            if (st != ORC_OK) return st;
            if (u > best) best = u;
        }
        row[j] = best;
    }
    return ORC_OK;
}

typedef struct {
    double key;
    int32_t id;
} scored_page;

/* Higher score first; equal scores: lower logical id first. */
static int by_score_then_id(const void *pa, const void *pb)
{
    const scored_page *a = (const scored_page *)pa, *b = (const scored_page *)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

/* Marks the selected pages of the unit in flags[0..P) and returns how many. */
static int64_t unit_select_flags(const orc_layout *lay, const orc_batch *bat,
                                 const orc_policy *pol, const double *row,
                                 int32_t b, int32_t g, uint8_t *flags,
                                 scored_page *cand)
{
    const int32_t ps = lay->page_size;
    int32_t L = bat->seq_lens[b];
    int64_t P = num_pages(L, ps);
    memset(flags, 0, (size_t)P);
    if (is_static(pol, g)) {
        int64_t sink_end = pol->sink_tokens < L ? pol->sink_tokens : L;   /* t < sink_end */
        int64_t win_begin = (int64_t)L - pol->window_tokens;              /* t >= win_begin */
        if (win_begin < 0) win_begin = 0;
        for (int64_t j = 0; j < P; j++) {
            int64_t a = j * ps, e = (j + 1) * ps < L ? (j + 1) * ps : L;  /* tokens [a, e) */
            if (a < sink_end || e > win_begin) flags[j] = 1;
        }
    } else {
        for (int64_t j = 0; j < P && j < pol->n_sink_pages; j++) flags[j] = 1;
        for (int64_t j = P - pol->n_local_pages; j < P; j++)
            if (j >= 0) flags[j] = 1;
        int64_t n = 0;
        for (int64_t j = pol->n_sink_pages; j < P - pol->n_local_pages; j++) {
            cand[n].key = row[j];
            cand[n].id = (int32_t)j;
            n++;
        }
        qsort(cand, (size_t)n, sizeof(scored_page), by_score_then_id);
        int64_t take = pol->top_k < n ? pol->top_k : n;
        for (int64_t i = 0; i < take; i++) flags[cand[i].id] = 1;
    }
    int64_t count = 0;
    for (int64_t j = 0; j < P; j++) count += flags[j];
    return count;
}

/* Attention of the query heads of group g over the selected pages, for
 * query i of nq (q and out rows [b][i][h]).  Query i sits at position
 * L - nq + i and sees the tokens before and at it: it attends as a one-token
 * step of length L - nq + 1 + i would (nq = 1: the sequence's last token). */
static void unit_attend(const orc_layout *lay, const orc_batch *bat,
                        const orc_policy *pol, const uint16_t *q,
                        const uint16_t *k_pool, const uint16_t *v_pool,
                        const orc_quant *qz,
                        const int32_t *sel, int32_t count, double scale,
                        int32_t b, int32_t g, int32_t nq, int32_t i,
                        double *out, double *s_buf)
{
    const int32_t ps = lay->page_size, D = lay->head_dim_k, Dv = lay->head_dim_v;
    const int32_t G = bat->num_q_heads / lay->num_kv_heads;
    int64_t L = (int64_t)bat->seq_lens[b] - nq + 1 + i;
    int64_t sink_end = pol->sink_tokens < L ? pol->sink_tokens : L;
    int64_t win_begin = L - pol->window_tokens;
    int st = is_static(pol, g);
    /* pages below q_end are read back from the quantised pool */
    int64_t q_end = qz ? num_pages(bat->seq_lens[b], ps) - qz->residual_pages : 0;
    for (int32_t h = g * G; h < (g + 1) * G; h++) {
        const uint16_t *qh = q + (((int64_t)b * nq + i) * bat->num_q_heads + h) * D;
        double *o = out + (((int64_t)b * nq + i) * bat->num_q_heads + h) * Dv;
        /* scores of every attended token, in page then token order */
        int64_t n = 0;
        double m = -INFINITY;
        for (int32_t i = 0; i < count; i++) {
            int32_t j = sel[i];
            int32_t phys = bat->page_table[(int64_t)b * bat->pt_stride + j];
            for (int32_t t = 0; t < ps; t++) {
                int64_t pos = (int64_t)j * ps + t;
                int use = pos < L && (!st || pos < sink_end || pos >= win_begin);
                if (!use) {
                    s_buf[n++] = -INFINITY;
                    continue;
                }
                double dot = 0.0;
                if (j < q_end) {
                    int64_t row = ((int64_t)phys * lay->num_kv_heads + g) * ps + t;
                    const uint8_t *kc = qz->k_codes + row * D;
                    const uint16_t *km = qz->k_meta + row * (D / 32) * 2;
                    for (int32_t d = 0; d < D; d++) dot += bf16_value(qh[d]) * dequant(kc, km, d);
                } else {
                    const uint16_t *kt = key_at(lay, k_pool, phys, g, t);
                    for (int32_t d = 0; d < D; d++) dot += bf16_value(qh[d]) * bf16_value(kt[d]);
                }
                s_buf[n] = scale * dot;
                if (s_buf[n] > m) m = s_buf[n];
                n++;
            }
        }
        for (int32_t dv = 0; dv < Dv; dv++) o[dv] = 0.0;
        if (m == -INFINITY) continue;                 /* no token: output 0 */
        double denom = 0.0;
        n = 0;
        for (int32_t i = 0; i < count; i++) {
            int32_t j = sel[i];
            int32_t phys = bat->page_table[(int64_t)b * bat->pt_stride + j];
            for (int32_t t = 0; t < ps; t++, n++) {
                if (s_buf[n] == -INFINITY) continue;
                double w = exp(s_buf[n] - m);
                denom += w;
                if (j < q_end) {
                    int64_t row = ((int64_t)phys * lay->num_kv_heads + g) * ps + t;
                    const uint8_t *vc = qz->v_codes + row * Dv;
                    const uint16_t *vm = qz->v_meta + row * (Dv / 32) * 2;
                    for (int32_t dv = 0; dv < Dv; dv++) o[dv] += w * dequant(vc, vm, dv);
                } else {
                    for (int32_t dv = 0; dv < Dv; dv++)
                        o[dv] += w * value_at(lay, k_pool, v_pool, phys, g, t, dv);
                }
            }
        }
        for (int32_t dv = 0; dv < Dv; dv++) o[dv] /= denom;
    }
}

/* ------------------------------------------------------------------------ */
/* Public entry points                                                       */
/* ------------------------------------------------------------------------ */

int32_t orc_max_sel(const orc_layout *lay, const orc_policy *pol, int32_t max_pages)
{
    if (!check_layout(lay) || !pol) return ORC_ERR_ARG;
    int64_t qa = (int64_t)pol->n_sink_pages + pol->n_local_pages + pol->top_k;
    int64_t ps = lay->page_size;
    int64_t stat = (pol->sink_tokens + ps - 1) / ps + (pol->window_tokens + ps - 1) / ps + 1;
    int64_t m = qa > stat ? qa : stat;
    if (m > max_pages) m = max_pages;
    return (int32_t)m;
}

static int check_policy(const orc_policy *pol)
{
    return pol && pol->n_sink_pages >= 0 && pol->n_local_pages >= 0 && pol->top_k >= 0 &&
           pol->sink_tokens >= 0 && pol->window_tokens >= 0;
}

static int32_t scores_nq(const orc_layout *lay, const orc_batch *bat,
                         const orc_policy *pol, int32_t nq, const uint16_t *q,
                         const uint16_t *summ_pool, double *scores, int32_t max_pages)
{
    if (!check_layout(lay) || !check_batch(lay, bat) || !check_policy(pol) || nq < 1) return ORC_ERR_ARG;
    if (bat->batch == 0) return ORC_OK;
    if (!q || !summ_pool || !scores) return ORC_ERR_ARG;
    for (int32_t b = 0; b < bat->batch; b++)
        if (num_pages(bat->seq_lens[b], lay->page_size) > max_pages) return ORC_ERR_ARG;
    double *terms = (double *)malloc(sizeof(double) * (size_t)lay->head_dim_k);
    if (!terms) return ORC_ERR_ARG;
    int32_t rc = ORC_OK;
    for (int32_t b = 0; b < bat->batch && rc == ORC_OK; b++)
        for (int32_t g = 0; g < lay->num_kv_heads && rc == ORC_OK; g++)
            rc = unit_scores(lay, bat, pol, q, nq, summ_pool, b, g,
                             scores + ((int64_t)b * lay->num_kv_heads + g) * max_pages,
                             max_pages, terms);
    free(terms);
    return rc;
}

int32_t orc_scores(const orc_layout *lay, const orc_batch *bat,
                   const orc_policy *pol, const uint16_t *q,
                   const uint16_t *summ_pool, double *scores, int32_t max_pages)
{
    return scores_nq(lay, bat, pol, 1, q, summ_pool, scores, max_pages);
}

int32_t orc_scores_multi(const orc_layout *lay, const orc_batch *bat,
                         const orc_policy *pol, int32_t nq, const uint16_t *q,
                         const uint16_t *summ_pool, double *scores, int32_t max_pages)
{
    return scores_nq(lay, bat, pol, nq, q, summ_pool, scores, max_pages);
}

int32_t orc_select(const orc_layout *lay, const orc_batch *bat,
                   const orc_policy *pol, const double *scores, int32_t max_pages,
                   int32_t *sel, int32_t *sel_count, int32_t max_sel)
{
    if (!check_layout(lay) || !check_batch(lay, bat) || !check_policy(pol)) return ORC_ERR_ARG;
    if (bat->batch == 0) return ORC_OK;
    if (!scores || !sel || !sel_count || max_sel < 0) return ORC_ERR_ARG;
    for (int32_t b = 0; b < bat->batch; b++)
        if (num_pages(bat->seq_lens[b], lay->page_size) > max_pages) return ORC_ERR_ARG;
    uint8_t *flags = (uint8_t *)malloc((size_t)max_pages + 1);
    scored_page *cand = (scored_page *)malloc(sizeof(scored_page) * ((size_t)max_pages + 1));
    int32_t rc = (flags && cand) ? ORC_OK : ORC_ERR_ARG;
    for (int32_t b = 0; b < bat->batch && rc == ORC_OK; b++) {
        int64_t P = num_pages(bat->seq_lens[b], lay->page_size);
        for (int32_t g = 0; g < lay->num_kv_heads && rc == ORC_OK; g++) {
            int64_t u = (int64_t)b * lay->num_kv_heads + g;
            int64_t count = unit_select_flags(lay, bat, pol, scores + u * max_pages, b, g, flags, cand);
            if (count > max_sel) {
                rc = ORC_ERR_MAX_SEL;
                break;
            }
            int32_t *row = sel + u * max_sel;
            int64_t n = 0;
            for (int64_t j = 0; j < P; j++)
                if (flags[j]) row[n++] = (int32_t)j;
            for (; n < max_sel; n++) row[n] = -1;
            sel_count[u] = (int32_t)count;
        }
    }
    free(flags);
    free(cand);
    return rc;
}

/* Draft queries share the unit's selection.  For a static head the page set
 * is the union of the queries' own sink + window sets; the queries' windows
 * [L_i - w, L_i) end at L_i = L - nq + 1 ... L, so for w >= 1 they chain
 * into one window of w + nq - 1 tokens ending at L (w = 0: all empty). */
int32_t orc_select_multi(const orc_layout *lay, const orc_batch *bat,
                         const orc_policy *pol, int32_t nq, const double *scores, int32_t max_pages,
                         int32_t *sel, int32_t *sel_count, int32_t max_sel)
{
    if (!pol || nq < 1) return ORC_ERR_ARG;
    orc_policy wide = *pol;
    if (pol->window_tokens > 0) wide.window_tokens = pol->window_tokens + nq - 1;
    return orc_select(lay, bat, &wide, scores, max_pages, sel, sel_count, max_sel);
}

static int32_t attend_nq(const orc_layout *lay, const orc_batch *bat,
                         const orc_policy *pol, int32_t nq, const uint16_t *q,
                         const uint16_t *k_pool, const uint16_t *v_pool, const orc_quant *qz,
                         const int32_t *sel, const int32_t *sel_count, int32_t max_sel,
                         double scale, double *out)
{
    if (!check_layout(lay) || !check_batch(lay, bat) || !check_policy(pol) || nq < 1) return ORC_ERR_ARG;
    if (bat->batch == 0) return ORC_OK;
    if (!q || !k_pool || (!v_pool && !lay->v_from_k) || !sel || !sel_count || !out) return ORC_ERR_ARG;
    double *s_buf = (double *)malloc(sizeof(double) * ((size_t)max_sel * lay->page_size + 1));
    if (!s_buf) return ORC_ERR_ARG;
    int32_t rc = ORC_OK;
    for (int32_t b = 0; b < bat->batch && rc == ORC_OK; b++) {
        int64_t P = num_pages(bat->seq_lens[b], lay->page_size);
        for (int32_t g = 0; g < lay->num_kv_heads; g++) {
            int64_t u = (int64_t)b * lay->num_kv_heads + g;
            int32_t count = sel_count[u];
            const int32_t *row = sel + u * max_sel;
            if (count < 0 || count > max_sel) { rc = ORC_ERR_ARG; break; }
            for (int32_t i = 0; i < count; i++)
                if (row[i] < 0 || row[i] >= P) rc = ORC_ERR_ARG;
            if (rc != ORC_OK) break;
            for (int32_t i = 0; i < nq; i++)
                unit_attend(lay, bat, pol, q, k_pool, v_pool, qz, row, count, scale, b, g, nq, i, out, s_buf);
        }
    }
    free(s_buf);
    return rc;
}

int32_t orc_attend(const orc_layout *lay, const orc_batch *bat,
                   const orc_policy *pol, const uint16_t *q,
                   const uint16_t *k_pool, const uint16_t *v_pool,
                   const int32_t *sel, const int32_t *sel_count, int32_t max_sel,
                   double scale, double *out)
{
    return attend_nq(lay, bat, pol, 1, q, k_pool, v_pool, NULL, sel, sel_count, max_sel, scale, out);
}

int32_t orc_attend_multi(const orc_layout *lay, const orc_batch *bat,
                         const orc_policy *pol, int32_t nq, const uint16_t *q,
                         const uint16_t *k_pool, const uint16_t *v_pool,
                         const int32_t *sel, const int32_t *sel_count, int32_t max_sel,
                         double scale, double *out)
{
    return attend_nq(lay, bat, pol, nq, q, k_pool, v_pool, NULL, sel, sel_count, max_sel, scale, out);
}

int32_t orc_quantize(const orc_layout *lay, const orc_batch *bat, int32_t residual_pages,
                     const uint16_t *k_pool, const uint16_t *v_pool, uint8_t *k_codes, uint16_t *k_meta,
                     uint8_t *v_codes, uint16_t *v_meta)
{
    if (!check_layout(lay) || !check_batch(lay, bat) || residual_pages < 1) return ORC_ERR_ARG;
    if (lay->v_from_k || lay->head_dim_k % 32 || lay->head_dim_v % 32) return ORC_ERR_ARG;
    if (bat->batch == 0) return ORC_OK;
    if (!k_pool || !v_pool || !k_codes || !k_meta || !v_codes || !v_meta) return ORC_ERR_ARG;
    const int32_t ps = lay->page_size, D = lay->head_dim_k, Dv = lay->head_dim_v;
    float x[32];
    for (int32_t b = 0; b < bat->batch; b++) {
        int64_t P = num_pages(bat->seq_lens[b], ps);
        for (int64_t j = 0; j < P - residual_pages; j++) {   /* complete pages: j < P - 1 */
            int32_t phys = bat->page_table[(int64_t)b * bat->pt_stride + j];
            for (int32_t g = 0; g < lay->num_kv_heads; g++)
                for (int32_t t = 0; t < ps; t++) {
                    int64_t row = ((int64_t)phys * lay->num_kv_heads + g) * ps + t;
                    const uint16_t *kt = key_at(lay, k_pool, phys, g, t);
                    for (int32_t c = 0; c < D; c += 32) {
                        for (int32_t i = 0; i < 32; i++) x[i] = (float)bf16_value(kt[c + i]);
                        uint16_t *ms = k_meta + (row * (D / 32) + c / 32) * 2;
                        quant_group(x, 32, &ms[0], &ms[1], k_codes + row * D + c);
                    }
                    for (int32_t c = 0; c < Dv; c += 32) {
                        for (int32_t i = 0; i < 32; i++)
                            x[i] = (float)value_at(lay, k_pool, v_pool, phys, g, t, c + i);
                        uint16_t *ms = v_meta + (row * (Dv / 32) + c / 32) * 2;
                        quant_group(x, 32, &ms[0], &ms[1], v_codes + row * Dv + c);
                    }
                }
        }
    }
    return ORC_OK;
}

int32_t orc_attend_quant(const orc_layout *lay, const orc_batch *bat, const orc_policy *pol,
                         int32_t residual_pages, const uint16_t *q, const uint16_t *k_pool,
                         const uint16_t *v_pool, const uint8_t *k_codes, const uint16_t *k_meta,
                         const uint8_t *v_codes, const uint16_t *v_meta, const int32_t *sel,
                         const int32_t *sel_count, int32_t max_sel, double scale, double *out)
{
    if (residual_pages < 1 || lay == NULL || lay->v_from_k || lay->head_dim_k % 32 || lay->head_dim_v % 32)
        return ORC_ERR_ARG;
    if (!k_codes || !k_meta || !v_codes || !v_meta) return ORC_ERR_ARG;
    orc_quant qz = {residual_pages, k_codes, k_meta, v_codes, v_meta};
    return attend_nq(lay, bat, pol, 1, q, k_pool, v_pool, &qz, sel, sel_count, max_sel, scale, out);
}

uint16_t orc_half_bits(double x) { return half_bits(x); }

int32_t orc_decode(const orc_layout *lay, const orc_batch *bat,
                   const orc_policy *pol, const uint16_t *q,
                   const uint16_t *k_pool, const uint16_t *v_pool,
                   const uint16_t *summ_pool, double scale, double *out,
                   int32_t *sel, int32_t *sel_count, int32_t max_sel,
                   int32_t num_threads)
{
    if (!check_layout(lay) || !check_batch(lay, bat) || !check_policy(pol)) return ORC_ERR_ARG;
    if (bat->batch == 0) return ORC_OK;
    if (!q || !k_pool || (!v_pool && !lay->v_from_k) || !out) return ORC_ERR_ARG;
    int64_t max_pages = 0;
    for (int32_t b = 0; b < bat->batch; b++) {
        int64_t P = num_pages(bat->seq_lens[b], lay->page_size);
        if (P > max_pages) max_pages = P;
    }
    int need_summ = 0;
    for (int32_t g = 0; g < lay->num_kv_heads; g++) need_summ |= !is_static(pol, g);
    if (need_summ && !summ_pool) return ORC_ERR_ARG;
    if (max_sel <= 0) max_sel = (int32_t)max_pages;
    if (num_threads <= 0) num_threads = 1;
    const int64_t units = (int64_t)bat->batch * lay->num_kv_heads;
    int32_t rc = ORC_OK;

#pragma omp parallel num_threads(num_threads)
    {
        double *row = (double *)malloc(sizeof(double) * ((size_t)max_pages + 1));
        double *terms = (double *)malloc(sizeof(double) * (size_t)lay->head_dim_k);
        uint8_t *flags = (uint8_t *)malloc((size_t)max_pages + 1);
        scored_page *cand = (scored_page *)malloc(sizeof(scored_page) * ((size_t)max_pages + 1));
        int32_t *list = (int32_t *)malloc(sizeof(int32_t) * ((size_t)max_pages + 1));
        double *s_buf = (double *)malloc(sizeof(double) * ((size_t)max_pages * lay->page_size + 1));
        int ok = row && terms && flags && cand && list && s_buf;
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; u++) {
            if (!ok) continue;
            int32_t b = (int32_t)(u / lay->num_kv_heads), g = (int32_t)(u % lay->num_kv_heads);
            int64_t P = num_pages(bat->seq_lens[b], lay->page_size);
            int st = unit_scores(lay, bat, pol, q, 1, summ_pool, b, g, row, (int32_t)max_pages, terms);
            if (st != ORC_OK) {
#pragma omp critical
                rc = st;
                continue;
            }
            int64_t count = unit_select_flags(lay, bat, pol, row, b, g, flags, cand);
            int64_t n = 0;
            for (int64_t j = 0; j < P; j++)
                if (flags[j]) list[n++] = (int32_t)j;
            if (sel && sel_count) {
                if (count > max_sel) {
#pragma omp critical
                    rc = ORC_ERR_MAX_SEL;
                    continue;
                }
                for (int64_t i = 0; i < max_sel; i++) sel[u * max_sel + i] = i < n ? list[i] : -1;
                sel_count[u] = (int32_t)count;
            }
            unit_attend(lay, bat, pol, q, k_pool, v_pool, NULL, list, (int32_t)count, scale, b, g, 1, 0, out, s_buf);
        }
        if (!ok) {
#pragma omp critical
            rc = ORC_ERR_ARG;
        }
        free(row);
        free(terms);
        free(flags);
        free(cand);
        free(list);
        free(s_buf);
    }
    return rc;
}
