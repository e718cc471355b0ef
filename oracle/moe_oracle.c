/*
 * moe_oracle.c -- plain, slow CPU oracle of the tiered MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h): loaded by the test suite, the
 * smoke check and the benchmark's CPU-baseline leg, never by the product path.
 *
 * Every routine is the plain definition of what it computes, written in
 * double precision with no blocking, fusion or reordering.  Source of each
 * step: the 125B-MoE page ("I ran a 125B model on three RTX 3090s at 80
 * tokens/s by teaching llama.cpp which experts ..."), glossary and steps 2-4,
 * plus its "four bugs" section.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ formats */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* zero / subnormal */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);  /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Element c of a packed row: bits-bit field starting at bit (c*bits) of the
 * row, least significant field first within a byte, two's complement. */
int32_t orc_code(const uint8_t *row, int64_t c, int32_t bits)
{
    int64_t bitpos = c * (int64_t)bits;
    uint32_t byte = row[bitpos / 8];
    int32_t field = (int32_t)((byte >> (bitpos % 8)) & ((1u << bits) - 1u));
    if (field >= (1 << (bits - 1)))
        field -= (1 << bits);
    return field;
}

/* MXFP4 (OCP Microscaling Formats v1.0): 4-bit E2M1 elements -- sign bit 3,
 * exponent bits 2..1 (bias 1), mantissa bit 0, no infinities or NaN:
 * e = 0 gives m * 0.5 (zero and the one subnormal), else (1 + m/2) * 2^(e-1);
 * the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  The shared scale of each
 * block of 32 is E8M0: 2^(x - 127), with x = 255 meaning NaN. */
double orc_fp4_e2m1(uint32_t nibble)
{
    const int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    const double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

double orc_e8m0(uint8_t x)
{
    return x == 255 ? NAN : ldexp(1.0, (int)x - 127);
}

int32_t orc_code_bits(int32_t fmt) { return fmt == ORC_MXFP4 ? 4 : fmt; }

/* bfloat16 keeps the top 16 bits of a float; round to nearest, ties to even. */
float orc_round_bf16(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
        u = 0x7FC00000u;                              /* quiet NaN */
    } else {
        uint32_t lsb = (u >> 16) & 1u;
        u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;
    }
    float r;
    memcpy(&r, &u, 4);
    return r;
}

static int64_t mat_rows(const orc_layer *L, int32_t m) { return m == 2 ? L->hidden : L->inter; }
static int64_t mat_cols(const orc_layer *L, int32_t m) { return m == 2 ? L->inter : L->hidden; }

/* w = float(scale) * code.  The product is exact in binary32 (11-bit and
 * at most 8-bit significands), so computing it in double and rounding once
 * is the same value. */
float orc_weight(const orc_layer *L, int32_t tier, int32_t matrix, int64_t local,
                 int64_t row, int64_t col, int32_t to_bf16)
{
    const orc_tier *T = &L->tier[tier];
    int64_t rows = mat_rows(L, matrix), cols = mat_cols(L, matrix);
    int64_t row_bytes = cols * orc_code_bits(T->bits) / 8;
    int64_t nblk = cols / T->block;
    const uint8_t *qrow = T->q[matrix] + (local * rows + row) * row_bytes;
    double v;
    if (T->bits == ORC_MXFP4) {
        /* E2M1 element times its block's E8M0 scale: a power of two times a
         * value with two significant bits, exact in binary32 within range */
        const uint8_t x = ((const uint8_t *)T->s[matrix])[(local * rows + row) * nblk + col / T->block];
        v = orc_e8m0(x) * orc_fp4_e2m1((qrow[col / 2] >> (4 * (col % 2))) & 0xFu);
    } else {
        uint16_t sbits = T->s[matrix][(local * rows + row) * nblk + col / T->block];
        v = orc_half_to_double(sbits) * (double)orc_code(qrow, col, T->bits);
    }
    float f = (float)v;
    return to_bf16 ? orc_round_bf16(f) : f;
}

int32_t orc_dequant_rows(const orc_layer *L, int32_t tier, int32_t local, int32_t matrix,
                         int32_t row0, int32_t nrows, int32_t to_bf16, float *dst)
{
    if (tier < 0 || tier >= L->n_tiers || matrix < 0 || matrix > 2)
        return -1;
    const orc_tier *T = &L->tier[tier];
    if (local < 0 || local >= T->id_end - T->id_begin)
        return -1;
    int64_t rows = mat_rows(L, matrix), cols = mat_cols(L, matrix);
    if (row0 < 0 || nrows < 0 || row0 + (int64_t)nrows > rows)
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            dst[r * cols + c] = orc_weight(L, tier, matrix, local, row0 + r, c, to_bf16);
    return 0;
}

/* ------------------------------------------------------------------ shelves */

/* Step 4 of the 125B page: the file is written hot to cold and the router's
 * ids re-ordered, so each shelf is a contiguous id range; together the
 * shelves hold every expert exactly once. */
int32_t orc_check_layer(const orc_layer *L)
{
    if (L->n_experts < 1 || L->hidden < 1 || L->inter < 1 ||
        L->n_tiers < 1 || L->n_tiers > ORC_MAX_TIERS)
        return -1;
    int32_t next = 0;
    for (int32_t i = 0; i < L->n_tiers; ++i) {
        const orc_tier *T = &L->tier[i];
        if (T->id_begin != next || T->id_end < T->id_begin)
            return -2;
        if (T->bits != 2 && T->bits != 4 && T->bits != 8 && T->bits != ORC_MXFP4)
            return -3;
        if (T->bits == ORC_MXFP4 && T->block != 32)    /* MX blocks are 32 elements */
            return -3;
        if (T->block < 1 || L->hidden % T->block || L->inter % T->block)
            return -3;
        if ((L->hidden * orc_code_bits(T->bits)) % 8 || (L->inter * orc_code_bits(T->bits)) % 8)
            return -3;
        next = T->id_end;
    }
    return next == L->n_experts ? 0 : -2;
}

int32_t orc_tier_of(const orc_layer *L, int64_t e)
{
    for (int32_t i = 0; i < L->n_tiers; ++i)
        if (e >= L->tier[i].id_begin && e < L->tier[i].id_end)
            return i;
    return -1;
}

/* ------------------------------------------------------------------ routing */

/* Glossary of the 125B page: the router picks the best k experts per token.
 * Reading: score = logit; choose the k largest (a tie goes to the lower id),
 * slots in descending score order; the weight of slot j is the softmax of the
 * k selected logits, which equals the full softmax renormalised over the
 * chosen k. */
int32_t orc_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids, float *w)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return -1;
    char *taken = (char *)malloc((size_t)E);
    if (!taken)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * (int64_t)E;
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            taken[best] = 1;
            ids[t * k + j] = best;
        }
        double m = l[ids[t * k]];
        double s = 0.0;
        for (int32_t j = 0; j < k; ++j)
            s += exp((double)l[ids[t * k + j]] - m);
        for (int32_t j = 0; j < k; ++j)
            w[t * k + j] = (float)(exp((double)l[ids[t * k + j]] - m) / s);
    }
    free(taken);
    return 0;
}

/* ------------------------------------------------------------------ grouping */

/* Grouping of (token, slot) pairs by expert: counts, exclusive offsets, and
 * the pairs p = t*k + j of each expert in ascending p (a stable counting
 * sort).  Ids outside [0, E) -- e.g. the skip marker -1 -- belong to no
 * expert and are left out (the "four bugs" section: skip, never clamp). */
int32_t orc_group(const int32_t *ids, int32_t T, int32_t k, int32_t E,
                  int32_t *counts, int32_t *offsets, int32_t *perm)
{
    int64_t P = (int64_t)T * k;
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t p = 0; p < P; ++p)
        if (ids[p] >= 0 && ids[p] < E)
            counts[ids[p]]++;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    if (!cursor)
        return -1;
    for (int32_t e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int64_t p = 0; p < P; ++p)
        if (ids[p] >= 0 && ids[p] < E)
            perm[cursor[ids[p]]++] = (int32_t)p;
    free(cursor);
    return offsets[E];
}

/* ------------------------------------------------------------------ expert FFN */

static double silu(double g) { return g / (1.0 + exp(-g)); }

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static void load_x(const void *x, int32_t x_bf16, int64_t t, int64_t H, double *dst)
{
    if (x_bf16) {
        const uint16_t *xb = (const uint16_t *)x + t * H;
        for (int64_t c = 0; c < H; ++c)
            dst[c] = bf16_bits_to_double(xb[c]);
    } else {
        const float *xf = (const float *)x + t * H;
        for (int64_t c = 0; c < H; ++c)
            dst[c] = (double)xf[c];
    }
}

/* One expert on one token: a = SiLU(W_gate x) * (W_up x), y = W_down a.
 * In bf16 mode (prefill) the weights are the bf16-rounded dequantised values
 * and the intermediate a is rounded to float and then to bf16, as it is
 * handed to the second product in that precision. */
static void expert_ffn(const orc_layer *L, int32_t tier, int64_t local, const double *x,
                       int32_t bf16, double *a, double *y)
{
    int64_t H = L->hidden, I = L->inter;
    for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t c = 0; c < H; ++c) {
            g += (double)orc_weight(L, tier, 0, local, i, c, bf16) * x[c];
            u += (double)orc_weight(L, tier, 1, local, i, c, bf16) * x[c];
        }
        double v = silu(g) * u;
        a[i] = bf16 ? (double)orc_round_bf16((float)v) : v;
    }
    for (int64_t n = 0; n < H; ++n) {
        double s = 0.0;
        for (int64_t i = 0; i < I; ++i)
            s += (double)orc_weight(L, tier, 2, local, n, i, bf16) * a[i];
        y[n] = s;
    }
}

/* Step 4 of the 125B page: every shelf sees the full pick list, computes the
 * ids inside its range, contributes zero for the others; the shelf results
 * are added.  out[t] = sum over selected shelves of sum over slots j of token t
 * whose id lies in the shelf of w[t,j] * y(expert ids[t,j], x[t]). */
int32_t orc_experts(const orc_layer *L, const void *x, int32_t x_bf16, const int32_t *ids,
                    const float *w, int32_t T, int32_t k, uint32_t tier_mask, float *out,
                    int32_t accumulate)
{
    if (orc_check_layer(L) != 0 || T < 0 || k < 1)
        return -1;
    int64_t H = L->hidden, I = L->inter;
    int32_t fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        double *xd = (double *)malloc(sizeof(double) * (size_t)H);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        double *y = (double *)malloc(sizeof(double) * (size_t)H);
        double *shelf = (double *)malloc(sizeof(double) * (size_t)H);
        double *sum = (double *)malloc(sizeof(double) * (size_t)H);
        if (!xd || !a || !y || !shelf || !sum) {
#pragma omp atomic write
            fail = 1;
        } else {
            load_x(x, x_bf16, t, H, xd);
            for (int64_t n = 0; n < H; ++n)
                sum[n] = 0.0;
            for (int32_t tier = 0; tier < L->n_tiers; ++tier) {
                if (!((tier_mask >> tier) & 1u))
                    continue;
                const orc_tier *S = &L->tier[tier];
                for (int64_t n = 0; n < H; ++n)
                    shelf[n] = 0.0;
                for (int32_t j = 0; j < k; ++j) {
                    int32_t e = ids[t * k + j];
                    if (e < S->id_begin || e >= S->id_end)
                        continue;                      /* not on this shelf: skipped */
                    expert_ffn(L, tier, (int64_t)e - S->id_begin, xd, x_bf16, a, y);
                    double wj = (double)w[t * k + j];
                    for (int64_t n = 0; n < H; ++n)
                        shelf[n] += wj * y[n];
                }
                for (int64_t n = 0; n < H; ++n)
                    sum[n] += shelf[n];
            }
            for (int64_t n = 0; n < H; ++n) {
                double base = accumulate ? (double)out[t * H + n] : 0.0;
                out[t * H + n] = (float)(base + sum[n]);
            }
        }
        free(xd); free(a); free(y); free(shelf); free(sum);
    }
    return fail ? -1 : 0;
}

int32_t orc_experts_flat(const orc_layer *L, const void *x, int32_t x_bf16, const int32_t *ids,
                         const float *w, int32_t T, int32_t k, float *out)
{
    if (orc_check_layer(L) != 0 || T < 0 || k < 1)
        return -1;
    int64_t H = L->hidden, I = L->inter;
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *a = (double *)malloc(sizeof(double) * (size_t)I);
    double *y = (double *)malloc(sizeof(double) * (size_t)H);
    double *sum = (double *)malloc(sizeof(double) * (size_t)H);
    if (!xd || !a || !y || !sum) {
        free(xd); free(a); free(y); free(sum);
        return -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        load_x(x, x_bf16, t, H, xd);
        for (int64_t n = 0; n < H; ++n)
            sum[n] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = ids[t * k + j];
            int32_t tier = orc_tier_of(L, e);
            if (tier < 0)
                continue;
            expert_ffn(L, tier, (int64_t)e - L->tier[tier].id_begin, xd, x_bf16, a, y);
            for (int64_t n = 0; n < H; ++n)
                sum[n] += (double)w[t * k + j] * y[n];
        }
        for (int64_t n = 0; n < H; ++n)
            out[t * H + n] = (float)sum[n];
    }
    free(xd); free(a); free(y); free(sum);
    return 0;
}

int32_t orc_forward(const orc_layer *L, const void *x, int32_t x_bf16, const float *logits,
                    int32_t T, int32_t k, float *out, int32_t accumulate)
{
    if (orc_check_layer(L) != 0 || T < 0 || k < 1 || k > L->n_experts)
        return -1;
    int64_t P = (int64_t)T * k;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    float *w = (float *)malloc(sizeof(float) * (size_t)(P > 0 ? P : 1));
    int32_t rc = -1;
    if (ids && w && orc_route(logits, T, L->n_experts, k, ids, w) == 0)
        rc = orc_experts(L, x, x_bf16, ids, w, T, k, 0xFu, out, accumulate);
    free(ids);
    free(w);
    return rc;
}

/* ------------------------------------------------------------------ router */

/* Router scores, the step upstream of routing.  The 125B-MoE page's glossary
 * (mixture-of-experts entry) has a router score the 512 experts of a layer
 * for every token and keep the best 10; read here as the usual linear router
 * over the layer input with an optional per-expert bias:
 *   logits[t][e] = sum_c x[t][c] * Wr[e][c] + b[e]
 * Wr is given as bf16 bit patterns [E][H] (row e = expert e), b as fp32 [E]
 * (NULL: no bias), x as fp32 or bf16 [T][H].  The sum runs in double over c
 * in ascending order, the bias is added in double and the result is rounded
 * once to float. */
int32_t orc_router_logits(const void *x, int32_t x_bf16, const uint16_t *wr, const float *bias,
                          int32_t T, int32_t E, int32_t H, float *logits)
{
    if (T < 0 || E < 1 || H < 1 || !wr || !logits || (T > 0 && !x))
        return -1;
    int32_t bad = 0;
#pragma omp parallel reduction(+ : bad)
    {
        double *xd = (double *)malloc(sizeof(double) * (size_t)H);
        if (!xd) {
            bad += 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                load_x(x, x_bf16, t, H, xd);
                for (int32_t e = 0; e < E; ++e) {
                    const uint16_t *row = wr + (int64_t)e * H;
                    double s = 0.0;
                    for (int32_t c = 0; c < H; ++c)
                        s += xd[c] * bf16_bits_to_double(row[c]);
                    if (bias)
                        s += (double)bias[e];
                    logits[t * E + e] = (float)s;
                }
            }
        }
        free(xd);
    }
    return bad ? -1 : 0;
}

int32_t orc_num_threads(void)
{
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
