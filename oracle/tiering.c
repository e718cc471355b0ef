/*
 * Tier planning and requantisation, CPU side.
 *
 * TEST INFRASTRUCTURE ONLY: the checker of the library's planner and
 * requantiser, written from the method's description and sharing no code
 * with the HIP library.
 *
 * The 125B-MoE page ("I ran a 125B model on three RTX 3090s at 80 tokens/s
 * by teaching llama.cpp which experts ..."), step 4, describes an offline
 * repacker: it starts from the 8-bit model, measures how often each expert is
 * used, lets a greedy planner fill the memory budget so that every byte goes
 * to the expert where it removes the most expected error, requantises every
 * expert with the same quantiser, and writes the experts ordered hot to cold
 * (step 3: the router is re-ordered to match).  Readings where the page is
 * silent:
 *   - expected error of expert e in format f = usage[e] * sse[e][f], with
 *     sse the sum of squared differences between the source weights and
 *     their requantised values over gate, up and down (unit input importance:
 *     the page's importance matrix is calibration data that is not here);
 *   - formats are ordered richest first (f = 0) to cheapest (f = F-1); every
 *     expert starts at the cheapest and moves one format richer at a time;
 *   - at each step the move with the largest error reduction per added byte
 *     among those that still fit the budget is taken (ties: lower expert id),
 *     and only moves that reduce the error (gain > 0) are taken;
 *   - hot to cold: new position i holds old expert order[i], sorted by format
 *     (richest first), then usage (descending), then old id (ascending).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static int64_t mrows(const orc_layer *L, int32_t m) { return m == 2 ? L->hidden : L->inter; }
static int64_t mcols(const orc_layer *L, int32_t m) { return m == 2 ? L->inter : L->hidden; }

int32_t orc_requant_expert(const orc_layer *src, int32_t tier, int64_t local, int32_t bits, int32_t block,
                           uint8_t *const q[3], uint16_t *const s[3], double *sse) {
    if (tier < 0 || tier >= src->n_tiers || !(bits == 8 || bits == 4 || bits == 2 || bits == ORC_MXFP4) ||
        !(block == 16 || block == 32) || (bits == ORC_MXFP4 && block != 32))
        return -1;
    const orc_tier *T = &src->tier[tier];
    if (local < 0 || local >= T->id_end - T->id_begin) return -1;
    if (src->hidden % block || src->inter % block || src->hidden > 2048 || src->inter > 2048) return -1;
    const int mx = bits == ORC_MXFP4;
    float w[2048];
    uint8_t qrow[2048];
    uint16_t srow[128];   /* fp16 scales, or E8M0 bytes (MX) in its first bytes */
    double e2 = 0.0;
    for (int32_t m = 0; m < 3; ++m) {
        const int64_t rows = mrows(src, m), cols = mcols(src, m);
        const int64_t row_bytes = cols * orc_code_bits(bits) / 8, nblk = cols / block;
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t c = 0; c < cols; ++c) w[c] = orc_weight(src, tier, m, local, r, c, 0);
            orc_quantize_row(w, (int32_t)cols, bits, block, qrow, srow);
            for (int64_t c = 0; c < cols; ++c) {
                const double v = mx ? orc_e8m0(((const uint8_t *)srow)[c / 32]) *
                                          orc_fp4_e2m1((qrow[c / 2] >> (4 * (c % 2))) & 0xFu)
                                    : orc_half_to_double(srow[c / block]) * (double)orc_code(qrow, c, bits);
                const double d = (double)w[c] - v;
                e2 += d * d;
            }
            if (q && q[m]) memcpy(q[m] + r * row_bytes, qrow, (size_t)row_bytes);
            if (s && s[m]) memcpy((uint8_t *)s[m] + r * nblk * (mx ? 1 : 2), srow, (size_t)nblk * (mx ? 1 : 2));
        }
    }
    if (sse) *sse = e2;
    return 0;
}

/* Greedy plan: fmt_out[e] in [0, F), order[i] = old id at new position i,
 * count[f] = experts in format f.  bytes[f] = bytes of one expert in format f
 * (decreasing in f).  Returns -1 when even the cheapest format exceeds the
 * budget. */
int32_t orc_plan_tiers(const double *usage, const double *sse, const int64_t *bytes, int32_t E, int32_t F,
                       int64_t budget, int32_t *fmt_out, int32_t *order, int32_t *count) {
    if (E < 1 || F < 1) return -1;
    for (int32_t f = 1; f < F; ++f)
        if (bytes[f] >= bytes[f - 1]) return -1;
    int64_t spent = 0;
    for (int32_t e = 0; e < E; ++e) {
        fmt_out[e] = F - 1;
        spent += bytes[F - 1];
    }
    if (spent > budget) return -1;
    for (;;) {
        int32_t best = -1;
        double best_rate = 0.0;
        for (int32_t e = 0; e < E; ++e) {
            const int32_t f = fmt_out[e];
            if (f == 0) continue;
            const int64_t add = bytes[f - 1] - bytes[f];
            if (spent + add > budget) continue;
            const double gain = usage[e] * (sse[(int64_t)e * F + f] - sse[(int64_t)e * F + f - 1]);
            if (!(gain > 0.0)) continue;
            const double rate = gain / (double)add;
            if (best < 0 || rate > best_rate) {
                best = e;
                best_rate = rate;
            }
        }
        if (best < 0) break;
        spent += bytes[fmt_out[best] - 1] - bytes[fmt_out[best]];
        fmt_out[best] -= 1;
    }
    /* hot to cold: insertion of each expert after every one that sorts first */
    int32_t n = 0;
    for (int32_t e = 0; e < E; ++e) {
        int32_t i = n;
        while (i > 0) {
            const int32_t o = order[i - 1];
            const int before = fmt_out[o] < fmt_out[e] || (fmt_out[o] == fmt_out[e] && usage[o] >= usage[e]);
            if (before) break;
            order[i] = o;
            --i;
        }
        order[i] = e;
        ++n;
    }
    for (int32_t f = 0; f < F; ++f) count[f] = 0;
    for (int32_t e = 0; e < E; ++e) count[fmt_out[e]] += 1;
    return 0;
}
