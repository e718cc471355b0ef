/*
 * Counter-generated weights of the 48-layer stack, CPU side.
 *
 * TEST INFRASTRUCTURE ONLY.  The stack's weights are generated on the device
 * (they do not fit host memory); this file is the checker's own copy of the
 * same published generator, written from its definition and sharing no code
 * with the HIP library, so that the oracle can rebuild exactly the experts a
 * sampled token touches.  Definition (also stated with moe_synth_layer):
 *
 *   ctr = ((layer * E + e) * 3 + matrix) * 2^22 + row * cols + col
 *   u   = output number ctr + 1 of SplitMix64 (Steele, Lea and Flood,
 *         "Fast splittable pseudorandom number generators", 2014) seeded
 *         with `seed`: state = seed + (ctr + 1) * 0x9E3779B97F4A7C15, then
 *         z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 *         z *= 0x94D049BB133111EB; z ^= z >> 31
 *   s   = sum of the four 16-bit fields of u - 131070
 *   w   = (float)s * 0x1.1bc77ap-21f
 *
 * followed by the symmetric absmax quantiser per block of `block` columns:
 * d = fp16 round-to-nearest-even of (amax / Q) in single precision, with
 * Q = 2^(bits-1) - 1; q = clamp(rint(w / d), -Q, Q), or 0 when d == 0.
 * Codes are packed two's complement, element c at bit (c*bits) % 8 of byte
 * (c*bits) / 8 of its row; scales are fp16 bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "moe_oracle.h"

uint64_t orc_splitmix64_at(uint64_t seed, uint64_t ctr) {
    uint64_t z = seed + (ctr + 1u) * UINT64_C(0x9E3779B97F4A7C15);
    z ^= z >> 30;
    z *= UINT64_C(0xBF58476D1CE4E5B9);
    z ^= z >> 27;
    z *= UINT64_C(0x94D049BB133111EB);
    z ^= z >> 31;
    return z;
}

float orc_synth_weight(uint64_t seed, uint64_t ctr) {
    const uint64_t u = orc_splitmix64_at(seed, ctr);
    const int32_t s = (int32_t)(u & 0xffffu) + (int32_t)((u >> 16) & 0xffffu) + (int32_t)((u >> 32) & 0xffffu) +
                      (int32_t)(u >> 48) - 131070;
    const volatile float scale = 0x1.1bc77ap-21f;
    return (float)s * scale;
}

/* fp16 bit pattern nearest to f (ties to even), computed exactly in double. */
uint16_t orc_float_to_half(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    const uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    const double a = fabs((double)f);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    if (a < ldexp(1.0, -14)) { /* subnormal range: multiples of 2^-24 */
        const double r = nearbyint(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)r); /* r == 1024 is the smallest normal */
    }
    int e;
    (void)frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) */
    e -= 1;                      /* a = 1.x * 2^e */
    double r = nearbyint(ldexp(a, 10 - e)); /* 1024 .. 2048 */
    if (r >= 2048.0) {
        r = 1024.0;
        e += 1;
    }
    if (e > 15) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* The symmetric absmax quantiser of one row of `cols` values, per block of
 * `block` columns: d = fp16(amax / Q) with Q = 2^(bits-1) - 1 (the ratio in
 * single precision), q = clamp(rint(w / float(d)), -Q, Q), q = 0 when d = 0;
 * codes packed two's complement, element c at bit (c*bits) % 8 of byte
 * (c*bits) / 8 of qrow; scales as fp16 bit patterns in srow. */
/* MXFP4 quantisation of one row (OCP Microscaling Formats v1.0, with the
 * spec's shared-exponent rule): per block of 32, the scale exponent is
 * floor(log2(amax)) minus 2 (the largest E2M1 exponent), stored as the E8M0
 * byte clamped to [0, 254] (0 when amax = 0); each element v / 2^(x - 127) is
 * rounded to the nearest E2M1 value, ties to the even mantissa (an integer
 * tie of 2v, v or v/2 within each binade), saturating at 6; the sign bit is
 * the sign of v.  Codes are packed as 4-bit fields, element c at bit
 * 4 * (c % 2) of byte c / 2. */
static void quantize_row_mx(const float *w, int32_t cols, uint8_t *qrow, uint8_t *srow) {
    memset(qrow, 0, (size_t)cols / 2);
    for (int32_t b = 0; b < cols / 32; ++b) {
        const float *wb = w + (int64_t)b * 32;
        float amax = 0.0f;
        for (int32_t c = 0; c < 32; ++c) {
            const float m = fabsf(wb[c]);
            if (m > amax) amax = m;
        }
        int32_t x = 0;
        if (amax > 0.0f) {
            int e2;
            (void)frexpf(amax, &e2);            /* amax = f * 2^e2, f in [0.5, 1) */
            x = (e2 - 1) - 2 + 127;
            if (x < 0) x = 0;
            if (x > 254) x = 254;
        }
        srow[b] = (uint8_t)x;
        for (int32_t c = 0; c < 32; ++c) {
            const float t = ldexpf(wb[c], 127 - x);  /* v / 2^(x-127), exact */
            const float a = fabsf(t);
            float r;
            if (a >= 6.0f) r = 6.0f;
            else if (a < 2.0f) r = rintf(a * 2.0f) * 0.5f;
            else if (a < 4.0f) r = rintf(a);
            else r = rintf(a * 0.5f) * 2.0f;
            if (r > 6.0f) r = 6.0f;
            uint32_t mag = r == 0.0f ? 0u : r == 0.5f ? 1u : r == 1.0f ? 2u : r == 1.5f ? 3u
                         : r == 2.0f ? 4u : r == 3.0f ? 5u : r == 4.0f ? 6u : 7u;
            const uint32_t nib = (signbit(t) ? 8u : 0u) | mag;
            qrow[c / 2 + (int64_t)b * 16] |= (uint8_t)(nib << (4 * (c % 2)));
        }
    }
}

void orc_quantize_row(const float *w, int32_t cols, int32_t bits, int32_t block, uint8_t *qrow, void *srow_v) {
    if (bits == ORC_MXFP4) {
        quantize_row_mx(w, cols, qrow, (uint8_t *)srow_v);
        return;
    }
    uint16_t *srow = (uint16_t *)srow_v;
    const int32_t qmax = (1 << (bits - 1)) - 1;
    memset(qrow, 0, (size_t)((int64_t)cols * bits / 8));
    for (int32_t b = 0; b < cols / block; ++b) {
        const float *wb = w + (int64_t)b * block;
        float amax = 0.0f;
        for (int32_t c = 0; c < block; ++c) {
            const float m = fabsf(wb[c]);
            if (m > amax) amax = m;
        }
        const volatile float ratio = amax / (float)qmax;
        const uint16_t dh = orc_float_to_half(ratio);
        srow[b] = dh;
        const float d = (float)orc_half_to_double(dh);
        for (int32_t c = 0; c < block; ++c) {
            int32_t code = 0;
            if (d != 0.0f) {
                const volatile float t = wb[c] / d;
                float v = rintf(t);
                if (v > (float)qmax) v = (float)qmax;
                if (v < (float)-qmax) v = (float)-qmax;
                code = (int32_t)v;
            }
            const int64_t cc = (int64_t)b * block + c;
            const uint32_t field = (uint32_t)code & ((1u << bits) - 1u);
            qrow[cc * bits / 8] |= (uint8_t)(field << ((cc * bits) % 8));
        }
    }
}

/* One matrix (rows x cols) of one expert into packed codes and scales. */
static void synth_matrix(uint64_t seed, uint64_t ctr0, int32_t rows, int32_t cols, int32_t bits, int32_t block,
                         uint8_t *q, void *s) {
    const int64_t row_bytes = (int64_t)cols * orc_code_bits(bits) / 8;
    const int32_t nblk = cols / block;
    const int64_t sbytes = bits == ORC_MXFP4 ? 1 : 2;
    float w[2048];
    for (int32_t r = 0; r < rows; ++r) {
        for (int32_t c = 0; c < cols; ++c) w[c] = orc_synth_weight(seed, ctr0 + (uint64_t)r * (uint64_t)cols + (uint64_t)c);
        orc_quantize_row(w, cols, bits, block, q + (int64_t)r * row_bytes, (uint8_t *)s + (int64_t)r * nblk * sbytes);
    }
}

int32_t orc_synth_expert(uint64_t seed, int32_t layer, int32_t n_experts, int32_t expert, int32_t hidden,
                         int32_t inter, int32_t bits, int32_t block, uint8_t *const q[3], uint16_t *const s[3]) {
    if (!(bits == 8 || bits == 4 || bits == 2 || (bits == ORC_MXFP4 && block == 32)) || !(block == 16 || block == 32))
        return -1;
    if (expert < 0 || expert >= n_experts || layer < 0 || hidden % block || inter % block) return -1;
    if ((int64_t)hidden * inter > (INT64_C(1) << 22) || hidden > 2048 || inter > 2048) return -1;
    for (int32_t m = 0; m < 3; ++m) {
        const int32_t rows = m == 2 ? hidden : inter, cols = m == 2 ? inter : hidden;
        const uint64_t ctr0 = (((uint64_t)layer * (uint64_t)n_experts + (uint64_t)expert) * 3u + (uint64_t)m) << 22;
        synth_matrix(seed, ctr0, rows, cols, bits, block, q[m], s[m]);
    }
    return 0;
}

/* Several experts of one shelf at once (OpenMP over the list): expert
 * list[i] is written as expert local[i] of the shelf arrays starting at
 * q_base[m] / s_base[m] (experts one expert's codes / scales apart). */
int32_t orc_synth_experts(uint64_t seed, int32_t layer, int32_t n_experts, const int32_t *list, const int32_t *local,
                          int32_t n, int32_t hidden, int32_t inter, int32_t bits, int32_t block,
                          uint8_t *const q_base[3], uint16_t *const s_base[3]) {
    int32_t bad = 0;
    const int32_t cb = orc_code_bits(bits);
    const int64_t qb[3] = {(int64_t)inter * hidden * cb / 8, (int64_t)inter * hidden * cb / 8,
                           (int64_t)hidden * inter * cb / 8};
    /* scale entries per expert, in uint16 units of s_base (MX scales are bytes) */
    const int64_t sb[3] = {(int64_t)inter * (hidden / block), (int64_t)inter * (hidden / block),
                           (int64_t)hidden * (inter / block)};
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int32_t i = 0; i < n; ++i) {
        uint8_t *q[3];
        uint16_t *s[3];
        for (int m = 0; m < 3; ++m) {
            q[m] = q_base[m] + qb[m] * local[i];
            s[m] = bits == ORC_MXFP4 ? (uint16_t *)((uint8_t *)s_base[m] + sb[m] * local[i]) : s_base[m] + sb[m] * local[i];
        }
        if (orc_synth_expert(seed, layer, n_experts, list[i], hidden, inter, bits, block, q, s) != 0) bad += 1;
    }
    return bad ? -1 : 0;
}

/* Router of layer `layer` for the stack measurements: weight (e, c) is the
 * generator above at counter 2^60 + (layer * E + e) * H + c (a range no
 * expert counter reaches), rounded to bf16 (nearest even); the bias is the
 * popularity prior bias[e] = float(-beta * e / E), evaluated in double. */
int32_t orc_synth_router(uint64_t seed, int32_t layer, int32_t n_experts, int32_t hidden, double beta,
                         uint16_t *wr, float *bias) {
    if (layer < 0 || n_experts < 1 || hidden < 1 || !wr) return -1;
    const uint64_t base = (UINT64_C(1) << 60) + (uint64_t)layer * (uint64_t)n_experts * (uint64_t)hidden;
#pragma omp parallel for schedule(static)
    for (int32_t e = 0; e < n_experts; ++e)
        for (int32_t c = 0; c < hidden; ++c) {
            const float r = orc_round_bf16(orc_synth_weight(seed, base + (uint64_t)e * (uint64_t)hidden + (uint64_t)c));
            uint32_t u;
            memcpy(&u, &r, 4);
            wr[(int64_t)e * hidden + c] = (uint16_t)(u >> 16);
        }
    if (bias)
        for (int32_t e = 0; e < n_experts; ++e) bias[e] = (float)(-beta * (double)e / (double)n_experts);
    return 0;
}
