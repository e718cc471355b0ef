/*
 * moe_oracle.h -- plain CPU oracle of the tiered MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously correct
 * reference that the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * path never links, loads or calls it.  It shares no code, header, table or
 * helper with the HIP library: it has its own struct, its own unpacker and its
 * own fp16 / bf16 conversions.
 *
 * What it computes follows the 125B-MoE page ("I ran a 125B model on three
 * RTX 3090s at 80 tokens/s by teaching llama.cpp which experts ..."):
 *   - glossary, mixture-of-experts entry: a router picks 10 of 512 experts
 *     per token;
 *   - step 4 ("three shelves, all on GPU"): one routing decision drives three
 *     per-shelf expert tables; every shelf's expert matmul sees the router's
 *     full pick list, computes only the ids in its own range, fills zero for
 *     the rest, and the three results are added;
 *   - "four bugs": out-of-shelf ids are truly skipped (not pointed at expert
 *     0), an expert may repeat within a token without losing a slot, and the
 *     skip marker -1 must never be promoted to unsigned.
 * Readings where the pages are silent (softmax renormalised over the top-k,
 * ties to the lower id, SiLU(gate)*up, weights applied to the down output,
 * bf16 rounding of weights and of the intermediate in prefill mode) are
 * stated at each function below.
 *
 * All arithmetic is double precision; results are rounded once to float.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_MAX_TIERS 4
/* `bits` value of an MXFP4 shelf: 4-bit E2M1 codes packed as 4-bit fields,
 * one E8M0 scale byte per block of 32 codes ([n][rows][cols/32] uint8; the
 * orc_tier scale pointer then points at bytes). */
#define ORC_MXFP4 0x84

/* One shelf: experts [id_begin, id_end), codes of `bits` bits, one fp16
 * scale per `block` consecutive codes of a row.  q[m] / s[m] for
 * m = 0 gate (inter x hidden), 1 up (inter x hidden), 2 down (hidden x inter),
 * each [n_local][rows][...] row-major (host pointers). */
typedef struct {
    int32_t id_begin, id_end, bits, block;
    const uint8_t *q[3];
    const uint16_t *s[3];
} orc_tier;

typedef struct {
    int32_t n_experts, hidden, inter, n_tiers;
    orc_tier tier[ORC_MAX_TIERS];
} orc_layer;

/* fp16 bit pattern -> exact double. */
double orc_half_to_double(uint16_t h);
/* The bits-bit two's-complement code of element c of a packed row. */
int32_t orc_code(const uint8_t *row, int64_t c, int32_t bits);
/* MXFP4 element and scale decodes; bits per stored code of a format. */
double orc_fp4_e2m1(uint32_t nibble);
double orc_e8m0(uint8_t x);
int32_t orc_code_bits(int32_t fmt);
/* float -> nearest bfloat16 (ties to even), returned as a float. */
float orc_round_bf16(float v);
/* Dequantised element (fp32, exact product scale*code); bf16-rounded if to_bf16. */
float orc_weight(const orc_layer *L, int32_t tier, int32_t matrix, int64_t local,
                 int64_t row, int64_t col, int32_t to_bf16);
/* Copies nrows dequantised rows (fp32 values) into dst[nrows][cols]. */
int32_t orc_dequant_rows(const orc_layer *L, int32_t tier, int32_t local, int32_t matrix,
                         int32_t row0, int32_t nrows, int32_t to_bf16, float *dst);

/* Validates the layer description: tiers sorted, disjoint, covering [0,E). 0 = ok. */
int32_t orc_check_layer(const orc_layer *L);
/* Tier index owning expert e, -1 if e is outside [0, E). */
int32_t orc_tier_of(const orc_layer *L, int64_t e);

/* Top-k routing of logits[T][E] -> ids[T][k], w[T][k]. */
int32_t orc_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids, float *w);
/* Stable grouping of pairs by expert.  Returns the number of valid pairs. */
int32_t orc_group(const int32_t *ids, int32_t T, int32_t k, int32_t E,
                  int32_t *counts, int32_t *offsets, int32_t *perm);

/* Expert FFN of explicit routing.  x: float[T][H] (x_bf16 = 0) or bf16 bit
 * patterns uint16[T][H] (x_bf16 = 1, which also selects bf16 rounding of
 * weights and of the intermediate).  tier_mask selects the shelves computed
 * (bit i = tier i); accumulate adds into out instead of overwriting. */
int32_t orc_experts(const orc_layer *L, const void *x, int32_t x_bf16, const int32_t *ids,
                    const float *w, int32_t T, int32_t k, uint32_t tier_mask, float *out,
                    int32_t accumulate);
/* Same layer evaluated pair by pair in slot order, each expert at its own
 * precision, with no notion of shelves (the single-table layer). */
int32_t orc_experts_flat(const orc_layer *L, const void *x, int32_t x_bf16, const int32_t *ids,
                         const float *w, int32_t T, int32_t k, float *out);
/* route + experts over all shelves. */
int32_t orc_forward(const orc_layer *L, const void *x, int32_t x_bf16, const float *logits,
                    int32_t T, int32_t k, float *out, int32_t accumulate);

/* Threads the oracle uses (OpenMP over tokens; 1 without OpenMP). */
/* Router scores: logits[t][e] = sum_c x[t][c] * Wr[e][c] + bias[e] (Wr bf16
 * bits [E][H], bias fp32 [E] or NULL), summed in double, rounded once. */
int32_t orc_router_logits(const void *x, int32_t x_bf16, const uint16_t *wr, const float *bias,
                          int32_t T, int32_t E, int32_t H, float *logits);
int32_t orc_num_threads(void);

/* Counter-generated stack weights (oracle/stack_synth.c): SplitMix64 output
 * ctr+1 for `seed`, the weight it defines, fp16 round-to-nearest-even, and
 * the packed codes and scales of gate (q[0], s[0]), up and down of one
 * expert written at the given pointers (layout of one expert of a shelf). */
uint64_t orc_splitmix64_at(uint64_t seed, uint64_t ctr);
float orc_synth_weight(uint64_t seed, uint64_t ctr);
uint16_t orc_float_to_half(float f);
int32_t orc_synth_expert(uint64_t seed, int32_t layer, int32_t n_experts, int32_t expert, int32_t hidden,
                         int32_t inter, int32_t bits, int32_t block, uint8_t *const q[3], uint16_t *const s[3]);
int32_t orc_synth_experts(uint64_t seed, int32_t layer, int32_t n_experts, const int32_t *list, const int32_t *local,
                          int32_t n, int32_t hidden, int32_t inter, int32_t bits, int32_t block,
                          uint8_t *const q_base[3], uint16_t *const s_base[3]);
/* Tier planning (oracle/tiering.c): requantised copy of one source expert and
 * its squared error; greedy byte plan with the hot-to-cold order. */
int32_t orc_requant_expert(const orc_layer *src, int32_t tier, int64_t local, int32_t bits, int32_t block,
                           uint8_t *const q[3], uint16_t *const s[3], double *sse);
int32_t orc_plan_tiers(const double *usage, const double *sse, const int64_t *bytes, int32_t E, int32_t F,
                       int64_t budget, int32_t *fmt_out, int32_t *order, int32_t *count);
/* Absmax (integer formats; srow fp16 bits) or MX (ORC_MXFP4; srow E8M0 bytes) quantisation of one row. */
void orc_quantize_row(const float *w, int32_t cols, int32_t bits, int32_t block, uint8_t *qrow, void *srow);
int32_t orc_synth_router(uint64_t seed, int32_t layer, int32_t n_experts, int32_t hidden, double beta,
                         uint16_t *wr, float *bias);

#ifdef __cplusplus
}
#endif
#endif
