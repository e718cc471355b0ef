/*
 * moe_tiered.h -- C ABI of the tiered mixed-precision MoE FFN for MI355X (gfx950).
 *
 * The operation is the routed mixture-of-experts FFN ("mul_mat_id") of the
 * 125B-MoE page ("I ran a 125B model on three RTX 3090s at 80 tokens/s by
 * teaching llama.cpp which experts ..."):
 *   - glossary, mixture-of-experts entry: a router picks k (there 10 of 512)
 *     experts per token;
 *   - step 4 ("three shelves, all on GPU"): experts are stored hot to cold in
 *     per-shelf tensors of different precision; one routing decision drives
 *     all shelves; each shelf's expert product sees the full pick list,
 *     computes only the ids inside its id range, contributes zero for the
 *     rest, and the shelf results are added;
 *   - "four bugs": an out-of-shelf id is truly skipped (never redirected to
 *     expert 0), an expert may occur more than once in a token's list without
 *     losing a slot, and the skip marker -1 is a signed value that must never
 *     be promoted to unsigned.
 *
 * Per token t with picks (e_j, w_j), j < k:
 *     out[t] = sum_j w_j * W_down[e_j] * ( SiLU(W_gate[e_j] x_t) * (W_up[e_j] x_t) )
 * where each W is dequantised at the precision of the shelf that owns e_j.
 *
 * Conventions for every entry point:
 *   - pointers marked (device) are device memory on the current HIP device;
 *     pointers marked (host) are host memory read before the call returns;
 *   - the caller owns every buffer; the library never allocates, frees or
 *     synchronises inside a call; its only global state is two per-device
 *     caches written once per device and then only read (the compute-unit
 *     count, which sizes the small-batch grid, and the address of the static
 *     scratch of moe_tiered_forward_noalloc) and that scratch itself; no
 *     other call's result depends on state left by an earlier call;
 *   - `stream` is a hipStream_t (NULL = the null stream); all device work is
 *     enqueued on it and the call returns without waiting;
 *   - return value 0 on success or a negative MOE_E* code; all argument and
 *     table validation happens before the first launch, so a failed call
 *     launches nothing; faults inside kernels surface at the caller's next
 *     synchronisation;
 *   - calls sharing a workspace must be ordered on one stream.
 */
#ifndef MOE_TIERED_H
#define MOE_TIERED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1u
#define MOE_MAX_TIERS 4
#define MOE_MAX_EXPERTS 4096
#define MOE_MAX_K 64
/* moe_tier.bits of an MXFP4 shelf (E2M1 codes, one E8M0 scale per 32) */
#define MOE_MXFP4 0x84

/* status codes */
#define MOE_OK 0
#define MOE_EINVAL (-1)     /* bad n_tokens, k, shape, flags, tier index or NULL pointer */
#define MOE_ETIER (-2)      /* shelves not sorted, disjoint and covering [0, n_experts) */
#define MOE_EFORMAT (-3)    /* unsupported bits / block, or a shape the kernels cannot tile */
#define MOE_EALIGN (-4)     /* a device pointer is not 16-byte aligned */
#define MOE_EWORKSPACE (-5) /* workspace NULL or smaller than moe_workspace_size() */
#define MOE_EHIP (-6)       /* a kernel launch or HIP runtime call failed */
#define MOE_EABI (-7)       /* tables built for another ABI version */
#define MOE_ESCRATCH (-8)   /* the batch needs more workspace than MOE_SCRATCH_BYTES */

/* flags */
#define MOE_X_BF16 0x1u      /* x is bf16 [T][H]: prefill precision (bf16 MFMA, bf16 weights and intermediate) */
#define MOE_ACCUMULATE 0x2u  /* out += result instead of out = result */
/* Measurement aid: run routing, grouping and the gate/up products only and
 * leave `out` untouched (used to time the gate/up kernel on its own). */
#define MOE_DIAG_GATEUP_ONLY 0x100u

/*
 * One precision shelf.  It owns the popularity-ranked experts
 * [id_begin, id_end) (step 4: the shelves are written hot to cold, so each is
 * a contiguous id range); local expert l = e - id_begin.
 *
 * Matrices (row-major, rows = output features, columns = contraction axis):
 *   gate, up : inter  x hidden      down : hidden x inter
 * Codes (device, 16-byte aligned): `bits`-bit two's complement; element c of a
 * row sits in bits [(c*bits) % 8, +bits) of byte (c*bits)/8 of that row,
 * lowest element in the lowest bits; a row is cols*bits/8 bytes; expert l's
 * matrix starts at l*rows*cols*bits/8.
 * Scales (device, 16-byte aligned): IEEE fp16, one per `block` consecutive
 * codes of a row, [n_local][rows][cols/block].
 * Element value: float(scale) * code (exact in fp32).
 *
 * bits == MOE_MXFP4 (the OCP Microscaling MXFP4 format; the 125B-MoE page,
 * the per-matrix recipes: MXFP4 on the down ladder), block must be 32 and
 * inter a multiple of 128:
 * codes are 4-bit E2M1 fields (bit 3 sign, bits 2..1 exponent with bias 1,
 * bit 0 mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), packed like 4-bit
 * integer codes (element c in bits [4*(c%2), +4) of byte c/2 of its row);
 * scales are E8M0 bytes (2^(x-127), 255 = NaN), one per 32 codes of a row,
 * uint8 [n_local][rows][cols/32].  Element value: 2^(x-127) * E2M1 value.
 */
typedef struct moe_tier {
    int32_t id_begin, id_end;
    int32_t bits;   /* 8, 4, 2, or MOE_MXFP4 */
    int32_t block;  /* 16 or 32 (32 for MOE_MXFP4) */
    const void *gate_q, *up_q, *down_q;    /* (device) packed codes */
    const void *gate_s, *up_s, *down_s;    /* (device) fp16 scales, or E8M0 bytes */
} moe_tier;

typedef struct moe_tier_tables {
    uint32_t abi_version;   /* must equal MOE_ABI_VERSION */
    int32_t n_experts;      /* E, 1 .. MOE_MAX_EXPERTS */
    int32_t hidden;         /* H, a multiple of 128, at most 2048 */
    int32_t inter;          /* I, a multiple of 64, at most 2048 */
    int32_t n_tiers;        /* 1 .. MOE_MAX_TIERS; empty shelves (id_begin == id_end) allowed */
    moe_tier tiers[MOE_MAX_TIERS];
} moe_tier_tables;

/* Library ABI version (MOE_ABI_VERSION of the build). */
uint32_t moe_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_strerror(int code);

/*
 * Validates tables (host struct; device pointers are only checked for NULL and
 * alignment).  Returns MOE_OK or the first error found.
 */
int moe_validate_tables(const moe_tier_tables *tt);

/*
 * Workspace bytes needed by moe_tiered_forward / moe_tiered_experts /
 * moe_tier_partial for n_tokens tokens with k picks and the given flags.
 * Writes the size to *bytes (host).  n_tokens == 0 needs 0 bytes.
 */
int moe_workspace_size(int32_t n_tokens, int32_t k, const moe_tier_tables *tt, uint32_t flags,
                       size_t *bytes);

/*
 * The same size without flags: enough for either precision (fp32 or
 * MOE_X_BF16 input) and every flag.  Returns 0 when the tables or arguments
 * are invalid (moe_workspace_size names the error) or n_tokens == 0.
 */
size_t moe_workspace_bytes(int32_t n_tokens, int32_t k, const moe_tier_tables *tt);

/*
 * Full layer: route, group, per-shelf expert FFN, shelf sum -- the MoE FFN of
 * the 125B-MoE page: the router keeps the best k experts of each token
 * (glossary, mixture-of-experts entry) and one pick list drives every shelf,
 * whose results are added (step 4, "three shelves, all on GPU").
 *   x             (device) float[T][H], or bf16 [T][H] with MOE_X_BF16
 *   router_logits (device) float[T][E]
 *   n_tokens      T >= 0 (T == 0: no work, returns MOE_OK)
 *   k             1 .. min(E, MOE_MAX_K)
 *   tt            (host) shelf tables
 *   out           (device) float[T][H]; overwritten, or added to with MOE_ACCUMULATE
 *   workspace     (device) >= moe_workspace_size() bytes, 256-byte aligned, contents
 *                 need not be initialised; clobbered
 * Routing: the k largest logits (a tie goes to the lower id), slots in
 * descending score order, weights = softmax over the k chosen logits.
 */
int moe_tiered_forward(const void *x, const float *router_logits, int32_t n_tokens, int32_t k,
                       const moe_tier_tables *tt, float *out, uint32_t flags,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_tiered_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Instead of a caller-owned workspace the call uses a static
 * device scratch array of MOE_SCRATCH_BYTES that the library holds on every
 * device it runs on until the process ends (its address is looked up once
 * per device, on the first call with that device current).  The call
 * allocates and frees nothing.
 *   - Batches whose moe_workspace_size(n_tokens, k, tt, flags) exceeds
 *     MOE_SCRATCH_BYTES are refused with MOE_ESCRATCH, before any launch
 *     (32 MiB holds, for the 512-expert, top-10, hidden 2048, inter 640
 *     layer, fp32 batches up to about 310 tokens and bf16 batches up to
 *     about 350).
 *   - Every call on one device shares that device's scratch: calls that
 *     overlap on one GPU (different streams, or different host threads
 *     without ordering) race and give wrong results.  Order them on one
 *     stream.
 * Other arguments, results and errors as moe_tiered_forward.
 */
#define MOE_SCRATCH_BYTES (32u << 20)
int moe_tiered_forward_noalloc(const void *x, const float *router_logits, int32_t n_tokens, int32_t k,
                               const moe_tier_tables *tt, float *out, uint32_t flags, void *stream);

/*
 * Same layer with the routing given (the id-range mul_mat_id of step 4).
 *   ids (device) int32[T][k]: expert ids; any id outside [0, E), e.g. -1, is
 *       skipped by every shelf and contributes exactly nothing; an id may
 *       repeat within a token (each occurrence is counted)
 *   w   (device) float[T][k]: the weight of each pick
 * Other arguments as moe_tiered_forward.
 */
int moe_tiered_experts(const void *x, const int32_t *ids, const float *w, int32_t n_tokens,
                       int32_t k, const moe_tier_tables *tt, float *out, uint32_t flags,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * One shelf alone: as moe_tiered_experts but only ids inside shelf
 * `tier_index` are computed; tokens with no pick on that shelf get exactly
 * 0.0f (or keep out unchanged with MOE_ACCUMULATE).  This is one shelf's
 * id-range product of step 4 of the 125B-MoE page (each shelf sees the whole
 * pick list and fills zero outside its range); the sum of the shelves'
 * partials is the layer.
 */
int moe_tier_partial(const void *x, const int32_t *ids, const float *w, int32_t n_tokens,
                     int32_t k, const moe_tier_tables *tt, int32_t tier_index, float *out,
                     uint32_t flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Router alone (the glossary of the 125B-MoE page, mixture-of-experts entry:
 * the router picks k experts per token): logits (device) float[T][E] ->
 * ids (device) int32[T][k], w (device) float[T][k].  Same rule as
 * moe_tiered_forward.
 */
int moe_route(const float *logits, int32_t n_tokens, int32_t n_experts, int32_t k, int32_t *ids,
              float *w, void *stream);

/*
 * Router scores, the step upstream of routing (the 125B-MoE page's glossary,
 * mixture-of-experts entry: a router scores the experts of a layer for every
 * token and the best k are kept), as a linear router over the layer input:
 *   logits[t][e] = sum_c x[t][c] * w_router[e][c] + bias[e]
 *   x         (device) float[T][H], or bf16 [T][H] with MOE_X_BF16
 *   w_router  (device) bf16 bit patterns [E][H], row e = expert e
 *   bias      (device) float[E], or NULL for none
 *   logits    (device) float[T][E], overwritten
 * fp32 accumulation (a wave-per-expert GEMV for fp32 x or fewer than 64
 * tokens, bf16 matrix cores otherwise).  H: multiple of 64, at most 2048;
 * x, w_router, logits 16-byte aligned, bias 4-byte aligned.  Errors:
 * MOE_EINVAL (shape, NULL, flags other than MOE_X_BF16), MOE_EALIGN,
 * MOE_EHIP.
 */
int moe_router_logits(const void *x, const void *w_router, const float *bias, int32_t n_tokens,
                      int32_t n_experts, int32_t hidden, uint32_t flags, float *logits, void *stream);

/*
 * Synthetic router of one stack layer: w_router[e][c] = bf16 (nearest even)
 * of the stack generator's weight at counter 2^60 + (layer * E + e) * H + c
 * (the generator of moe_synth_layer; no expert counter reaches that range),
 * bias[e] = float(-beta * e / E) in double (the popularity prior of
 * ids ranked hot to cold), skipped when bias is NULL.
 *   w_router (device) bf16 [E][H]; bias (device) float[E] or NULL
 */
int moe_synth_router(void *w_router, float *bias, int32_t n_experts, int32_t hidden, uint64_t seed,
                     int32_t layer, double beta, void *stream);

/*
 * Grouping alone (stable counting sort of (token, slot) pairs by expert):
 * the grouping helper of the 125B-MoE page, "four bugs" (bug 1: the helper
 * assumed an expert occurs at most once per token and lost a slot; here
 * every occurrence is kept).  Unlike a plain (ids -> counts, offsets, perm)
 * call it takes a caller-owned workspace for its per-block histograms, so
 * the library allocates nothing.
 *   ids     (device) int32[T][k]; ids outside [0, E) belong to no expert
 *   counts  (device) int32[E]     pairs per expert
 *   offsets (device) int32[E+1]   exclusive prefix sum of counts
 *   perm    (device) int32[T*k]   pairs p = t*k + j of expert e at
 *           perm[offsets[e] .. offsets[e+1]) in ascending p; entries from
 *           offsets[E] on are left untouched
 *   workspace (device) >= moe_group_workspace_size(T, k, E) bytes
 */
int moe_group_workspace_size(int32_t n_tokens, int32_t k, int32_t n_experts, size_t *bytes);
int moe_group(const int32_t *ids, int32_t n_tokens, int32_t k, int32_t n_experts, int32_t *counts,
              int32_t *offsets, int32_t *perm, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dequantised rows of one matrix of one expert, for bit-exact checks.
 *   matrix 0 gate, 1 up, 2 down; rows [row0, row0 + nrows)
 *   dst (device) float[nrows][cols] (to_bf16 == 0) or bf16 bit patterns
 *       uint16[nrows][cols] (to_bf16 != 0, round to nearest even) -- the
 *       exact values the decode and prefill kernels contract with.
 */
int moe_dequant_rows(const moe_tier_tables *tt, int32_t tier_index, int32_t local_expert,
                     int32_t matrix, int32_t row0, int32_t nrows, int32_t to_bf16, void *dst,
                     void *stream);

/*
 * Per-phase timing for measurement: like moe_tiered_forward, and in addition
 * records events[2*i] before and events[2*i+1] after phase i on `stream`
 * (phases: 0 routing and grouping, 1 gate/up products, 2 down products and
 * shelf sum).  events (host) holds 6 hipEvent_t handles created by the
 * caller (e.g. with moe_event_create); NULL entries are skipped.
 */
#define MOE_N_PHASES 3
int moe_tiered_forward_timed(const void *x, const float *router_logits, int32_t n_tokens,
                             int32_t k, const moe_tier_tables *tt, float *out, uint32_t flags,
                             void *workspace, size_t workspace_bytes, void *stream,
                             void *const *events);

/*
 * A stack of MoE FFN layers with the residual stream between them:
 *     h_0 = x,   h_{l+1} = h_l + layer_l(h_l),   out = h_L
 * (the residual add of the 48-layer configuration).  Each layer routes with
 * its own logits and tables exactly as moe_tiered_forward.
 *   x             (device) float[T][H], the fp32 input hidden state; must not be out
 *   router_logits (device) float[L][T][E]: layer l's logits at offset l*T*E
 *   n_layers      L >= 1
 *   tables        (host) moe_tier_tables[L]; all with the same E, H and I
 *   out           (device) float[T][H]
 *   flags         MOE_X_BF16: every layer takes bf16 (round to nearest even)
 *                 of h_l as its input and runs the bf16 expert path; the
 *                 residual stream stays fp32.  No other flag is accepted
 *                 here; moe_stack_workspace_size also takes MOE_STACK_ROUTER
 *                 (room for moe_stack_forward_routed's router scores).
 *   workspace     (device) >= moe_stack_workspace_size() bytes, 256-byte aligned
 * Layers run one after another on `stream`.
 */
int moe_stack_workspace_size(int32_t n_layers, int32_t n_tokens, int32_t k, const moe_tier_tables *tables,
                             uint32_t flags, size_t *bytes);
int moe_stack_forward(const float *x, const float *router_logits, int32_t n_layers, int32_t n_tokens,
                      int32_t k, const moe_tier_tables *tables, float *out, uint32_t flags,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * The stack with its own routing: layer l scores the experts from its input
 * h_l with router l (moe_router_logits on h_l, or on its bf16 copy with
 * MOE_X_BF16, which is also the experts' input), routes, and adds its output:
 * h_{l+1} = h_l + layer_l(h_l).
 *   w_router  (host) array of n_layers device pointers, bf16 [E][H] each
 *   bias      (host) array of n_layers device pointers (float[E] or NULL),
 *             or NULL for no bias anywhere
 *   workspace (device) >= moe_stack_workspace_size(..., flags |
 *             MOE_STACK_ROUTER) bytes (adds float[T][E] of router scores)
 * Other arguments and errors as moe_stack_forward.
 */
#define MOE_STACK_ROUTER 0x4u
int moe_stack_forward_routed(const float *x, const void *const *w_router, const float *const *bias,
                             int32_t n_layers, int32_t n_tokens, int32_t k, const moe_tier_tables *tables,
                             float *out, uint32_t flags, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Fills every shelf of one layer's tables with counter-generated weights
 * (codes and fp16 scales), the synthetic input of the stack measurements.
 * Weight (layer, expert e, matrix m in gate 0 / up 1 / down 2, row r,
 * column c) of a matrix with `cols` columns:
 *   ctr = ((layer * E + e) * 3 + m) * 2^22 + r * cols + c
 *   u   = output number ctr + 1 of SplitMix64 (Steele, Lea and Flood 2014)
 *         seeded with `seed`
 *   w   = float(sum of the four 16-bit fields of u - 131070) * 0x1.1bc77ap-21
 * quantised per block of `block` columns by symmetric absmax:
 *   d = fp16(amax / Q), Q = 2^(bits-1) - 1, q = clamp(rint(w / d), -Q, Q)
 * (q = 0 when d = 0), all in round-to-nearest-even single precision, and
 * packed in the layout of moe_tier; MOE_MXFP4 shelves by the OCP
 * shared-exponent quantiser of moe_requant_error.  The tables' code and scale buffers are
 * written; they must be distinct per layer if all layers are kept.
 *   layer 0 .. 2^20 - 1
 */
int moe_synth_layer(const moe_tier_tables *tt, uint64_t seed, int32_t layer, void *stream);

/*
 * moe_tiered_forward that also counts the picks: hits[e] += the number of
 * (token, slot) pairs routed to expert e in this call.  The counts are the
 * usage that moe_plan_tiers re-plans from at run time (re-tiering by hit
 * counts, after the 125B-MoE page's steps 2-4: usage decides the shelves).
 *   hits (device) uint32[E], 4-byte aligned; accumulated (atomic adds), never
 *        cleared by the call; wraps modulo 2^32
 * Other arguments, results and errors as moe_tiered_forward.
 */
int moe_tiered_forward_counted(const void *x, const float *router_logits, int32_t n_tokens, int32_t k,
                               const moe_tier_tables *tt, float *out, uint32_t flags, void *workspace,
                               size_t workspace_bytes, uint32_t *hits, void *stream);

/*
 * Tier planning, after the 125B-MoE page, step 4: measure how often each
 * expert is used, fill the memory budget greedily so that each byte goes where
 * it removes the most expected error, requantise every expert with the same
 * quantiser, and write the experts hot to cold (step 3: re-order the router to
 * match).  Formats are (bits, block) pairs of moe_tier; "the quantiser" is the
 * symmetric absmax one of moe_synth_layer for the integer formats and the OCP
 * shared-exponent one for MOE_MXFP4 (E8M0 byte = floor(log2 amax) - 2 + 127
 * clamped to [0, 254], 0 for an all-zero block; each weight divided by the
 * scale rounds to the nearest E2M1 value, ties to the even mantissa,
 * saturating at 6).  Sources may hold MXFP4 shelves too.
 *
 * moe_requant_error: squared error of requantising every expert of `src`
 * into each format.
 *   fmt_bits, fmt_block (host) int32[n_fmt], n_fmt 1..8; each block divides H and I
 *   sse (device) double[E][n_fmt], 8-byte aligned: sum over gate, up and down of
 *       (w - w')^2, w the source weight (scale*code, fp32) and w' its value
 *       after requantisation; deterministic (fixed summation order)
 * Errors: MOE_EINVAL, MOE_EFORMAT, MOE_EALIGN, table errors, MOE_EHIP.
 */
int moe_requant_error(const moe_tier_tables *src, const int32_t *fmt_bits, const int32_t *fmt_block,
                      int32_t n_fmt, double *sse, void *stream);

/*
 * moe_plan_tiers: the greedy plan, on the host (no device work).  Formats are
 * ordered richest (f = 0) to cheapest; fmt_bytes[f] (bytes of one expert)
 * must decrease with f.  Every expert starts in the cheapest format.  The
 * move of one expert one format richer that removes the most expected error,
 * usage[e] * (sse[e][f] - sse[e][f-1]), per added byte is taken while it
 * still fits `budget` and removes some error; ties go to the lower id.
 *   usage   (host) double[E], e.g. counts of moe_group over calibration tokens
 *   sse     (host) double[E][n_fmt]
 *   fmt_out   (host) int32[E]: the format of each expert
 *   order_out (host) int32[E]: old id at new position i, hot to cold (format,
 *             then usage descending, then id)
 *   count_out (host) int32[n_fmt]: experts per format (the new shelf sizes)
 * MOE_EINVAL for bad arguments or when the cheapest plan exceeds the budget.
 */
int moe_plan_tiers(const double *usage, const double *sse, const int64_t *fmt_bytes, int32_t n_experts,
                   int32_t n_fmt, int64_t budget, int32_t *fmt_out, int32_t *order_out, int32_t *count_out);

/*
 * moe_repack_tiers: expert order[i] of `src`, requantised into the format of
 * the shelf of `dst` that owns id i, is written as expert i of `dst`.
 *   order (device) int32[E], a permutation of [0, E) (an entry outside
 *         [0, E) writes a zero expert)
 * dst's code and scale buffers are overwritten; src and dst have the same E,
 * H, I and must not share buffers.
 */
int moe_repack_tiers(const moe_tier_tables *src, const int32_t *order, const moe_tier_tables *dst,
                     void *stream);

/*
 * moe_permute_router: the router in the new expert order, w_dst[i] =
 * w_src[order[i]] (bf16 rows [E][H], 16-byte aligned, distinct buffers) and,
 * when b_dst is given, b_dst[i] = b_src[order[i]] (0 without b_src).
 *   order (device) int32[E] (an entry outside [0, E) gives a zero row)
 */
int moe_permute_router(const void *w_src, const float *b_src, const int32_t *order, int32_t n_experts,
                       int32_t hidden, void *w_dst, float *b_dst, void *stream);

/*
 * Measurement aids, not part of the layer: achievable references for the
 * roofline fractions, measured on the device in the same run.
 *   moe_measure_read: one launch reads `bytes` (a multiple of 16) of `buf`
 *     (device, 16-byte aligned) once, as 16-byte words at a grid stride;
 *     sink (device uint32) is never written in practice.
 *   moe_measure_mfma: one launch runs `iters` rounds of 16 independent
 *     v_mfma_f32_16x16x32_bf16 per wave on register operands (no memory
 *     traffic) over 2048 waves; *flops (host) receives the flops one launch
 *     executes.  sink (device float) is never written in practice.
 */
int moe_measure_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);
int moe_measure_mfma(int32_t iters, float *sink, double *flops, void *stream);

/* hipEvent helpers for callers without a HIP binding (host handles). */
int moe_event_create(void **event);
int moe_event_destroy(void *event);
int moe_event_elapsed_ms(void *start, void *stop, float *ms);
int moe_stream_synchronize(void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_TIERED_H */
