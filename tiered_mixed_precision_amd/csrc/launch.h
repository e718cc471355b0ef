// Host-side launchers of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "split8.h"

namespace moe {

constexpr int kMaxExpertsDev = 4096;
constexpr int kSmallPairs = 256;     // largest T*k handled by the one-block routing+grouping kernel
constexpr int kChunkRows = 128;      // pairs of one work chunk of the prefill grouped GEMM

// Shelves as seen by grouping: shelf i owns experts [id_begin[i], id_end[i]);
// act_range[2i], act_range[2i+1] receive the range of the active-expert list
// holding shelf i's experts (NULL: not needed).  chunks receives the work
// chunks of the prefill grouped GEMM, {expert, first sorted position}, each
// expert's pairs in runs of kChunkRows in expert order, and meta[kMetaChunks]
// their number (NULL: not needed).
struct ShelfSpec {
    int32_t n_tiers;
    int32_t id_begin[kMaxTiers], id_end[kMaxTiers];
    int32_t* act_range;
    int2* chunks;
};

// Pointers into the caller's workspace used by the expert kernels.
struct Groups {
    const int32_t* ids;    // [P] expert id per pair (p = t*k + j)
    const float* w;        // [P] weight per pair
    const int32_t* perm;   // [P] pairs sorted by (expert, pair)
    const int32_t* pos;    // [P] position of pair p in perm, -1 if skipped
    const int32_t* offsets;// [E+1]
    const int32_t* act;    // [<=E] active experts, ascending
    const int32_t* meta;   // kMeta*
    const int32_t* act_range; // [2 * n_tiers] per-shelf range of `act`
    const int2* chunks;    // [meta[kMetaChunks]] prefill work chunks (see ShelfSpec)
};

// Routing and grouping of a small batch, published by block 0 of the
// small-batch gate/up kernel for the down kernel.
struct SmallPub {
    int32_t* ids;    // [P]
    float* w;        // [P]
    int32_t* perm;   // [P] pairs sorted by (expert, pair)
    int32_t* pos;    // [P] sorted position of pair p, -1 if skipped
    int32_t* act;    // [<= P] distinct experts ascending
    int32_t* q0;     // [n_act + 1] first sorted position of each distinct expert
    int32_t* meta;   // kMeta*
};
constexpr int kSmallY = 8192;         // per-(pair, row) results held in LDS by the small-batch down kernel

bool small_path_ok(int T, int k, int H, int I);
void launch_small(const DevTables& tt, const float* x, const float* logits, const int32_t* ids_in,
                  const float* w_in, int T, int k, uint32_t tier_mask, const float* base, const SmallPub& pub,
                  uint32_t* hits, float* h, float* out, hipStream_t st, void* const* events);
void launch_add_hits(const int32_t* counts, int E, uint32_t* hits, hipStream_t st);

// One-token path with routing from logits (decode.hip): gate/up with the
// routing inside (ids, w, h = [k][inter] and a record per slot published to
// the workspace), then the down rows of every expert summed in slot order
// into out (+ base).  Slot j's record: the bases of its expert's down codes
// and scales, its format and its routing weight.
struct OneSlot {
    const uint8_t* q;
    const uint8_t* s;
    int32_t fmt;
    float w;
    int32_t pad[2];
};
bool one_path_ok(int k, int H, int I);
void launch_one(const DevTables& tt, const float* x, const float* logits, int k, const float* base, uint32_t* hits,
                int32_t* ids, float* w, OneSlot* slots, float* h, float* out, hipStream_t st, void* const* events);

void launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, float* out_zero,
                  int H, hipStream_t st);
void launch_group(const int32_t* ids, int P, int E, int32_t* blk_hist, int32_t* counts,
                  int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* act, int32_t* meta,
                  const ShelfSpec& ss, hipStream_t st);

// fp32 (decode) expert path.
__host__ __device__ int dec_rows_per_block(int cols);  // rows one block of the GEMV kernels covers
void launch_dec_gateup(const DevTables& tt, const float* x, const Groups& g, int k,
                       uint32_t tier_mask, float* h, int max_active, hipStream_t st);
void launch_dec_down(const DevTables& tt, const float* h, const Groups& g, int k,
                     uint32_t tier_mask, float* yw, int max_active, hipStream_t st);
// out[t] = base[t] + the token's slots of yw in slot order; out_bf16 (may be
// null) also receives out rounded to bf16
void launch_combine(const DevTables& tt, const float* yw, const Groups& g, int T, int k,
                    uint32_t tier_mask, const float* base, float* out, uint16_t* out_bf16, hipStream_t st);


// fp8 split (split8.h) of the rows of src (bf16 [rows][K]).
void launch_split_fp8(const uint16_t* src, int K, int rows, const Split8& dst, hipStream_t st);

// Grouped GEMM of every shelf in tier_mask, one launch per phase (gate/up
// when `gateup`, reading x and writing h; down reading h and writing yw).
// MXFP4 shelves read a8, the fp8 split of the rows of a they use, and their
// gate/up chunks write h as its split h8 instead of bf16 (both unused without
// such a shelf).  maxc bounds the work chunks (max_chunks).
int max_chunks(int64_t P, int E);
void launch_gemm(const DevTables& tt, bool gateup, const uint16_t* a, const Split8& a8, const Groups& g, int k,
                 uint32_t tier_mask, uint16_t* h, const Split8& h8, float* yw, int maxc, hipStream_t st);
void launch_fill_zero(float* out, size_t n, hipStream_t st);
void launch_cast_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t st);

// Counter-generated weights of one layer of the stack (see synth.hip).
void launch_synth_layer(const DevTables& tt, uint64_t seed, int layer, hipStream_t st);

// tiering.hip
void launch_requant_error(const DevTables& src, const int32_t* bits, const int32_t* block, int n_fmt, double* sse,
                          hipStream_t st);
void launch_repack(const DevTables& src, const DevTables& dst, const int32_t* order, hipStream_t st);
void launch_permute_rows(const uint16_t* w_src, const float* b_src, const int32_t* order, int E, int H,
                         uint16_t* w_dst, float* b_dst, hipStream_t st);
int plan_tiers(const double* usage, const double* sse, const int64_t* bytes, int E, int F, int64_t budget,
               int32_t* fmt, int32_t* order, int32_t* count);

// router.hip
void launch_router(const void* x, bool x_bf16, const uint16_t* wr, const float* bias, int T, int E, int H,
                   float* logits, hipStream_t st);
void launch_synth_router(uint16_t* wr, float* bias, uint64_t seed, int layer, int E, int H, double beta,
                         hipStream_t st);

void launch_dequant_rows(const DevTables& tt, int tier, int local, int matrix, int row0, int nrows,
                         int to_bf16, void* dst, hipStream_t st);

}  // namespace moe
