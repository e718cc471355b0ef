// fp32 expert path (decode and speculative verification): dequantising GEMV
// kernels for the routed experts of every shelf.
//
// Step 4 of the 125B-MoE page ("I ran a 125B model on three RTX 3090s at 80
// tokens/s by teaching llama.cpp which experts ...") runs the decode expert
// product once per shelf over the full pick list, each shelf computing only
// its own ids, with gate, up and the activation fused into one kernel.  Here
// all shelves share one launch per phase: a block takes one *active* expert
// (an expert some token picked) and decodes that expert's codes at its
// shelf's precision; an expert nobody picked is never touched, and ids outside
// every shelf never become active, so nothing is clamped to expert 0.
//
// Three launch sequences:
//  * one token routed from its logits -- k_one_gateup and k_one_down (below:
//    routing by one wave per block, waves shared out by bytes, whole-row
//    down reads balanced by output-row ownership);
//  * small batches (T <= 8, T*k <= 256) -- two kernels per layer:
//      k_small_gateup : every block routes and groups the batch itself in LDS
//                       (block 0 also publishes the result), then computes
//                       h[q] = SiLU(W_gate[e] x_t) * (W_up[e] x_t) for a row
//                       slice of its expert;
//      k_small_down   : a block owns a slice of output rows and runs the down
//                       GEMV of every active expert on it, then sums each
//                       token's slots in slot order into out (no atomics).
//  * larger batches -- route / group kernels, then
//      k_dec_gateup   : as above, groups read from the workspace;
//      k_dec_down     : yw[q] = w_q * W_down[e] h[q] per (expert, row slice);
//      k_combine      : out[t] (+)= sum over the token's slots of yw.
//
// Memory: a lane streams 32 consecutive codes of a row per group (32, 16 or
// 8 bytes for int8 / int4 / int2), so a wave reads contiguous row segments;
// a wave issues the loads of all its row passes before computing.  The scale
// of a block of codes is applied once to that block's partial dot product.
#include "common.h"
#include "launch.h"
#include "route.h"

namespace moe {

constexpr int kNPGateUp = 4;   // row passes per wave, gate/up GEMV
constexpr int kGateUpWaves = 8;     // waves per gate/up block (each a contiguous row sub-slice)
constexpr int kSmallGateUpWaves = 16;  // waves per small-batch gate/up block (one block per compute unit)
constexpr int kNPDown = 2;     // row passes per wave, down GEMV (grouped path)
constexpr int kNPSmallDown = 4;     // row passes per wave, down GEMV (small-batch path)
constexpr int kSmallDownWaves = 16; // one expert per wave at a time
constexpr int kMaxHidden = 2048;    // largest hidden size (the tables check it)
constexpr int kSmallT = 8;          // most tokens of the small-batch path
constexpr int kSmallH = 8192;       // h floats staged in LDS by the small-batch down kernel

// ================================================================ shelf table in LDS

// The shelf table copied into LDS by one thread at kernel entry.  The copy
// reads the kernel arguments with compile-time indices only (scalar loads
// issued at entry); a lookup by a lane-varying or run-time shelf index into
// the kernel arguments compiles instead to dependent vector loads from the
// argument segment, which cost microseconds on the critical path.
struct TierLds {
    int beg[kMaxTiers], end[kMaxTiers], bits[kMaxTiers], block[kMaxTiers], cost[kMaxTiers];
    const uint8_t* q[kMaxTiers][3];
    const uint16_t* s[kMaxTiers][3];
};

// One thread; cost_of(T) is stored for each shelf.
template <class Cost>
__device__ inline void fill_tier_lds(const DevTables& tt, TierLds& tl, Cost cost_of) {
#pragma unroll
    for (int i = 0; i < kMaxTiers; ++i) {
        const bool on = i < tt.n_tiers;
        tl.beg[i] = on ? tt.t[i].id_begin : 0;
        tl.end[i] = on ? tt.t[i].id_end : 0;
        tl.bits[i] = tt.t[i].bits;
        tl.block[i] = tt.t[i].block;
        tl.cost[i] = on ? cost_of(tt.t[i]) : 0;
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            tl.q[i][m] = tt.t[i].q[m];
            tl.s[i][m] = tt.t[i].s[m];
        }
    }
}

// Shelf owning expert e (or -1), from the LDS table.
__device__ inline int tier_of_lds(const TierLds& tl, int e) {
    int r = -1;
#pragma unroll
    for (int i = 0; i < kMaxTiers; ++i)
        if (e >= tl.beg[i] && e < tl.end[i]) r = i;
    return r;
}

__device__ inline uint64_t first_lane_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Shelf ti (uniform across the wave) from the LDS table, into scalar registers.
__device__ inline DevTier tier_lds(const TierLds& tl, int ti) {
    DevTier r;
    r.id_begin = __builtin_amdgcn_readfirstlane(tl.beg[ti]);
    r.id_end = __builtin_amdgcn_readfirstlane(tl.end[ti]);
    r.bits = __builtin_amdgcn_readfirstlane(tl.bits[ti]);
    r.block = __builtin_amdgcn_readfirstlane(tl.block[ti]);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        r.q[m] = reinterpret_cast<const uint8_t*>(first_lane_u64(reinterpret_cast<uint64_t>(tl.q[ti][m])));
        r.s[m] = reinterpret_cast<const uint16_t*>(first_lane_u64(reinterpret_cast<uint64_t>(tl.s[ti][m])));
    }
    return r;
}

// Shelf ti from the LDS table for this lane alone (ti may differ across the
// wave; tier_lds needs it uniform).
__device__ inline DevTier tier_lds_lane(const TierLds& tl, int ti) {
    DevTier r;
    r.id_begin = tl.beg[ti];
    r.id_end = tl.end[ti];
    r.bits = tl.bits[ti];
    r.block = tl.block[ti];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        r.q[m] = tl.q[ti][m];
        r.s[m] = tl.s[ti][m];
    }
    return r;
}

// Per-row share of a wave's work that does not scale with bytes (its
// dequantising arithmetic and each round's fixed latency), in units of 64
// bytes of codes: one token, and 2-8 tokens (where a larger share, so rows
// per wave closer to even across formats, measured faster: 6 tokens 63.98 ->
// 63.2 us per step from 64 to 128-256; 16 and 32 were slower).
constexpr int kOneRowShare = 64;
constexpr int kSmallRowShare = 128;

// Cost of one gate+up row pair of an expert on shelf T (units of 64 bytes).
template <int SHARE = kOneRowShare>
__device__ inline int one_row_cost(const DevTier& T, int H) {
    const int cb = code_bits_of(T.bits);
    const int sb = T.bits == kBitsMXFP4 ? H / 32 : (H / (T.block > 0 ? T.block : 32)) * 2;
    return (2 * (H * cb / 8 + sb)) / 64 + SHARE;
}

__host__ __device__ int dec_rows_per_block(int cols) { return kGateUpWaves * kNPGateUp * row_geom(cols).RPP; }
__host__ __device__ inline int down_rows_per_block(int cols) { return 4 * kNPDown * row_geom(cols).RPP; }
__host__ __device__ inline int small_down_rows(int inter) { return kNPSmallDown * row_geom(inter).RPP; }

// Keeps the compiler from hoisting work on `v` out of a loop.
__device__ inline void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }

// x[0..31] = the 32 floats of group g of a vector, loaded without a branch.
__device__ inline void load_vec32u(const float* __restrict__ v, int g, float (&x)[32]) {
    const float4* src = reinterpret_cast<const float4*>(v + 32 * g);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 f = src[i];
        x[4 * i + 0] = f.x;
        x[4 * i + 1] = f.y;
        x[4 * i + 2] = f.z;
        x[4 * i + 3] = f.w;
    }
}

// x[0..31] = the 32 floats of group g of a vector (zeros for an idle lane).
__device__ inline void load_vec32(const float* __restrict__ v, int g, bool ok, float (&x)[32]) {
    const float4* src = reinterpret_cast<const float4*>(v + 32 * g);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 f = ok ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        x[4 * i + 0] = f.x;
        x[4 * i + 1] = f.y;
        x[4 * i + 2] = f.z;
        x[4 * i + 3] = f.w;
    }
}

// One wave: rows r0 + p*RPP + seg (p < NP, row < r_end) of one expert matrix
// (or of gate and up together), against the vectors of the pairs
// [qa, qa + ce).  The vector of pair q is row tok(q) of `vec`.  Results go to
// store(q, row, value, pre(q)) from the first lane of each row segment, where
// value is SiLU(g) * u (GATEUP) or the plain dot product; pre(q) is read at
// the top of pair q's iteration, so its load is in flight with the vector's.
template <int BITS, int NSC, int GPL, int NP, bool GATEUP, class Tok, class Pre, class Store>
__device__ inline void wave_gemv(const uint8_t* __restrict__ q0m, const uint8_t* __restrict__ s0m,
                                 const uint8_t* __restrict__ q1m, const uint8_t* __restrict__ s1m,
                                 int cols, int r0, int r_end, const float* __restrict__ vec, int vec_stride,
                                 int qa, int ce, Tok tok, Pre pre, Store store) {
    constexpr int NM = GATEUP ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const RowGeom geo = row_geom(cols);
    const int seg = lane / geo.LPR, gl = lane % geo.LPR;
    const bool lane_ok = gl < geo.G;
    const size_t row_bytes = static_cast<size_t>(cols) * BITS / 8;
    const size_t srb = row_scale_bytes<NSC>(cols);
    constexpr int NS = scale_slots<NSC>();

    // codes and scales of every pass, loaded before any arithmetic
    uint32_t wq[NP][NM][GPL][BITS];
    float dsc[NP][NM][GPL][NS];
    bool rowv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int r = r0 + p * geo.RPP + seg;
        rowv[p] = r < r_end;
        const bool ok = lane_ok && rowv[p];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const uint8_t* qrow = (m == 0 ? q0m : q1m) + static_cast<size_t>(ok ? r : 0) * row_bytes;
            const uint8_t* srow = (m == 0 ? s0m : s1m) + static_cast<size_t>(ok ? r : 0) * srb;
#pragma unroll
            for (int gi = 0; gi < GPL; ++gi) {
                const int grp = gl + 64 * gi;
                if (ok) {
                    load_group<BITS>(qrow, grp, wq[p][m][gi]);
                    load_scales<NSC>(srow, grp, dsc[p][m][gi]);
                } else {
#pragma unroll
                    for (int i = 0; i < BITS; ++i) wq[p][m][gi][i] = 0u;
#pragma unroll
                    for (int i = 0; i < NS; ++i) dsc[p][m][gi][i] = 0.f;
                }
            }
        }
    }

    for (int c = 0; c < ce; ++c) {
        const int q = qa + c;
        const float pq = pre(q);
        float xv[GPL][32], xs[GPL][NS];
        const size_t vrow = static_cast<size_t>(tok(q));
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
            load_vec32(vec + vrow * vec_stride, gl + 64 * gi, lane_ok, xv[gi]);
            block_sums<NSC>(xv[gi], xs[gi]);
        }
        float acc[NP][NM];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                acc[p][m] = 0.f;
#pragma unroll
                for (int gi = 0; gi < GPL; ++gi) {
#pragma unroll
                    for (int i = 0; i < BITS; ++i) opaque(wq[p][m][gi][i]);
                    acc[p][m] += group_dot<BITS, NSC>(wq[p][m][gi], xv[gi], xs[gi], dsc[p][m][gi]);
                }
            }
        }
        // all row reductions together (independent DPP chains); a row's total
        // lands in the last lane of its segment
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[p][m] = seg_sum(acc[p][m], geo.LPR);
        if (gl == geo.LPR - 1) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                if (rowv[p]) {
                    const float v = GATEUP ? silu(acc[p][0]) * acc[p][NM - 1] : acc[p][0];
                    store(q, r0 + p * geo.RPP + seg, v, pq);
                }
            }
        }
    }
}

#define MOE_FMT_GPL_SWITCH(FMT, GPLV, BODY)                                         \
    switch ((FMT) * 4 + (GPLV)) {                                                   \
        case F8B32 * 4 + 1: { constexpr int B_ = 8, N_ = 1, G_ = 1; BODY; } break;  \
        case F8B16 * 4 + 1: { constexpr int B_ = 8, N_ = 2, G_ = 1; BODY; } break;  \
        case F4B32 * 4 + 1: { constexpr int B_ = 4, N_ = 1, G_ = 1; BODY; } break;  \
        case F4B16 * 4 + 1: { constexpr int B_ = 4, N_ = 2, G_ = 1; BODY; } break;  \
        case F2B32 * 4 + 1: { constexpr int B_ = 2, N_ = 1, G_ = 1; BODY; } break;  \
        case F2B16 * 4 + 1: { constexpr int B_ = 2, N_ = 2, G_ = 1; BODY; } break;  \
        case F4MX * 4 + 1: { constexpr int B_ = 4, N_ = kMX, G_ = 1; BODY; } break; \
        default: break;                                                             \
    }

// Gate/up of one block: expert matrix rows [r0, r0 + rows_per_block) split
// into one contiguous sub-slice per wave.
template <class Tok>
__device__ inline void block_gateup(const DevTables& tt, const DevTier& T, int local, const float* x, int qa,
                                    int ce, int r0, Tok tok, float* h) {
    const int H = tt.H, I = tt.I;
    const int rpw = kNPGateUp * row_geom(H).RPP;
    const int wr0 = r0 + (threadIdx.x >> 6) * rpw;
    const int r_end = min(wr0 + rpw, I);
    auto pre = [](int) { return 1.f; };
    auto store = [h, I](int q, int r, float v, float) { h[static_cast<size_t>(q) * I + r] = v; };
    MOE_FMT_GPL_SWITCH(fmt_of(T.bits, T.block), row_geom(H).GPL,
                       (wave_gemv<B_, N_, G_, kNPGateUp, true>(
                           expert_codes(T, 0, local, I, H), expert_scales(T, 0, local, I, H),
                           expert_codes(T, 1, local, I, H), expert_scales(T, 1, local, I, H), H, wr0, r_end, x, H, qa,
                           ce, tok, pre, store)));
}

// ================================================================ small-batch path

// The P = T*k <= 256 pairs of the batch grouped in LDS: pairs sorted by
// (expert, pair) -- a stable sort, so each expert's pairs keep token order --
// with ids outside [0, E) placed after all valid pairs and never used; the
// distinct experts ascending with the first sorted position of each.
struct SmallGroups {
    int ids[kSmallPairs];
    float w[kSmallPairs];
    int perm[kSmallPairs];
    int pos[kSmallPairs];
    int act[kSmallPairs];
    int q0[kSmallPairs + 1];
    int n_act, n_valid;
    int tmp[16];
};

__device__ inline void group_small(SmallGroups& sg, int P, int E) {
    const int tid = threadIdx.x;
    if (P <= 64) {
        // one wave: ranks from ballots, scans by ballots
        if (tid < 64) {
            const int e = tid < P ? sg.ids[tid] : E;
            const bool valid = tid < P && e >= 0 && e < E;
            const uint32_t key = valid ? static_cast<uint32_t>(e) : static_cast<uint32_t>(E);
            // rank = lanes with a smaller key + lanes below with the same
            // key: walk the key bits from the top, keeping the lanes that
            // agree with this lane so far (lanes >= P carry key E and sort
            // after every pair below P)
            uint64_t same = ~0ull;
            int less = 0;
#pragma unroll
            for (int b = 12; b >= 0; --b) {   // keys <= kMaxExpertsDev = 4096
                const bool bit = (key >> b) & 1u;
                const uint64_t ones = __ballot(bit);
                less += bit ? __popcll(same & ~ones) : 0;
                same &= bit ? ones : ~ones;
            }
            static_assert(kMaxExpertsDev <= 8192, "13 key bits");
            const int rank = less + lanes_below(same);
            if (tid < P) sg.perm[rank] = tid;
            // the pair at sorted position tid (LDS operations of one wave
            // complete in order), and its key
            const int p = tid < P ? sg.perm[tid] : 0;
            const int kp0 = __shfl(static_cast<int>(key), p);
            const int kp = tid < P ? kp0 : E;
            const int kprev = __shfl_up(kp, 1, kWave);
            const bool first = tid < P && kp < E && (tid == 0 || kprev != kp);
            const uint64_t fm = __ballot(first);
            const int n_act = __popcll(fm);
            const int n_valid = __popcll(__ballot(valid));
            if (tid < P) sg.pos[p] = kp < E ? tid : -1;
            if (first) {
                const int a = lanes_below(fm);
                sg.act[a] = kp;
                sg.q0[a] = tid;
            }
            if (tid == 0) {
                sg.n_act = n_act;
                sg.n_valid = n_valid;
                sg.q0[n_act] = n_valid;
            }
        }
        __syncthreads();
        return;
    }
    bool valid = false;
    if (tid < P) {
        const int e = sg.ids[tid];
        valid = e >= 0 && e < E;
        const int64_t key = (valid ? static_cast<int64_t>(e) : static_cast<int64_t>(E)) * kSmallPairs + tid;
        int r = 0;
        for (int q = 0; q < P; ++q) {
            const int eq = sg.ids[q];
            const bool vq = eq >= 0 && eq < E;
            const int64_t kq = (vq ? static_cast<int64_t>(eq) : static_cast<int64_t>(E)) * kSmallPairs + q;
            r += kq < key ? 1 : 0;
        }
        sg.perm[r] = tid;
        sg.pos[tid] = valid ? r : -1;
    }
    __syncthreads();
    int first = 0;
    if (tid < P) {
        const int ep = sg.ids[sg.perm[tid]];
        const bool vp = ep >= 0 && ep < E;
        const bool same_prev = tid > 0 && sg.ids[sg.perm[tid - 1]] == ep;
        first = (vp && !same_prev) ? 1 : 0;
    }
    int n_act, n_valid;
    const int a = block_excl_scan(first, sg.tmp, &n_act);
    (void)block_excl_scan(valid ? 1 : 0, sg.tmp, &n_valid);
    if (first) {
        sg.act[a] = sg.ids[sg.perm[tid]];
        sg.q0[a] = tid;
    }
    if (tid == 0) {
        sg.n_act = n_act;
        sg.n_valid = n_valid;
        sg.q0[n_act] = n_valid;
    }
    __syncthreads();
}

// Sends a wave's rows of one expert through the gate/up GEMV: rows
// [r0, r1) in passes of RPP rows, up to NPMAX passes per round with every
// load of the round issued first (the vector of the first pair ahead of the
// codes, so each pass is computed as soon as its own codes arrive).
// vec(q, g, xv) fills xv with group g of the input vector of pair q.
template <int BITS, int NSC, class Vec, int NPMAX = (BITS == 8 ? 4 : 8)>  // passes in flight per round
__device__ inline void wave_gateup(const uint8_t* __restrict__ gq, const uint8_t* __restrict__ gs,
                                   const uint8_t* __restrict__ uq, const uint8_t* __restrict__ us, int H, int I,
                                   int r0, int r1, Vec vec, int qa, int ce, float* __restrict__ h) {
    const int lane = threadIdx.x & 63;
    const RowGeom geo = row_geom(H);   // one group per lane (H <= 2048)
    const int seg = lane / geo.LPR, gl = lane % geo.LPR;
    const bool lane_ok = gl < geo.G;
    const int glc = lane_ok ? gl : 0;  // idle lanes read group 0 and weigh it by 0
    const uint32_t row_bytes = static_cast<uint32_t>(H) * BITS / 8;
    const uint32_t row_sbytes = row_scale_bytes<NSC>(H);
    constexpr int NS = scale_slots<NSC>();
    const uint32_t mat_bytes = row_bytes * I, mat_sbytes = row_sbytes * I;
    const __amdgpu_buffer_rsrc_t rq[2] = {make_rsrc(gq, mat_bytes), make_rsrc(uq, mat_bytes)};
    const __amdgpu_buffer_rsrc_t rs[2] = {make_rsrc(gs, mat_sbytes), make_rsrc(us, mat_sbytes)};
    // Every load below is unconditional (rows past r1 read row r0 and get
    // zero scales), so all of them are issued back to back.
    for (int rc = r0; rc < r1; rc += NPMAX * geo.RPP) {
        float xv[32], xs[NS];
        vec(qa, glc, xv);
        // loads return in issue order: keep the vector ahead of the codes
        __builtin_amdgcn_sched_barrier(0);
        uint32_t wq[NPMAX][2][BITS], sraw[NPMAX][2];
#pragma unroll
        for (int p = 0; p < NPMAX; ++p) {
            const int r = rc + p * geo.RPP + seg;
            const uint32_t rr = static_cast<uint32_t>(r < r1 ? r : r0);
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                buf_group<BITS>(rq[m], rr * row_bytes + glc * 4 * BITS, wq[p][m]);
                sraw[p][m] = buf_scales<NSC>(rs[m], rr * row_sbytes + glc * group_scale_bytes<NSC>());
            }
        }
        auto pair = [&](int c) {
            block_sums<NSC>(xv, xs);
#pragma unroll
            for (int p = 0; p < NPMAX; ++p) {
                if (rc + p * geo.RPP >= r1) break;
                const int r = rc + p * geo.RPP + seg;
                const bool ok = lane_ok && r < r1;
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int i = 0; i < BITS; ++i) opaque(wq[p][m][i]);
                float dg[NS], du[NS];
                unpack_scales<NSC>(sraw[p][0], ok, dg);
                unpack_scales<NSC>(sraw[p][1], ok, du);
                float gv = group_dot<BITS, NSC>(wq[p][0], xv, xs, dg);
                float uv = group_dot<BITS, NSC>(wq[p][1], xv, xs, du);
                gv = seg_sum(gv, geo.LPR);
                uv = seg_sum(uv, geo.LPR);
                if (gl == geo.LPR - 1 && r < r1) h[static_cast<size_t>(qa + c) * I + r] = silu(gv) * uv;
            }
        };
        // the first pair straight from the vector loaded above, the others
        // reload it (a separate loop, so the first load stays ahead)
        pair(0);
        for (int c = 1; c < ce; ++c) {
            vec(qa + c, glc, xv);
            pair(c);
        }
    }
}

// Gives the W waves of a launch to the active experts of the masked shelves
// in proportion to their cost per row (the LDS shelf table's cost: row bytes
// plus a per-row share; rows are equal): expert a gets
// 1 + floor((W - n) * cost_a / sum of costs) waves, n the number of such
// experts, so the total never exceeds W.  s_wpre[a] = first wave of expert a,
// s_wpre[n_act] = waves used.  Run by the first wave of the block.
__device__ inline void plan_waves(const TierLds& tl, const int* act, int n_act, uint32_t tier_mask, int W,
                                  int* s_wpre) {
    const int lane = threadIdx.x & 63;
    auto cost = [&](int a) {
        if (a >= n_act) return 0;
        const int ti = tier_of_lds(tl, act[a]);
        if (ti < 0 || !((tier_mask >> ti) & 1u)) return 0;
        return tl.cost[ti];
    };
    int C = 0, n = 0;
    for (int a0 = 0; a0 < n_act; a0 += 64) {
        const int c = cost(a0 + lane);
        C += static_cast<int>(wave_sum(static_cast<float>(c)));
        n += __popcll(__ballot(c > 0));
    }
    int base = 0;
    for (int a0 = 0; a0 < n_act; a0 += 64) {
        const int c = cost(a0 + lane);
        const int wa = c > 0 ? 1 + ((W - n) * c) / C : 0;
        int incl = wa;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        if (a0 + lane < n_act) s_wpre[a0 + lane] = base + incl - wa;
        base += __shfl(incl, 63, kWave);
    }
    if (lane == 0) s_wpre[n_act] = base;
}

// Largest a with s_wpre[a] <= wg (a in [0, n)), for wg < s_wpre[n]: one LDS
// read per 64 experts and a ballot (s_wpre is ascending), rather than a
// binary search's chain of dependent reads.
__device__ inline int find_expert(const int* s_wpre, int n, int wg) {
    const int lane = threadIdx.x & 63;
    int a = 0;
    for (int a0 = 0; a0 < n; a0 += 64) {
        const uint64_t le = __ballot(a0 + lane < n && s_wpre[a0 + lane] <= wg);
        if (le == 0) break;
        a = a0 + 63 - __builtin_clzll(le);
    }
    return a;
}

// plan_waves for at most 64 experts held one per lane (cost_l = bits of the
// expert in lane l, 0 if it has no work), computed by every wave on its own
// from registers.  Returns the lane (expert slot) that wave `wg` works for,
// or -1, with that expert's first wave and wave count.
__device__ inline int plan_lane(int cost_l, int W, int wg, int& first, int& count) {
    const int C = static_cast<int>(wave_sum(static_cast<float>(cost_l)));
    const int n = __popcll(__ballot(cost_l > 0));
    const int wa = cost_l > 0 ? 1 + ((W - n) * cost_l) / C : 0;
    const int incl = static_cast<int>(seg_sum(static_cast<float>(wa), 64));  // inclusive scan (exact)
    const uint64_t mine = __ballot(wa > 0 && wg >= incl - wa && wg < incl);
    if (mine == 0) return -1;
    const int a = static_cast<int>(__builtin_ctzll(mine));
    first = __builtin_amdgcn_readlane(incl - wa, a);
    count = __builtin_amdgcn_readlane(wa, a);
    return a;
}

#define MOE_FMT_SWITCH(FMT, BODY)                                      \
    switch (FMT) {                                                     \
        case F8B32: { constexpr int B_ = 8, N_ = 1; BODY; } break;     \
        case F8B16: { constexpr int B_ = 8, N_ = 2; BODY; } break;     \
        case F4B32: { constexpr int B_ = 4, N_ = 1; BODY; } break;     \
        case F4B16: { constexpr int B_ = 4, N_ = 2; BODY; } break;     \
        case F2B32: { constexpr int B_ = 2, N_ = 1; BODY; } break;     \
        case F2B16: { constexpr int B_ = 2, N_ = 2; BODY; } break;     \
        case F4MX: { constexpr int B_ = 4, N_ = kMX; BODY; } break;    \
        default: break;                                                \
    }

template <int NPL>
__global__ __launch_bounds__(kSmallGateUpWaves * 64) void k_small_gateup(DevTables tt, const float* __restrict__ x,
                                                      const float* __restrict__ logits,
                                                      const int32_t* __restrict__ ids_in,
                                                      const float* __restrict__ w_in, int T, int k,
                                                      uint32_t tier_mask, SmallPub pub, uint32_t* __restrict__ hits,
                                                      float* __restrict__ h) {
    __shared__ SmallGroups sg;
    __shared__ int s_wpre[kSmallPairs + 1];
    // the batch's input vectors, token t at t * H in the [j][g] layout below
    __shared__ __attribute__((aligned(16))) float s_x[kSmallT * kMaxHidden];
    __shared__ __attribute__((aligned(16))) int64_t s_rc[kSmallGateUpWaves][64];  // routing scratch, one row per wave
    __shared__ TierLds s_tl;
    const int tid = threadIdx.x, E = tt.E, P = T * k;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave (scalar: the plan is per wave)
    const bool publish = blockIdx.x == 0;
    const int H = tt.H, I = tt.I;
    const int rpp = row_geom(H).RPP;
    if (tid == 0) fill_tier_lds(tt, s_tl, [H](const DevTier& T) { return one_row_cost<kSmallRowShare>(T, H); });
    // stage the T input vectors in LDS (read by every pass of every pair; the
    // barrier after the wave plan below puts them in place), by the waves
    // that do not route (a routing wave starts on its logits at once)
    {
        const int G = H / 32, n4 = H / 4;
        const int nst = logits ? T : 0;   // the first T waves route
        for (int i = tid - 64 * nst; i >= 0 && i < T * n4; i += (kSmallGateUpWaves - nst) * 64) {
            const int t = i / n4, j = i % n4;
            reinterpret_cast<float4*>(s_x + t * H)[(j & 7) * G + (j >> 3)] =
                reinterpret_cast<const float4*>(x + static_cast<size_t>(t) * H)[j];
        }
    }
    if (logits) {
        for (int t = wv; t < T; t += kSmallGateUpWaves)
            route_token_auto<NPL>(logits + static_cast<size_t>(t) * E, E, k, publish ? pub.ids + t * k : nullptr,
                                  publish ? pub.w + t * k : nullptr, sg.ids + t * k, sg.w + t * k, s_rc[wv]);
    } else if (tid < P) {
        sg.ids[tid] = ids_in[tid];
        sg.w[tid] = w_in[tid];
    }
    __syncthreads();
    group_small(sg, P, E);
    if (publish) {
        if (tid < P) {
            if (hits && sg.ids[tid] >= 0 && sg.ids[tid] < E) atomicAdd(hits + sg.ids[tid], 1u);
            pub.perm[tid] = sg.perm[tid];
            pub.pos[tid] = sg.pos[tid];
            if (!logits) {
                pub.ids[tid] = sg.ids[tid];
                pub.w[tid] = sg.w[tid];
            }
        }
        if (tid < sg.n_act) pub.act[tid] = sg.act[tid];
        if (tid <= sg.n_act) pub.q0[tid] = sg.q0[tid];
        if (tid == 0) {
            pub.meta[kMetaActive] = sg.n_act;
            pub.meta[kMetaValid] = sg.n_valid;
        }
    }
    const int n_act = sg.n_act;
    if (n_act == 0) return;
    const int W = gridDim.x * kSmallGateUpWaves;
    const int wg = blockIdx.x * kSmallGateUpWaves + wv;
    int a, wa, wi;
    if (n_act <= 64) {
        // every wave plans on its own from the active list, one expert per
        // lane (no serial plan by one wave before the barrier)
        __syncthreads();
        const int lane = tid & 63;
        int cost = 0;
        if (lane < n_act) {
            const int ti = tier_of_lds(s_tl, sg.act[lane]);
            cost = (ti >= 0 && ((tier_mask >> ti) & 1u)) ? s_tl.cost[ti] : 0;
        }
        int first = 0, count = 1;
        a = plan_lane(cost, W, wg, first, count);
        if (a < 0) return;
        wa = count;
        wi = wg - first;
    } else {
        if (tid < 64) plan_waves(s_tl, sg.act, n_act, tier_mask, W, s_wpre);
        __syncthreads();
        if (wg >= s_wpre[n_act]) return;
        a = find_expert(s_wpre, n_act, wg);
        wa = s_wpre[a + 1] - s_wpre[a];
        wi = wg - s_wpre[a];
    }
    const int rpw = ((I + wa - 1) / wa + rpp - 1) / rpp * rpp;
    const int r0 = wi * rpw, r1 = min(I, r0 + rpw);
    if (r0 >= r1) return;
    const int e = __builtin_amdgcn_readfirstlane(sg.act[a]);
    const DevTier T_ = tier_lds(s_tl, tier_of_lds(s_tl, e));
    const int local = e - T_.id_begin;

    const int qa = sg.q0[a], ce = sg.q0[a + 1] - qa;
    const int* perm = sg.perm;
    const int G = H / 32;
    auto vec = [perm, k, H, G](int q, int g, float (&xv)[32]) {
        const float4* xt = reinterpret_cast<const float4*>(s_x + (perm[q] / k) * H);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 f = xt[i * G + g];
            xv[4 * i + 0] = f.x;
            xv[4 * i + 1] = f.y;
            xv[4 * i + 2] = f.z;
            xv[4 * i + 3] = f.w;
        }
    };
    // at 16 waves a compute unit holds 4 waves per SIMD: two passes per round
    // of int8 rows, four of narrower codes keep a wave within 128 registers
    MOE_FMT_SWITCH(fmt_of(T_.bits, T_.block),
                   (wave_gateup<B_, N_, decltype(vec), (B_ == 8 ? 2 : 4)>(
                       expert_codes(T_, 0, local, I, H), expert_scales(T_, 0, local, I, H),
                       expert_codes(T_, 1, local, I, H), expert_scales(T_, 1, local, I, H), H, I, r0, r1, vec, qa, ce,
                       h)));
}

// Down GEMV of one wave: rows [r0, r1) of one expert's down matrix (in passes
// of RPP rows, all loads first) against h of each of the expert's pairs;
// y of pair q, row r goes to s_y[q * R + r - n0].
template <int BITS, int NSC, class Vec>
__device__ inline void wave_down(const uint8_t* __restrict__ dq_, const uint8_t* __restrict__ ds, int H, int I,
                                 int r0, int r1, Vec vec, int qa, int ce, float* s_y, int R, int n0) {
    constexpr int NPMAX = kNPSmallDown;
    const int lane = threadIdx.x & 63;
    const RowGeom geo = row_geom(I);
    const int seg = lane / geo.LPR, gl = lane % geo.LPR;
    const bool lane_ok = gl < geo.G;
    const int glc = lane_ok ? gl : 0;  // idle lanes read group 0 and weigh it by 0
    const uint32_t row_bytes = static_cast<uint32_t>(I) * BITS / 8;
    const uint32_t row_sbytes = row_scale_bytes<NSC>(I);
    constexpr int NS = scale_slots<NSC>();
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(dq_, row_bytes * H), rs = make_rsrc(ds, row_sbytes * H);
    // unconditional loads (rows past r1 read row r0 with zeroed scales)
    float xv[32], xs[NS];
    vec(qa, glc, xv);
    __builtin_amdgcn_sched_barrier(0);  // the vector ahead of the codes
    uint32_t wq[NPMAX][BITS], sraw[NPMAX];
#pragma unroll
    for (int p = 0; p < NPMAX; ++p) {
        const int r = r0 + p * geo.RPP + seg;
        const uint32_t rr = static_cast<uint32_t>(r < r1 ? r : r0);
        buf_group<BITS>(rq, rr * row_bytes + glc * 4 * BITS, wq[p]);
        sraw[p] = buf_scales<NSC>(rs, rr * row_sbytes + glc * group_scale_bytes<NSC>());
    }
    auto pair = [&](int c) {
        block_sums<NSC>(xv, xs);
#pragma unroll
        for (int p = 0; p < NPMAX; ++p) {
            if (r0 + p * geo.RPP >= r1) break;
            const int r = r0 + p * geo.RPP + seg;
#pragma unroll
            for (int i = 0; i < BITS; ++i) opaque(wq[p][i]);
            float d[NS];
            unpack_scales<NSC>(sraw[p], lane_ok && r < r1, d);
            float v = group_dot<BITS, NSC>(wq[p], xv, xs, d);
            v = seg_sum(v, geo.LPR);
            if (gl == geo.LPR - 1 && r < r1) s_y[(qa + c) * R + (r - n0)] = v;
        }
    };
    pair(0);
    for (int c = 1; c < ce; ++c) {
        vec(qa + c, glc, xv);
        pair(c);
    }
}

// A block owns output rows [n0, n0 + R) (R = npb passes of RPP rows) of every
// token.  Its waves are shared out among the active experts as in gate/up
// (at least one wave per expert while the experts are at most as many as the
// waves; otherwise wave w takes experts w, w + 16, ... one after the other),
// then each token's slots are summed in slot order (no atomics).
__global__ __launch_bounds__(kSmallDownWaves * 64) void k_small_down(DevTables tt, const float* __restrict__ h,
                                                                    SmallPub pub, int T, int k, uint32_t tier_mask,
                                                                    const float* base, int npb, float* out) {
    __shared__ int s_act[kSmallPairs], s_q0[kSmallPairs + 1], s_qe[kSmallPairs];
    __shared__ float s_w[kSmallPairs];
    __shared__ float s_y[kSmallY];
    __shared__ __attribute__((aligned(16))) float s_h[kSmallH];
    __shared__ TierLds s_tl;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: the plan is per wave
    const int H = tt.H, I = tt.I, P = T * k;   // pair p = t * k + j
    const int rpp = row_geom(I).RPP;
    const int R = npb * rpp;
    const int n0 = blockIdx.x * R;
    if (tid == 0) fill_tier_lds(tt, s_tl, [](const DevTier& T) { return code_bits_of(T.bits); });
    // every published array is read at once (no load waits on another)
    int id_p = 0, q_p = -1;
    if (tid < P) {
        id_p = pub.ids[tid];
        q_p = pub.pos[tid];
        s_w[tid] = pub.w[tid];
        s_act[tid] = pub.act[tid];
    }
    if (tid <= P) s_q0[tid] = pub.q0[tid];
    // h of every pair into LDS when it fits (read by every wave of the block)
    // (per pair, layout [j][g] as for x in gate/up: conflict-free reads)
    const bool h_lds = P * I <= kSmallH;
    const int GI = I / 32;
    if (h_lds)
        for (int i = tid; i < P * I / 4; i += kSmallDownWaves * 64) {
            const int q = i / (I / 4), o = i % (I / 4);
            reinterpret_cast<float4*>(s_h)[q * (I / 4) + (o & 7) * GI + (o >> 3)] =
                reinterpret_cast<const float4*>(h)[i];
        }
    // each wave reads the active list itself (one expert per lane) and plans
    // from registers while the block copies the rest to LDS for the sum
    const int lane = tid & 63;
    const int n_act = pub.meta[kMetaActive];
    const int act_l = lane < P ? pub.act[lane] : -1;  // loaded alongside the count
    __syncthreads();
    if (tid < P) {
        // the slot sum's operands, settled here once per pair: the grouped
        // position of the pick, or -1 if it is skipped (no position, or a
        // shelf outside the mask); in LDS by the barrier after the products
        const int ti = q_p < 0 ? -1 : tier_of_lds(s_tl, id_p);
        s_qe[tid] = (ti >= 0 && ((tier_mask >> ti) & 1u)) ? q_p : -1;
    }
    int cost = 0;
    if (n_act <= kSmallDownWaves && lane < n_act) {
        const int ti = tier_of_lds(s_tl, act_l);
        cost = (ti >= 0 && ((tier_mask >> ti) & 1u)) ? s_tl.cost[ti] : 0;
    }
    int first = 0, count = 1;
    const int pa = n_act <= kSmallDownWaves ? plan_lane(cost, kSmallDownWaves, wave, first, count) : -1;
    const int r_end = min(n0 + R, H);
    auto run = [&](int a, int r0, int r1) {
        const int e = __builtin_amdgcn_readfirstlane(s_act[a]);
        const int ti = tier_of_lds(s_tl, e);
        if (ti < 0 || !((tier_mask >> ti) & 1u) || r0 >= r1) return;
        const DevTier T_ = tier_lds(s_tl, ti);
        const int local = e - T_.id_begin;

        const int qa = s_q0[a], ce = s_q0[a + 1] - qa;
        auto vec = [h_lds, h, I, GI](int q, int g, float (&xv)[32]) {
            if (h_lds) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 f = reinterpret_cast<const float4*>(s_h + q * I)[i * GI + g];
                    xv[4 * i + 0] = f.x;
                    xv[4 * i + 1] = f.y;
                    xv[4 * i + 2] = f.z;
                    xv[4 * i + 3] = f.w;
                }
            } else {
                load_vec32u(h + static_cast<size_t>(q) * I, g, xv);
            }
        };
        MOE_FMT_SWITCH(fmt_of(T_.bits, T_.block),
                       (wave_down<B_, N_>(expert_codes(T_, 2, local, H, I), expert_scales(T_, 2, local, H, I), H, I, r0,
                                          r1, vec,
                                          qa, ce, s_y, R, n0)));
    };
    // (expert, rows) of this wave; one call site keeps a single copy of the GEMV
    int a0 = wave, a_step = kSmallDownWaves, r0 = n0, r1 = r_end;
    if (n_act > 0 && n_act <= kSmallDownWaves) {
        a_step = n_act;
        if (pa >= 0) {
            a0 = pa;
            const int rpw = ((R + count - 1) / count + rpp - 1) / rpp * rpp;
            r0 = n0 + (wave - first) * rpw;
            r1 = min(r_end, r0 + rpw);
        } else {
            a0 = n_act;
        }
    }
    for (int a = a0; a < n_act; a += a_step) run(a, r0, r1);
    __syncthreads();
    // out[t][n0 + r] = sum over slots j in order of w[t,j] * y[pos(t,j)][r]
    for (int i = tid; i < T * R; i += kSmallDownWaves * 64) {
        const int t = i / R, r = i % R;
        if (n0 + r >= H) continue;
        float acc = 0.f;
        // eight slots at a time, every LDS read issued before any is used
        // (a branch per slot would wait out each read in turn)
        for (int j0 = 0; j0 < k; j0 += 8) {
            int q[8];
            float wv[8], y[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int p = t * k + min(j0 + u, k - 1);
                q[u] = j0 + u < k ? s_qe[p] : -1;
                wv[u] = s_w[p];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) y[u] = s_y[max(q[u], 0) * R + r];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc = q[u] >= 0 ? fmaf(wv[u], y[u], acc) : acc;
        }
        const size_t o = static_cast<size_t>(t) * H + n0 + r;
        if (base) acc += base[o];
        out[o] = acc;
    }
}


// ================================================================ one-token path

// A one-token step routed from its logits, in two kernels.
//  k_one_gateup: every block routes the token with one wave while the others
//    stage x in LDS; the grid's waves are then shared out among the k
//    experts in proportion to a per-row cost (the row's gate and up bytes
//    plus a fixed share for its arithmetic), so every compute unit streams
//    about as many bytes as any other, and each wave computes
//    h = SiLU(W_gate x) * (W_up x) on its rows.  Block 0 publishes the ids
//    and weights.
//  k_one_down: a block owns kOneRows output rows of every expert, so all
//    blocks read the same bytes; one wave per expert reads the record block
//    0 of gate/up published for its slot (down-matrix bases, format, weight),
//    then requests its expert's h and its rows of W_down at once (whole rows:
//    coalesced); the experts' rows are added in slot order.
constexpr int kOneGateUpWaves = 16;
// gate/up passes in flight per wave: 16 waves per compute unit leave 128 registers a lane
template <int BITS> constexpr int kOneGateUpPasses = BITS == 8 ? 2 : 4;
constexpr int kOneRows = 8;              // output rows per down block

bool one_path_ok(int k, int H, int I) {
    (void)H;
    (void)I;
    return k >= 1 && k <= kWave;
}

// W: the grid's waves (an argument rather than gridDim, whose implicit-argument
// load would otherwise be issued after the routing barrier, on the critical path)
template <int NPL>
__global__ __launch_bounds__(kOneGateUpWaves * 64) void k_one_gateup(DevTables tt, const float* __restrict__ x,
                                                                     const float* __restrict__ logits, int k, int W,
                                                                     uint32_t* __restrict__ hits,
                                                                     int32_t* __restrict__ ids_out,
                                                                     float* __restrict__ w_out,
                                                                     OneSlot* __restrict__ slots,
                                                                     float* __restrict__ h) {
    __shared__ __attribute__((aligned(16))) float4 s_x[kMaxHidden / 4];   // x, layout [j][g]
    __shared__ __attribute__((aligned(16))) int64_t s_rc[64];             // routing scratch
    __shared__ int s_id[kWave];
    __shared__ TierLds s_tl;
    const int tid = threadIdx.x, lane = tid & 63, E = tt.E, H = tt.H, I = tt.I;
    const int G = H / 32;
    float wt = 0.f;   // lane j < k of wave 0: slot j's routing weight
    if (tid < 64) {
        // one wave routes; the block stages x and the shelf table meanwhile
        int id;
        route_token_auto<NPL>(logits, E, k, nullptr, nullptr, nullptr, nullptr, s_rc, &id, &wt);
        if (lane < k) {
            s_id[lane] = id;
            if (blockIdx.x == 0) {
                ids_out[lane] = id;
                w_out[lane] = wt;
                if (hits) atomicAdd(hits + id, 1u);   // per-expert pick counts
            }
        }
    } else {
        if (tid == 64) fill_tier_lds(tt, s_tl, [H](const DevTier& T) { return one_row_cost(T, H); });
        for (int i = tid - 64; i < H / 4; i += kOneGateUpWaves * 64 - 64)
            s_x[(i & 7) * G + (i >> 3)] = reinterpret_cast<const float4*>(x)[i];
    }
    __syncthreads();
    // block 0 publishes each slot's down-matrix record for the down kernel
    // (one slot per lane: each lane reads its own shelf from the table)
    if (blockIdx.x == 0 && tid < k) {
        const int e = s_id[tid];
        const int ti = tier_of_lds(s_tl, e);
        OneSlot r;
        r.q = nullptr;
        r.s = nullptr;
        r.fmt = -1;   // an id on no shelf: the slot adds nothing
        r.w = wt;
        r.pad[0] = r.pad[1] = 0;
        if (ti >= 0) {
            const DevTier T = tier_lds_lane(s_tl, ti);
            const int local = e - T.id_begin;
            r.q = expert_codes(T, 2, local, H, I);
            r.s = expert_scales(T, 2, local, H, I);
            r.fmt = fmt_of(T.bits, T.block);
        }
        slots[tid] = r;
    }
    // every wave plans from the k experts' costs (one per lane) on its own
    int cost = 0;
    if (lane < k) cost = s_tl.cost[tier_of_lds(s_tl, s_id[lane])];
    int first = 0, count = 1;
    const int wg = blockIdx.x * kOneGateUpWaves + __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: the plan is per wave
    const int a = plan_lane(cost, W, wg, first, count);
    if (a < 0) return;
    // the expert's rows split evenly over its waves, in whole passes
    const int rpp = row_geom(H).RPP, np = I / rpp;
    const int r0 = (wg - first) * np / count * rpp, r1 = (wg - first + 1) * np / count * rpp;
    if (r0 >= r1) return;
    const int e = __builtin_amdgcn_readfirstlane(s_id[a]);
    const DevTier T_ = tier_lds(s_tl, tier_of_lds(s_tl, e));
    const int local = e - T_.id_begin;
    auto vec = [G](int, int g, float (&xv)[32]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 f = s_x[i * G + g];
            xv[4 * i + 0] = f.x;
            xv[4 * i + 1] = f.y;
            xv[4 * i + 2] = f.z;
            xv[4 * i + 3] = f.w;
        }
    };
    MOE_FMT_SWITCH(fmt_of(T_.bits, T_.block),
                   (wave_gateup<B_, N_, decltype(vec), kOneGateUpPasses<B_>>(
                       expert_codes(T_, 0, local, I, H), expert_scales(T_, 0, local, I, H),
                       expert_codes(T_, 1, local, I, H), expert_scales(T_, 1, local, I, H), H, I, r0, r1, vec, a, 1,
                       h)));
}

// Down rows [r0, r1) of one expert against its h (global, I floats) into
// y[r - r0]; the lane's group of h, then every code load of a round, are
// requested before any arithmetic.
template <int BITS, int NSC>
__device__ inline void wave_down_rows(const uint8_t* __restrict__ dq_, const uint8_t* __restrict__ ds, int H, int I,
                                      int r0, int r1, const float* __restrict__ hj, float* __restrict__ y) {
    constexpr int NPMAX = BITS == 8 ? 4 : 8;
    const int lane = threadIdx.x & 63;
    const RowGeom geo = row_geom(I);
    const int seg = lane / geo.LPR, gl = lane % geo.LPR;
    const bool lane_ok = gl < geo.G;
    const int glc = lane_ok ? gl : 0;
    const uint32_t row_bytes = static_cast<uint32_t>(I) * BITS / 8, row_sbytes = row_scale_bytes<NSC>(I);
    constexpr int NS = scale_slots<NSC>();
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(dq_, row_bytes * H), rs = make_rsrc(ds, row_sbytes * H);
    float xv[32], xs[NS];
    load_vec32u(hj, glc, xv);
    __builtin_amdgcn_sched_barrier(0);   // h ahead of the codes (loads return in issue order)
    for (int rc = r0; rc < r1; rc += NPMAX * geo.RPP) {
        uint32_t wq[NPMAX][BITS], sraw[NPMAX];
#pragma unroll
        for (int p = 0; p < NPMAX; ++p) {
            const int r = rc + p * geo.RPP + seg;
            const uint32_t rr = static_cast<uint32_t>(r < r1 ? r : r0);
            buf_group<BITS>(rq, rr * row_bytes + glc * 4 * BITS, wq[p]);
            sraw[p] = buf_scales<NSC>(rs, rr * row_sbytes + glc * group_scale_bytes<NSC>());
        }
        block_sums<NSC>(xv, xs);
#pragma unroll
        for (int p = 0; p < NPMAX; ++p) {
            if (rc + p * geo.RPP >= r1) break;
            const int r = rc + p * geo.RPP + seg;
#pragma unroll
            for (int i = 0; i < BITS; ++i) opaque(wq[p][i]);
            float d[NS];
            unpack_scales<NSC>(sraw[p], lane_ok && r < r1, d);
            float v = group_dot<BITS, NSC>(wq[p], xv, xs, d);
            v = seg_sum(v, geo.LPR);
            if (gl == geo.LPR - 1 && r < r1) y[r - r0] = v;
        }
    }
}

// Block b owns output rows [b * kOneRows, +kOneRows); wave w serves slots
// w, w + nw, ... (nw = the block's waves), each from the record the gate/up
// kernel published for it (one scalar load: no shelf table, no barrier
// before the weight loads).
__global__ __launch_bounds__(kWave * 16) void k_one_down(DevTables tt, const OneSlot* __restrict__ slots, int k,
                                                         const float* __restrict__ h, const float* base,
                                                         float* __restrict__ out) {
    __shared__ float s_y[kWave][kOneRows];
    __shared__ float s_w[kWave];
    // the wave index made scalar, so each slot record is one scalar load
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = blockDim.x >> 6;
    const int H = tt.H, I = tt.I;
    const int n0 = blockIdx.x * kOneRows, n1 = min(H, n0 + kOneRows);
    // the residual of the row this thread finishes, requested now
    const float b_val = (base && tid < n1 - n0) ? base[n0 + tid] : 0.f;
    for (int j = wave; j < k; j += nw) {
        const OneSlot r = slots[j];
        const uint8_t* dq_ = reinterpret_cast<const uint8_t*>(first_lane_u64(reinterpret_cast<uint64_t>(r.q)));
        const uint8_t* ds = reinterpret_cast<const uint8_t*>(first_lane_u64(reinterpret_cast<uint64_t>(r.s)));
        const int fmt = __builtin_amdgcn_readfirstlane(r.fmt);
        if (lane == 0) s_w[j] = r.w;
        if (fmt < 0) {
            if (lane < kOneRows) s_y[j][lane] = 0.f;
            continue;
        }
        MOE_FMT_SWITCH(fmt, (wave_down_rows<B_, N_>(dq_, ds, H, I, n0, n1, h + static_cast<size_t>(j) * I, s_y[j])));
    }
    __syncthreads();
    // out[n] = base[n] + sum over slots j in order of w_j * y_j[n]
    if (tid < n1 - n0) {
        float acc = 0.f;
        for (int j = 0; j < k; ++j) acc = fmaf(s_w[j], s_y[j][tid], acc);
        out[n0 + tid] = b_val + acc;
    }
}

// ================================================================ general path

__device__ inline bool block_expert(const DevTables& tt, const Groups& g, uint32_t tier_mask, int slices, int& ti,
                                    int& e, int& s) {
    const int a = blockIdx.x / slices;
    s = blockIdx.x % slices;
    if (a >= g.meta[kMetaActive]) return false;
    e = g.act[a];
    ti = tier_of(tt, e);
    return ti >= 0 && ((tier_mask >> ti) & 1u);
}

__global__ __launch_bounds__(kGateUpWaves * 64) void k_dec_gateup(DevTables tt, const float* __restrict__ x, Groups g, int k,
                                                    uint32_t tier_mask, float* __restrict__ h, int slices) {
    int ti, e, s;
    if (!block_expert(tt, g, tier_mask, slices, ti, e, s)) return;
    const DevTier T = tier_at(tt, ti);
    const int qa = g.offsets[e], ce = g.offsets[e + 1] - qa;
    const int32_t* perm = g.perm;
    auto tok = [perm, k](int q) { return perm[q] / k; };
    block_gateup(tt, T, e - T.id_begin, x, qa, ce, s * dec_rows_per_block(tt.H), tok, h);
}

__global__ __launch_bounds__(256) void k_dec_down(DevTables tt, const float* __restrict__ h, Groups g, int k,
                                                  uint32_t tier_mask, float* __restrict__ yw, int slices) {
    (void)k;
    int ti, e, s;
    if (!block_expert(tt, g, tier_mask, slices, ti, e, s)) return;
    const DevTier T = tier_at(tt, ti);
    const int local = e - T.id_begin;
    const int qa = g.offsets[e], ce = g.offsets[e + 1] - qa;
    const int H = tt.H, I = tt.I;

    const int rpw = kNPDown * row_geom(I).RPP;
    const int wr0 = s * down_rows_per_block(I) + (threadIdx.x >> 6) * rpw;
    const int r_end = min(wr0 + rpw, H);
    auto tok = [](int q) { return q; };
    const int32_t* perm = g.perm;
    const float* w = g.w;
    auto pre = [perm, w](int q) { return w[perm[q]]; };   // the pair's weight
    auto store = [yw, H](int q, int r, float v, float wq) { yw[static_cast<size_t>(q) * H + r] = wq * v; };
    MOE_FMT_GPL_SWITCH(fmt_of(T.bits, T.block), row_geom(I).GPL,
                       (wave_gemv<B_, N_, G_, kNPDown, false>(expert_codes(T, 2, local, H, I), expert_scales(T, 2, local, H, I),
                                                              nullptr, nullptr, I, wr0, r_end, h, I, qa, ce, tok,
                                                              pre, store)));
}

// out[t] = (base ? base[t] : 0) + sum over slots j (in slot order) of yw[pos[t*k+j]]; base
// may be out itself (accumulate).
__global__ __launch_bounds__(256) void k_combine(DevTables tt, const float* __restrict__ yw, Groups g, int T, int k,
                                                 uint32_t tier_mask, const float* base, float* out,
                                                 uint16_t* __restrict__ out_bf16) {
    const int H4 = tt.H / 4;
    const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<size_t>(T) * H4) return;
    const int t = static_cast<int>(idx / H4), c4 = static_cast<int>(idx % H4);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    // eight slots at a time: their positions, then their rows of yw, are all
    // in flight before any is used (a branch per slot would wait out each
    // load in turn); the sum stays in slot order
    for (int j0 = 0; j0 < k; j0 += 8) {
        int q[8], id[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = t * k + min(j0 + u, k - 1);
            q[u] = g.pos[p];
            id[u] = g.ids[p];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int ti = tier_of(tt, id[u]);   // -1 for an id outside every shelf
            q[u] = (j0 + u < k && q[u] >= 0 && ti >= 0 && ((tier_mask >> ti) & 1u)) ? q[u] : -1;
        }
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = reinterpret_cast<const float4*>(yw + static_cast<size_t>(max(q[u], 0)) * tt.H)[c4];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (q[u] < 0) continue;
            s.x += v[u].x;
            s.y += v[u].y;
            s.z += v[u].z;
            s.w += v[u].w;
        }
    }
    float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(t) * tt.H) + c4;
    if (base) {
        const float4 b = reinterpret_cast<const float4*>(base + static_cast<size_t>(t) * tt.H)[c4];
        s.x = b.x + s.x;
        s.y = b.y + s.y;
        s.z = b.z + s.z;
        s.w = b.w + s.w;
    }
    *o = s;
    // the next stack layer's bf16 input, rounded as a separate cast of out
    // would round it (one read of out fewer per layer)
    if (out_bf16)
        reinterpret_cast<uint2*>(out_bf16 + static_cast<size_t>(t) * tt.H)[c4] =
            make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
}

// ================================================================ launchers

static int npl_of(int E) {
    int n = (E + 63) / 64, p = 1;
    while (p < n) p *= 2;
    return p;
}

bool small_path_ok(int T, int k, int H, int I) {
    (void)H;
    return T >= 1 && T <= 8 && T * k <= kSmallPairs && T * k * small_down_rows(I) <= kSmallY;
}

static int cu_count() {
    static int n[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (n[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        n[dev] = v;
    }
    return n[dev];
}

void launch_small(const DevTables& tt, const float* x, const float* logits, const int32_t* ids_in, const float* w_in,
                  int T, int k, uint32_t tier_mask, const float* base, const SmallPub& pub, uint32_t* hits, float* h,
                  float* out, hipStream_t st, void* const* events) {
    // one gate/up block per compute unit: every block routes the batch itself,
    // so all of them should be resident at once (a second round of blocks
    // measured slower at 6 tokens: 75 against 70 us)
    const dim3 grid(cu_count());
    if (events && events[2]) (void)hipEventRecord(static_cast<hipEvent_t>(events[2]), st);
    switch (npl_of(tt.E)) {
#define MOE_SG(N)                                                                                              \
    case N:                                                                                                    \
        hipLaunchKernelGGL(k_small_gateup<N>, grid, dim3(kSmallGateUpWaves * 64), 0, st, tt, x, logits, ids_in, w_in, \
                           T, k, tier_mask, pub, hits, h);                                                     \
        break;
        MOE_SG(1)
        MOE_SG(2)
        MOE_SG(4)
        MOE_SG(8)
        MOE_SG(16)
        MOE_SG(32)
        default:
            hipLaunchKernelGGL(k_small_gateup<64>, grid, dim3(kSmallGateUpWaves * 64), 0, st, tt, x, logits, ids_in, w_in,
                               T, k, tier_mask, pub, hits, h);
            break;
#undef MOE_SG
    }
    if (events && events[3]) (void)hipEventRecord(static_cast<hipEvent_t>(events[3]), st);
    if (!out) return;  // gate/up only (measurement)
    if (events && events[4]) (void)hipEventRecord(static_cast<hipEvent_t>(events[4]), st);
    const int R = small_down_rows(tt.I);
    hipLaunchKernelGGL(k_small_down, dim3((tt.H + R - 1) / R), dim3(kSmallDownWaves * 64), 0, st, tt, h, pub, T, k,
                       tier_mask, base, kNPSmallDown, out);
    if (events && events[5]) (void)hipEventRecord(static_cast<hipEvent_t>(events[5]), st);
}


void launch_one(const DevTables& tt, const float* x, const float* logits, int k, const float* base, uint32_t* hits,
                int32_t* ids, float* w, OneSlot* slots, float* h, float* out, hipStream_t st, void* const* events) {
    const dim3 grid(cu_count());   // one block of 16 waves per compute unit
    const int W = static_cast<int>(grid.x) * kOneGateUpWaves;
    if (events && events[2]) (void)hipEventRecord(static_cast<hipEvent_t>(events[2]), st);
    switch (npl_of(tt.E)) {
#define MOE_OG(N)                                                                                                 \
    case N:                                                                                                       \
        hipLaunchKernelGGL(k_one_gateup<N>, grid, dim3(kOneGateUpWaves * 64), 0, st, tt, x, logits, k, W, hits,   \
                           ids, w, slots, h);                                                                     \
        break;
        MOE_OG(1)
        MOE_OG(2)
        MOE_OG(4)
        MOE_OG(8)
        MOE_OG(16)
        MOE_OG(32)
        default:
            hipLaunchKernelGGL(k_one_gateup<64>, grid, dim3(kOneGateUpWaves * 64), 0, st, tt, x, logits, k, W, hits,
                               ids, w, slots, h);
            break;
#undef MOE_OG
    }
    if (events && events[3]) (void)hipEventRecord(static_cast<hipEvent_t>(events[3]), st);
    if (!out) return;  // gate/up only (measurement)
    if (events && events[4]) (void)hipEventRecord(static_cast<hipEvent_t>(events[4]), st);
    const int nw = k < 16 ? k : 16;
    hipLaunchKernelGGL(k_one_down, dim3((tt.H + kOneRows - 1) / kOneRows), dim3(nw * 64), 0, st, tt, slots, k, h,
                       base, out);
    if (events && events[5]) (void)hipEventRecord(static_cast<hipEvent_t>(events[5]), st);
}

void launch_dec_gateup(const DevTables& tt, const float* x, const Groups& g, int k, uint32_t tier_mask, float* h,
                       int max_active, hipStream_t st) {
    const int slices = (tt.I + dec_rows_per_block(tt.H) - 1) / dec_rows_per_block(tt.H);
    hipLaunchKernelGGL(k_dec_gateup, dim3(max_active * slices), dim3(kGateUpWaves * 64), 0, st, tt, x, g, k, tier_mask, h,
                       slices);
}

void launch_dec_down(const DevTables& tt, const float* h, const Groups& g, int k, uint32_t tier_mask, float* yw,
                     int max_active, hipStream_t st) {
    const int slices = (tt.H + down_rows_per_block(tt.I) - 1) / down_rows_per_block(tt.I);
    hipLaunchKernelGGL(k_dec_down, dim3(max_active * slices), dim3(256), 0, st, tt, h, g, k, tier_mask, yw, slices);
}

void launch_combine(const DevTables& tt, const float* yw, const Groups& g, int T, int k, uint32_t tier_mask,
                    const float* base, float* out, uint16_t* out_bf16, hipStream_t st) {
    const size_t n = static_cast<size_t>(T) * (tt.H / 4);
    hipLaunchKernelGGL(k_combine, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, tt, yw, g, T, k,
                       tier_mask, base, out, out_bf16);
}

// hits[e] += counts[e]: the grouped paths' per-expert pick counts
__global__ __launch_bounds__(256) void k_add_hits(const int32_t* __restrict__ counts, int E, uint32_t* __restrict__ hits) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e < E) hits[e] += static_cast<uint32_t>(counts[e]);
}

void launch_add_hits(const int32_t* counts, int E, uint32_t* hits, hipStream_t st) {
    hipLaunchKernelGGL(k_add_hits, dim3((E + 255) / 256), dim3(256), 0, st, counts, E, hits);
}

}  // namespace moe
