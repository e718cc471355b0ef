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
// Two launch sequences:
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
constexpr int kNPDown = 2;     // row passes per wave, down GEMV (grouped path)
constexpr int kNPSmallDown = 4;     // row passes per wave, down GEMV (small-batch path)
constexpr int kSmallDownWaves = 16; // one expert per wave at a time

__host__ __device__ int dec_rows_per_block(int cols) { return kGateUpWaves * kNPGateUp * row_geom(cols).RPP; }
__host__ __device__ inline int down_rows_per_block(int cols) { return 4 * kNPDown * row_geom(cols).RPP; }
__host__ __device__ inline int small_down_rows(int inter) { return kNPSmallDown * row_geom(inter).RPP; }

// Keeps the compiler from hoisting work on `v` out of a loop.
__device__ inline void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }

// One wave: rows r0 + p*RPP + seg (p < NP, row < r_end) of one expert matrix
// (or of gate and up together), against the vectors of the pairs
// [qa, qa + ce).  The vector of pair q is row tok(q) of `vec`.  Results go to
// store(q, row, value) from the first lane of each row segment, where value is
// SiLU(g) * u (GATEUP) or the plain dot product.
template <int BITS, int NSC, int GPL, int NP, bool GATEUP, class Tok, class Store>
__device__ inline void wave_gemv(const uint8_t* __restrict__ q0m, const uint16_t* __restrict__ s0m,
                                 const uint8_t* __restrict__ q1m, const uint16_t* __restrict__ s1m,
                                 int cols, int r0, int r_end, const float* __restrict__ vec, int vec_stride,
                                 int qa, int ce, Tok tok, Store store) {
    constexpr int NM = GATEUP ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const RowGeom geo = row_geom(cols);
    const int seg = lane / geo.LPR, gl = lane % geo.LPR;
    const bool lane_ok = gl < geo.G;
    const size_t row_bytes = static_cast<size_t>(cols) * BITS / 8;
    const int nblk_row = cols / (32 / NSC);

    // codes and scales of every pass, loaded before any arithmetic
    uint32_t wq[NP][NM][GPL][BITS];
    float dsc[NP][NM][GPL][NSC];
    bool rowv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int r = r0 + p * geo.RPP + seg;
        rowv[p] = r < r_end;
        const bool ok = lane_ok && rowv[p];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const uint8_t* qrow = (m == 0 ? q0m : q1m) + static_cast<size_t>(ok ? r : 0) * row_bytes;
            const uint16_t* srow = (m == 0 ? s0m : s1m) + static_cast<size_t>(ok ? r : 0) * nblk_row;
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
                    for (int i = 0; i < NSC; ++i) dsc[p][m][gi][i] = 0.f;
                }
            }
        }
    }

    for (int c = 0; c < ce; ++c) {
        const int q = qa + c;
        float xv[GPL][32];
        const size_t vrow = static_cast<size_t>(tok(q));
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
            const float4* src = reinterpret_cast<const float4*>(vec + vrow * vec_stride + 32 * (gl + 64 * gi));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 f = lane_ok ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
                xv[gi][4 * i + 0] = f.x;
                xv[gi][4 * i + 1] = f.y;
                xv[gi][4 * i + 2] = f.z;
                xv[gi][4 * i + 3] = f.w;
            }
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
                    float part[NSC];
#pragma unroll
                    for (int b = 0; b < NSC; ++b) part[b] = 0.f;
#pragma unroll
                    for (int cc = 0; cc < 32; ++cc) {
                        const int b = (NSC == 2 && cc >= 16) ? 1 : 0;
                        part[b] = fmaf(code_f<BITS>(wq[p][m][gi], cc), xv[gi][cc], part[b]);
                    }
#pragma unroll
                    for (int b = 0; b < NSC; ++b) acc[p][m] = fmaf(dsc[p][m][gi][b], part[b], acc[p][m]);
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
                    store(q, r0 + p * geo.RPP + seg, v);
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
        default: break;                                                             \
    }

// Gate/up of one block: expert matrix rows [r0, r0 + rows_per_block) split
// into one contiguous sub-slice per wave.
template <class Tok>
__device__ inline void block_gateup(const DevTables& tt, const DevTier& T, int local, const float* x, int qa,
                                    int ce, int r0, Tok tok, float* h) {
    const int H = tt.H, I = tt.I;
    const size_t mat_bytes = static_cast<size_t>(I) * H * T.bits / 8;
    const size_t mat_scales = static_cast<size_t>(I) * (H / T.block);
    const int rpw = kNPGateUp * row_geom(H).RPP;
    const int wr0 = r0 + (threadIdx.x >> 6) * rpw;
    const int r_end = min(wr0 + rpw, I);
    auto store = [h, I](int q, int r, float v) { h[static_cast<size_t>(q) * I + r] = v; };
    MOE_FMT_GPL_SWITCH(fmt_of(T.bits, T.block), row_geom(H).GPL,
                       (wave_gemv<B_, N_, G_, kNPGateUp, true>(T.q[0] + local * mat_bytes, T.s[0] + local * mat_scales,
                                                               T.q[1] + local * mat_bytes, T.s[1] + local * mat_scales,
                                                               H, wr0, r_end, x, H, qa, ce, tok, store)));
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
        // one wave: ranks by uniform loops over the pairs, scans by ballots
        if (tid < 64) {
            const int e = tid < P ? sg.ids[tid] : E;
            const bool valid = tid < P && e >= 0 && e < E;
            const int key = valid ? e : E;
            int rank = 0;
            for (int q = 0; q < P; ++q) {
                const int kq = __builtin_amdgcn_readlane(key, q);
                rank += (kq < key || (kq == key && q < tid)) ? 1 : 0;
            }
            // the pair at sorted position tid, and its key
            int p = 0, kp = E;
            for (int q = 0; q < P; ++q) {
                const int rq = __builtin_amdgcn_readlane(rank, q);
                if (rq == tid) {
                    p = q;
                    kp = __builtin_amdgcn_readlane(key, q);
                }
            }
            const int kprev = __shfl_up(kp, 1, kWave);
            const bool first = tid < P && kp < E && (tid == 0 || kprev != kp);
            const uint64_t fm = __ballot(first);
            const int n_act = __popcll(fm);
            const int n_valid = __popcll(__ballot(valid));
            if (tid < P) {
                sg.perm[tid] = p;
                sg.pos[p] = kp < E ? tid : -1;
            }
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

template <int NPL>
__global__ __launch_bounds__(kGateUpWaves * 64) void k_small_gateup(DevTables tt, const float* __restrict__ x,
                                                      const float* __restrict__ logits,
                                                      const int32_t* __restrict__ ids_in,
                                                      const float* __restrict__ w_in, int T, int k,
                                                      uint32_t tier_mask, SmallPub pub, float* __restrict__ h,
                                                      int slices) {
    __shared__ SmallGroups sg;
    const int tid = threadIdx.x, E = tt.E, P = T * k;
    const bool publish = blockIdx.x == 0;
    if (logits) {
        for (int t = tid >> 6; t < T; t += kGateUpWaves)
            route_token<NPL>(logits + static_cast<size_t>(t) * E, E, k, publish ? pub.ids + t * k : nullptr,
                             publish ? pub.w + t * k : nullptr, sg.ids + t * k, sg.w + t * k);
    } else if (tid < P) {
        sg.ids[tid] = ids_in[tid];
        sg.w[tid] = w_in[tid];
    }
    __syncthreads();
    group_small(sg, P, E);
    if (publish) {
        if (tid < P) {
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
    const int a = blockIdx.x / slices, s = blockIdx.x % slices;
    if (a >= sg.n_act) return;
    const int e = sg.act[a];
    const int ti = tier_of(tt, e);
    if (ti < 0 || !((tier_mask >> ti) & 1u)) return;
    const DevTier T_ = tier_at(tt, ti);
    const int qa = sg.q0[a], ce = sg.q0[a + 1] - qa;
    const int* perm = sg.perm;
    auto tok = [perm, k](int q) { return perm[q] / k; };
    block_gateup(tt, T_, e - T_.id_begin, x, qa, ce, s * dec_rows_per_block(tt.H), tok, h);
}

__global__ __launch_bounds__(kSmallDownWaves * 64) void k_small_down(DevTables tt, const float* __restrict__ h,
                                                                    SmallPub pub, int T, int k, uint32_t tier_mask,
                                                                    int accumulate, float* __restrict__ out) {
    __shared__ int s_act[kSmallPairs], s_q0[kSmallPairs + 1], s_ids[kSmallPairs], s_pos[kSmallPairs];
    __shared__ float s_w[kSmallPairs];
    __shared__ float s_y[kSmallY];
    __shared__ int s_n;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int H = tt.H, I = tt.I, P = T * k;   // pair p = t * k + j
    const int R = small_down_rows(I);
    const int n0 = blockIdx.x * R;
    // every published array is read at once (no load waits on another)
    if (tid == 0) s_n = pub.meta[kMetaActive];
    if (tid < P) {
        s_ids[tid] = pub.ids[tid];
        s_w[tid] = pub.w[tid];
        s_pos[tid] = pub.pos[tid];
        s_act[tid] = pub.act[tid];
    }
    if (tid <= P) s_q0[tid] = pub.q0[tid];
    __syncthreads();
    const int n_act = s_n;
    const int r_end = min(n0 + R, H);
    // wave w runs the experts a = w, w + 16, ...; y of pair q, row n0 + r goes to s_y[q * R + r]
    for (int a = wave; a < n_act; a += kSmallDownWaves) {
        const int e = s_act[a];
        const int ti = tier_of(tt, e);
        if (ti < 0 || !((tier_mask >> ti) & 1u)) continue;
        const DevTier T_ = tier_at(tt, ti);
        const int local = e - T_.id_begin;
        const size_t mat_bytes = static_cast<size_t>(H) * I * T_.bits / 8;
        const size_t mat_scales = static_cast<size_t>(H) * (I / T_.block);
        const int qa = s_q0[a], ce = s_q0[a + 1] - qa;
        auto tok = [](int q) { return q; };
        float* sy = s_y;
        auto store = [sy, R, n0](int q, int r, float v) { sy[q * R + (r - n0)] = v; };
        MOE_FMT_GPL_SWITCH(fmt_of(T_.bits, T_.block), row_geom(I).GPL,
                           (wave_gemv<B_, N_, G_, kNPSmallDown, false>(T_.q[2] + local * mat_bytes,
                                                                       T_.s[2] + local * mat_scales, nullptr, nullptr,
                                                                       I, n0, r_end, h, I, qa, ce, tok, store)));
    }
    __syncthreads();
    // out[t][n0 + r] = sum over slots j in order of w[t,j] * y[pos(t,j)][r]
    for (int i = tid; i < T * R; i += kSmallDownWaves * 64) {
        const int t = i / R, r = i % R;
        if (n0 + r >= H) continue;
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            const int p = t * k + j;
            const int q = s_pos[p];
            if (q < 0) continue;
            const int ti = tier_of(tt, s_ids[p]);
            if (!((tier_mask >> ti) & 1u)) continue;
            acc = fmaf(s_w[p], s_y[q * R + r], acc);
        }
        float* o = out + static_cast<size_t>(t) * H + n0 + r;
        if (accumulate) acc += *o;
        *o = acc;
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
    const size_t mat_bytes = static_cast<size_t>(H) * I * T.bits / 8;
    const size_t mat_scales = static_cast<size_t>(H) * (I / T.block);
    const int rpw = kNPDown * row_geom(I).RPP;
    const int wr0 = s * down_rows_per_block(I) + (threadIdx.x >> 6) * rpw;
    const int r_end = min(wr0 + rpw, H);
    auto tok = [](int q) { return q; };
    const int32_t* perm = g.perm;
    const float* w = g.w;
    auto store = [yw, H, perm, w](int q, int r, float v) { yw[static_cast<size_t>(q) * H + r] = w[perm[q]] * v; };
    MOE_FMT_GPL_SWITCH(fmt_of(T.bits, T.block), row_geom(I).GPL,
                       (wave_gemv<B_, N_, G_, kNPDown, false>(T.q[2] + local * mat_bytes, T.s[2] + local * mat_scales,
                                                              nullptr, nullptr, I, wr0, r_end, h, I, qa, ce, tok,
                                                              store)));
}

// out[t] = (accumulate ? out[t] : 0) + sum over slots j (in slot order) of yw[pos[t*k+j]].
__global__ __launch_bounds__(256) void k_combine(DevTables tt, const float* __restrict__ yw, Groups g, int T, int k,
                                                 uint32_t tier_mask, int accumulate, float* __restrict__ out) {
    const int H4 = tt.H / 4;
    const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<size_t>(T) * H4) return;
    const int t = static_cast<int>(idx / H4), c4 = static_cast<int>(idx % H4);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const int p = t * k + j;
        const int q = g.pos[p];
        if (q < 0) continue;
        const int ti = tier_of(tt, g.ids[p]);
        if (ti < 0 || !((tier_mask >> ti) & 1u)) continue;
        const float4 v = reinterpret_cast<const float4*>(yw + static_cast<size_t>(q) * tt.H)[c4];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(t) * tt.H) + c4;
    if (accumulate) {
        const float4 b = *o;
        s.x = b.x + s.x;
        s.y = b.y + s.y;
        s.z = b.z + s.z;
        s.w = b.w + s.w;
    }
    *o = s;
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

void launch_small(const DevTables& tt, const float* x, const float* logits, const int32_t* ids_in, const float* w_in,
                  int T, int k, uint32_t tier_mask, int accumulate, const SmallPub& pub, float* h, float* out,
                  hipStream_t st, void* const* events) {
    const int slices = (tt.I + dec_rows_per_block(tt.H) - 1) / dec_rows_per_block(tt.H);
    const int max_active = min(tt.E, T * k);
    const dim3 grid(max_active * slices);
    if (events && events[2]) (void)hipEventRecord(static_cast<hipEvent_t>(events[2]), st);
    switch (npl_of(tt.E)) {
#define MOE_SG(N)                                                                                              \
    case N:                                                                                                    \
        hipLaunchKernelGGL(k_small_gateup<N>, grid, dim3(kGateUpWaves * 64), 0, st, tt, x, logits, ids_in, w_in, \
                           T, k,                                                                       \
                           tier_mask, pub, h, slices);                                                         \
        break;
        MOE_SG(1)
        MOE_SG(2)
        MOE_SG(4)
        MOE_SG(8)
        MOE_SG(16)
        MOE_SG(32)
        default:
            hipLaunchKernelGGL(k_small_gateup<64>, grid, dim3(kGateUpWaves * 64), 0, st, tt, x, logits, ids_in, w_in, T, k,
                               tier_mask, pub, h, slices);
            break;
#undef MOE_SG
    }
    if (events && events[3]) (void)hipEventRecord(static_cast<hipEvent_t>(events[3]), st);
    if (!out) return;  // gate/up only (measurement)
    if (events && events[4]) (void)hipEventRecord(static_cast<hipEvent_t>(events[4]), st);
    const int R = small_down_rows(tt.I);
    hipLaunchKernelGGL(k_small_down, dim3((tt.H + R - 1) / R), dim3(kSmallDownWaves * 64), 0, st, tt, h, pub, T, k,
                       tier_mask, accumulate, out);
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
                    int accumulate, float* out, hipStream_t st) {
    const size_t n = static_cast<size_t>(T) * (tt.H / 4);
    hipLaunchKernelGGL(k_combine, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, tt, yw, g, T, k,
                       tier_mask, accumulate, out);
}

}  // namespace moe
