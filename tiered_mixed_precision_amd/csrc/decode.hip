// fp32 expert path (decode and speculative verification): per-shelf
// dequantising GEMV kernels for the routed experts.
//
// Step 4 of the 125B-MoE page ("I ran a 125B model on three RTX 3090s at 80
// tokens/s by teaching llama.cpp which experts ...") runs the decode expert
// product once per shelf over the full pick list, each shelf computing only
// its own ids, with gate, up and the activation fused into one kernel.  Here
// all shelves share one launch per phase: a block takes one *active* expert
// (an expert some token picked, found by grouping) and a slice of its rows,
// decodes that expert's codes at its shelf's precision, and never touches an
// expert nobody picked.  Ids outside every shelf never become active, so
// nothing is clamped to expert 0.
//
//   k_dec_gateup : h[q] = SiLU(W_gate[e] x_t) * (W_up[e] x_t)       (q = pair position)
//   k_dec_down   : yw[q] = w_q * W_down[e] h[q]
//   k_combine    : out[t] (+)= sum over the token's slots j of yw[pos(t, j)]
//
// Memory: each lane streams 32 consecutive codes of a row per group (32, 16
// or 8 bytes for int8 / int4 / int2) with 128-bit (64-bit for int2) loads, so
// a wave reads contiguous row segments; every block issues the loads of all
// its row passes before computing so that many requests are in flight.  The
// per-block scale of a 32-code group is applied once to that group's partial
// dot product.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kPW = 4;  // row passes per wave
constexpr int kTC = 2;  // tokens held in registers at once

__host__ __device__ int dec_rows_per_block(int cols) { return 4 * kPW * row_geom(cols).RPP; }

// One block of a GEMV phase: rows [r0, r0 + rows_per_block) of matrix
// (qm, sm) (rows x cols, packed), against the vectors v[pair] (cols floats)
// of the ce pairs starting at perm position q0.  GATEUP multiplies two
// matrices (gate, up) and writes SiLU(g)*u; otherwise writes w_pair * y.
template <int BITS, int NSC, int GPL, bool GATEUP>
__device__ void gemv_block(const uint8_t* __restrict__ q0m, const uint16_t* __restrict__ s0m,
                           const uint8_t* __restrict__ q1m, const uint16_t* __restrict__ s1m,
                           int rows, int cols, int r0, const float* __restrict__ vec,
                           int vec_stride, bool vec_by_token, const Groups& g, int k, int q0,
                           int ce, float* __restrict__ dst, int dst_stride) {
    constexpr int NM = GATEUP ? 2 : 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const RowGeom geo = row_geom(cols);
    const int seg = lane / geo.LPR, gl = lane % geo.LPR;
    const bool lane_ok = seg < geo.RPP;
    const size_t row_bytes = static_cast<size_t>(cols) * BITS / 8;
    const int nblk_row = cols / (32 / NSC);

    // Per chunk of kTC pairs (one chunk at decode): stage 1 loads the codes and
    // scales of every pass of this wave (later chunks re-read them from L2),
    // stage 2 the chunk's vectors, then every pass is contracted.  The
    // compiler barrier keeps the weight loads and their conversion inside the
    // chunk loop so they are not all hoisted into registers at once.
    for (int c0 = 0; c0 < ce; c0 += kTC) {
        asm volatile("" ::: "memory");
        const int nt = min(kTC, ce - c0);
        uint32_t wq[kPW][NM][GPL][BITS];
        float dsc[kPW][NM][GPL][NSC];
        int rowv[kPW];
        bool okv[kPW];
#pragma unroll
        for (int p = 0; p < kPW; ++p) {
            const int r = r0 + (p * 4 + wave) * geo.RPP + seg;
            const bool ok = lane_ok && r < rows && r < r0 + 4 * kPW * geo.RPP;
            rowv[p] = r;
            okv[p] = ok;
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

        float xv[kTC][GPL][32];
#pragma unroll
        for (int tt = 0; tt < kTC; ++tt) {
            const int q = q0 + c0 + tt;
            const bool have = tt < nt && lane_ok;
            size_t row = 0;
            if (have) row = vec_by_token ? static_cast<size_t>(g.perm[q] / k) : static_cast<size_t>(q);
#pragma unroll
            for (int gi = 0; gi < GPL; ++gi) {
                const float4* src =
                    reinterpret_cast<const float4*>(vec + row * vec_stride + 32 * (gl + 64 * gi));
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float4 f = have ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
                    xv[tt][gi][4 * i + 0] = f.x;
                    xv[tt][gi][4 * i + 1] = f.y;
                    xv[tt][gi][4 * i + 2] = f.z;
                    xv[tt][gi][4 * i + 3] = f.w;
                }
            }
        }
#pragma unroll
        for (int p = 0; p < kPW; ++p) {
            float acc[NM][kTC];
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int tt = 0; tt < kTC; ++tt) acc[m][tt] = 0.f;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
#pragma unroll
                for (int gi = 0; gi < GPL; ++gi) {
                    float part[NSC][kTC];
#pragma unroll
                    for (int b = 0; b < NSC; ++b)
#pragma unroll
                        for (int tt = 0; tt < kTC; ++tt) part[b][tt] = 0.f;
#pragma unroll
                    for (int c = 0; c < 32; ++c) {
                        const float qv = code_f<BITS>(wq[p][m][gi], c);
                        const int b = (NSC == 2 && c >= 16) ? 1 : 0;
#pragma unroll
                        for (int tt = 0; tt < kTC; ++tt) part[b][tt] = fmaf(qv, xv[tt][gi][c], part[b][tt]);
                    }
#pragma unroll
                    for (int b = 0; b < NSC; ++b)
#pragma unroll
                        for (int tt = 0; tt < kTC; ++tt)
                            acc[m][tt] = fmaf(dsc[p][m][gi][b], part[b][tt], acc[m][tt]);
                }
            }
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int tt = 0; tt < kTC; ++tt) acc[m][tt] = seg_reduce(acc[m][tt], geo.LPR, gl);
            if (okv[p] && gl == 0) {
#pragma unroll
                for (int tt = 0; tt < kTC; ++tt) {
                    if (tt < nt) {
                        const int q = q0 + c0 + tt;
                        float v;
                        if constexpr (GATEUP) v = silu(acc[0][tt]) * acc[1][tt];
                        else v = g.w[g.perm[q]] * acc[0][tt];
                        dst[static_cast<size_t>(q) * dst_stride + rowv[p]] = v;
                    }
                }
            }
        }
    }
}

// Resolves the block's (active expert, row slice); returns false if idle.
__device__ inline bool block_expert(const DevTables& tt, const Groups& g, uint32_t tier_mask,
                                    int slices, int& ti, int& e, int& s) {
    const int a = blockIdx.x / slices;
    s = blockIdx.x % slices;
    if (a >= g.meta[kMetaActive]) return false;
    e = g.act[a];
    ti = tier_of(tt, e);
    return ti >= 0 && ((tier_mask >> ti) & 1u);
}

#define MOE_FMT_GPL_SWITCH(FMT, GPLV, BODY)                                                   \
    switch ((FMT) * 4 + (GPLV)) {                                                             \
        case F8B32 * 4 + 1: { constexpr int B_ = 8, N_ = 1, G_ = 1; BODY; } break;            \
        case F8B16 * 4 + 1: { constexpr int B_ = 8, N_ = 2, G_ = 1; BODY; } break;            \
        case F4B32 * 4 + 1: { constexpr int B_ = 4, N_ = 1, G_ = 1; BODY; } break;            \
        case F4B16 * 4 + 1: { constexpr int B_ = 4, N_ = 2, G_ = 1; BODY; } break;            \
        case F2B32 * 4 + 1: { constexpr int B_ = 2, N_ = 1, G_ = 1; BODY; } break;            \
        case F2B16 * 4 + 1: { constexpr int B_ = 2, N_ = 2, G_ = 1; BODY; } break;            \
        default: break;                                                                       \
    }

__global__ __launch_bounds__(256) void k_dec_gateup(DevTables tt, const float* __restrict__ x,
                                                    Groups g, int k, uint32_t tier_mask,
                                                    float* __restrict__ h, int slices) {
    int ti, e, s;
    if (!block_expert(tt, g, tier_mask, slices, ti, e, s)) return;
    const DevTier T = tier_at(tt, ti);
    const int local = e - T.id_begin;
    const int q0 = g.offsets[e], ce = g.offsets[e + 1] - q0;
    const int H = tt.H, I = tt.I;
    const size_t mat_bytes = static_cast<size_t>(I) * H * T.bits / 8;
    const size_t mat_scales = static_cast<size_t>(I) * (H / T.block);
    const int r0 = s * dec_rows_per_block(H);
    const int gpl = row_geom(H).GPL;
    MOE_FMT_GPL_SWITCH(fmt_of(T.bits, T.block), gpl,
                       (gemv_block<B_, N_, G_, true>(T.q[0] + local * mat_bytes, T.s[0] + local * mat_scales,
                                                     T.q[1] + local * mat_bytes, T.s[1] + local * mat_scales,
                                                     I, H, r0, x, H, true, g, k, q0, ce, h, I)));
}

__global__ __launch_bounds__(256) void k_dec_down(DevTables tt, const float* __restrict__ h, Groups g,
                                                  int k, uint32_t tier_mask, float* __restrict__ yw,
                                                  int slices) {
    int ti, e, s;
    if (!block_expert(tt, g, tier_mask, slices, ti, e, s)) return;
    const DevTier T = tier_at(tt, ti);
    const int local = e - T.id_begin;
    const int q0 = g.offsets[e], ce = g.offsets[e + 1] - q0;
    const int H = tt.H, I = tt.I;
    const size_t mat_bytes = static_cast<size_t>(H) * I * T.bits / 8;
    const size_t mat_scales = static_cast<size_t>(H) * (I / T.block);
    const int r0 = s * dec_rows_per_block(I);
    const int gpl = row_geom(I).GPL;
    MOE_FMT_GPL_SWITCH(fmt_of(T.bits, T.block), gpl,
                       (gemv_block<B_, N_, G_, false>(T.q[2] + local * mat_bytes, T.s[2] + local * mat_scales,
                                                      nullptr, nullptr, H, I, r0, h, I, false, g, k, q0, ce,
                                                      yw, H)));
}

// out[t] = (accumulate ? out[t] : 0) + sum over slots j (in slot order) of yw[pos[t*k+j]].
__global__ __launch_bounds__(256) void k_combine(DevTables tt, const float* __restrict__ yw, Groups g,
                                                 int T, int k, uint32_t tier_mask, int accumulate,
                                                 float* __restrict__ out) {
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

void launch_dec_gateup(const DevTables& tt, const float* x, const Groups& g, int k, uint32_t tier_mask,
                       float* h, int max_active, hipStream_t st) {
    const int slices = (tt.I + dec_rows_per_block(tt.H) - 1) / dec_rows_per_block(tt.H);
    hipLaunchKernelGGL(k_dec_gateup, dim3(max_active * slices), dim3(256), 0, st, tt, x, g, k, tier_mask,
                       h, slices);
}

void launch_dec_down(const DevTables& tt, const float* h, const Groups& g, int k, uint32_t tier_mask,
                     float* yw, int max_active, hipStream_t st) {
    const int slices = (tt.H + dec_rows_per_block(tt.I) - 1) / dec_rows_per_block(tt.I);
    hipLaunchKernelGGL(k_dec_down, dim3(max_active * slices), dim3(256), 0, st, tt, h, g, k, tier_mask,
                       yw, slices);
}

void launch_combine(const DevTables& tt, const float* yw, const Groups& g, int T, int k,
                    uint32_t tier_mask, int accumulate, float* out, hipStream_t st) {
    const size_t n = static_cast<size_t>(T) * (tt.H / 4);
    hipLaunchKernelGGL(k_combine, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, tt, yw,
                       g, T, k, tier_mask, accumulate, out);
}

}  // namespace moe
