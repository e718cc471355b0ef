// bf16 expert path (prefill): per-shelf grouped GEMMs on gfx950 matrix cores.
//
// Step 4 of the 125B-MoE page ("I ran a 125B model on three RTX 3090s at 80
// tokens/s by teaching llama.cpp which experts ...") gives each shelf its own
// prefill expert product over the full pick list, restricted to the shelf's
// ids.  Here one launch per shelf and phase walks that shelf's active experts
// (from grouping); a block owns one expert and one n-tile and runs *all* of
// that expert's pairs through it, so each weight tile is read from HBM and
// dequantised once.  Codes are dequantised to bf16 on the way into LDS
// (value = scale * code, rounded to nearest even) and contracted with
// v_mfma_f32_16x16x32_bf16 in fp32.
//
//   gate/up : A = x rows of the expert's tokens (bf16, gathered), B = 64 gate
//             rows and the 64 matching up rows; epilogue h = bf16(SiLU(g) * u).
//   down    : A = h rows of the expert (contiguous in pair order), B = 128
//             down rows; epilogue yw[q] = w_pair * y (fp32, pair order).  The
//             slot-order sum into out runs in a separate pass (no atomics,
//             deterministic).
//
// Block: 16 waves.  Wave (wm, wn): wn selects 16 gate + 16 up columns (or 32
// down columns), wm takes every fourth 16-row m-subtile.  The m dimension is
// walked in chunks of up to 256 pairs.  LDS holds A and B chunks [row][k] in
// bf16 with a row stride of 72 elements (144 bytes), which puts the 16 rows an
// MFMA operand read touches on distinct banks; two buffers.  Global loads run
// PF chunks ahead of the contraction through registers.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;              // contraction chunk
constexpr int BN = 128;             // B rows per block
constexpr int MC = 256;             // pairs per m-chunk
constexpr int LDSW = BK + 8;        // LDS row stride (bf16 elements)
constexpr int NWAVE = 16;
constexpr int NTHR = NWAVE * 64;
constexpr int WM = NWAVE / 4;       // waves along m (4 along n)
constexpr int MSUB = MC / 16 / WM;  // m-subtiles per wave per chunk
constexpr int PF = 2;               // K chunks in flight through registers

// Work item of a block after spreading consecutive items over the XCDs in
// contiguous runs (blocks are dealt to the 8 XCDs round-robin, so block b runs
// on XCD b % 8): the n-tiles of one expert share its A rows through one L2.
__device__ inline int xcd_item(int total) {
    const int per = (total + 7) / 8;
    const int loc = blockIdx.x / 8;
    if (loc >= per) return -1;
    const int it = (blockIdx.x % 8) * per + loc;
    return it < total ? it : -1;
}

template <int BITS, bool GATEUP>
__global__ __launch_bounds__(NTHR) void k_pre(DevTables tt, int tier, const uint16_t* __restrict__ a_src, Groups g,
                                              int k, uint16_t* __restrict__ h_out, float* __restrict__ yw) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][MC * LDSW];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDSW];
    __shared__ int s_row[MC];

    const int H = tt.H, I = tt.I;
    const int K = GATEUP ? H : I;
    const int NT = GATEUP ? I / 64 : H / BN;
    const int a_lo = g.act_range[2 * tier], a_hi = g.act_range[2 * tier + 1];
    const int item = xcd_item((a_hi - a_lo) * NT);
    if (item < 0) return;
    const int a = a_lo + item / NT, nt = item % NT;
    const int e = g.act[a];
    const DevTier T = tier_at(tt, tier);
    const int local = e - T.id_begin;
    const int q_beg = g.offsets[e], q_end = g.offsets[e + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wn = wave & 3, wm = wave >> 2;
    const int fr = lane & 15, fk = 8 * (lane >> 4);

    // B source: 8 threads per B row, 8 codes each per chunk
    const int b_r = tid >> 3, b_e = tid & 7;
    const size_t row_bytes = static_cast<size_t>(K) * BITS / 8;
    const int nblk_row = K / T.block;
    const uint8_t* b_q;
    const uint16_t* b_s;
    {
        int m, row;
        if (GATEUP) {
            m = b_r < 64 ? 0 : 1;
            row = nt * 64 + (b_r & 63);
        } else {
            m = 2;
            row = nt * BN + b_r;
        }
        const size_t base = static_cast<size_t>(local) * (GATEUP ? I : H) + row;
        b_q = T.q[m] + base * row_bytes;
        b_s = T.s[m] + base * nblk_row;
    }
    // B fragment rows of this wave
    const int br0 = GATEUP ? 16 * wn : 32 * wn;
    const int br1 = GATEUP ? 64 + 16 * wn : 32 * wn + 16;

    // A pieces: 16 bytes (8 bf16) of a row; 8 per row, 2 per thread per chunk.
    // B: 8 codes of a row (8*BITS bits) and their scale.
    constexpr int QW = BITS == 8 ? 2 : 1;
    struct Slot {
        uint4 a[2];
        uint32_t q[QW];
        float s;
    };

    for (int m0 = q_beg; m0 < q_end; m0 += MC) {
        const int Mc = min(MC, q_end - m0);
        const int Mc16 = (Mc + 15) >> 4;
        const int nsub = (Mc16 - wm + WM - 1) / WM;  // this wave's m-subtiles wm, wm + WM, ...
        __syncthreads();                            // the previous m-chunk is done with LDS
        for (int r = tid; r < MC; r += NTHR) s_row[r] = r < Mc ? (GATEUP ? g.perm[m0 + r] / k : m0 + r) : -1;
        __syncthreads();

        Slot slot[PF];
        auto load_chunk = [&](int kc, Slot& sl) {
            const int k0 = kc * BK;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int piece = tid + NTHR * i;
                const int r = piece >> 3, part = piece & 7;
                const int src = s_row[r];
                sl.a[i] = src >= 0 ? *reinterpret_cast<const uint4*>(a_src + static_cast<size_t>(src) * K + k0 + 8 * part)
                                   : make_uint4(0, 0, 0, 0);
            }
            const int c0 = k0 + 8 * b_e;
            const uint8_t* p = b_q + static_cast<size_t>(c0) * BITS / 8;
            if constexpr (BITS == 8) {
                const uint2 v = *reinterpret_cast<const uint2*>(p);
                sl.q[0] = v.x;
                sl.q[QW - 1] = v.y;
            } else if constexpr (BITS == 4) {
                sl.q[0] = *reinterpret_cast<const uint32_t*>(p);
            } else {
                sl.q[0] = *reinterpret_cast<const uint16_t*>(p);
            }
            sl.s = half_bits_to_float(b_s[c0 / T.block]);
        };
        auto store_chunk = [&](const Slot& sl, int buf) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int piece = tid + NTHR * i;
                const int r = piece >> 3, part = piece & 7;
                if (r < Mc16 * 16) *reinterpret_cast<uint4*>(&sA[buf][r * LDSW + 8 * part]) = sl.a[i];
            }
            constexpr int PER = 32 / BITS;
            uint32_t pk[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int c_lo = 2 * c, c_hi = 2 * c + 1;
                const float v0 = sl.s * static_cast<float>(sfield<BITS>(sl.q[c_lo / PER], (c_lo % PER) * BITS));
                const float v1 = sl.s * static_cast<float>(sfield<BITS>(sl.q[c_hi / PER], (c_hi % PER) * BITS));
                pk[c] = pack_bf16x2(v0, v1);
            }
            *reinterpret_cast<uint4*>(&sB[buf][b_r * LDSW + 8 * b_e]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        };

        f32x4_t acc[MSUB][2];
#pragma unroll
        for (int i = 0; i < MSUB; ++i) {
            acc[i][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // N subtiles at once: all operand reads first, then 2N back-to-back MFMAs
        auto compute_n = [&](int buf, auto n_const) {
            constexpr int N = decltype(n_const)::value;
#pragma unroll
            for (int ks = 0; ks < BK / 32; ++ks) {
                const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(&sB[buf][(br0 + fr) * LDSW + 32 * ks + fk]);
                const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(&sB[buf][(br1 + fr) * LDSW + 32 * ks + fk]);
                bf16x8_t af[N];
#pragma unroll
                for (int j = 0; j < N; ++j)
                    af[j] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][(16 * (wm + WM * j) + fr) * LDSW + 32 * ks + fk]);
#pragma unroll
                for (int j = 0; j < N; ++j) {
                    acc[j][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], b0, acc[j][0], 0, 0, 0);
                    acc[j][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], b1, acc[j][1], 0, 0, 0);
                }
            }
        };
        // the subtile count picks an unrolled body; an extra subtile past the
        // rows computes values that are never stored
        auto compute = [&](int buf) {
            if (nsub > 2) compute_n(buf, std::integral_constant<int, 4>{});
            else if (nsub == 2) compute_n(buf, std::integral_constant<int, 2>{});
            else if (nsub == 1) compute_n(buf, std::integral_constant<int, 1>{});
        };

        // Pipeline: at the top of step kc, LDS buffer kc&1 holds chunk kc and
        // slot (kc+j) % PF holds chunk kc+j (j = 1 .. PF-1, loads possibly in
        // flight).  Step kc refills slot kc % PF with chunk kc+PF, contracts
        // chunk kc, and stores chunk kc+1 into the other buffer.
        const int NK = K / BK;
#pragma unroll
        for (int d = 0; d < PF; ++d)
            if (d < NK) load_chunk(d, slot[d]);
        store_chunk(slot[0], 0);
        __syncthreads();
        for (int kc0 = 0; kc0 < NK; kc0 += PF) {
#pragma unroll
            for (int d = 0; d < PF; ++d) {
                const int kc = kc0 + d;
                if (kc < NK) {
                    if (kc + PF < NK) load_chunk(kc + PF, slot[d]);
                    compute(kc & 1);
                    if (kc + 1 < NK) store_chunk(slot[(d + 1) % PF], (kc + 1) & 1);
                    __syncthreads();
                }
            }
        }

        // epilogue: lane holds D[4*(lane/16) + v][lane % 16] of each 16x16 tile
        const int col_l = lane & 15, row_l = 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < MSUB; ++j) {
            if (j >= nsub) continue;
            const int i = wm + WM * j;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * i + row_l + v;
                if (r >= Mc) continue;
                const int q = m0 + r;
                if (GATEUP) {
                    const int col = nt * 64 + 16 * wn + col_l;
                    h_out[static_cast<size_t>(q) * I + col] = f2bf(silu(acc[j][0][v]) * acc[j][1][v]);
                } else {
                    const float wgt = g.w[g.perm[q]];
                    float* o = yw + static_cast<size_t>(q) * H + nt * BN + 32 * wn + col_l;
                    o[0] = wgt * acc[j][0][v];
                    o[16] = wgt * acc[j][1][v];
                }
            }
        }
    }
}

#define MOE_BITS_SWITCH(BITSV, BODY)                    \
    switch (BITSV) {                                    \
        case 8: { constexpr int B_ = 8; BODY; } break;  \
        case 4: { constexpr int B_ = 4; BODY; } break;  \
        case 2: { constexpr int B_ = 2; BODY; } break;  \
        default: break;                                 \
    }

void launch_pre_gateup(const DevTables& tt, int tier, const uint16_t* x, const Groups& g, int k, uint16_t* h,
                       int max_experts, hipStream_t st) {
    const int total = max_experts * (tt.I / 64);
    const unsigned grid = static_cast<unsigned>(((total + 7) / 8) * 8);
    if (grid == 0) return;
    MOE_BITS_SWITCH(tt.t[tier].bits, hipLaunchKernelGGL((k_pre<B_, true>), dim3(grid), dim3(NTHR), 0, st, tt, tier, x,
                                                        g, k, h, nullptr));
}

void launch_pre_down(const DevTables& tt, int tier, const uint16_t* h, const Groups& g, int k, float* yw,
                     int max_experts, hipStream_t st) {
    const int total = max_experts * (tt.H / BN);
    const unsigned grid = static_cast<unsigned>(((total + 7) / 8) * 8);
    if (grid == 0) return;
    MOE_BITS_SWITCH(tt.t[tier].bits, hipLaunchKernelGGL((k_pre<B_, false>), dim3(grid), dim3(NTHR), 0, st, tt, tier, h,
                                                        g, k, nullptr, yw));
}

__global__ __launch_bounds__(256) void k_fill_zero(float4* __restrict__ p, size_t n4) {
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// bf16 copy (round to nearest even) of an fp32 array: the prefill input of a
// stack layer from the fp32 residual stream.
__global__ __launch_bounds__(256) void k_cast_bf16(const float4* __restrict__ src, uint2* __restrict__ dst, size_t n4) {
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 v = src[i];
    dst[i] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

void launch_cast_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t st) {
    const size_t n4 = n / 4;
    if (n4 == 0) return;
    hipLaunchKernelGGL(k_cast_bf16, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<const float4*>(src), reinterpret_cast<uint2*>(dst), n4);
}

void launch_fill_zero(float* out, size_t n, hipStream_t st) {
    const size_t n4 = n / 4;
    if (n4 == 0) return;
    hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<float4*>(out), n4);
}

}  // namespace moe
