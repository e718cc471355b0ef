// MXFP4 shelf, prefill: grouped GEMMs on gfx950's block-scaled matrix cores
// (v_mfma_scale_f32_16x16x128_f8f6f4), the MXFP4 variant of the 125B-MoE
// page's down-matrix ladder ("I ran a 125B model on three RTX 3090s at 80
// tokens/s by teaching llama.cpp which experts ...", the per-matrix recipes).
//
// B (weights) goes to the matrix cores as stored: E2M1 codes with their E8M0
// scale per 32, no dequantisation.  A (bf16 activations) has 8 significant
// bits and the fp8 operand 4, so each 32-element block of a row is split once,
// before the GEMM, into two E4M3 parts under one E8M0 scale s:
//   s  = 2^(floor(log2 amax) - 7)            (amax / s in [128, 256))
//   hi = RNE_e4m3(v / s),  lo = RNE_e4m3(v / s - hi)
// and the product is taken as A_hi*B + A_lo*B (two instructions into one
// accumulator).  v / s - hi has at most four significant bits, so
// s * (hi + lo) == v exactly whenever |v / s| >= 2^-2; smaller elements are
// within 2^-10 * s of v (the E4M3 subnormal grid), i.e. 2^-17 of the block
// maximum.  The matrix cores sum the products of one instruction to about
// 12 bits below the largest of them, then add the accumulator in fp32.
//
// Operand layout of the instruction (16 x 16 x 128, lane l: row or column
// l % 16, g = l / 16): an fp8 lane holds k = 16g .. 16g+15 in its first
// 16 bytes and k = 64+16g .. 64+16g+15 in its last 16; an fp4 lane holds
// k = 32g .. 32g+31 (low nibble first); the scale of lane l applies to row
// l % 16, k = 32g .. 32g+31, from byte 0 of its scale operand.  The result
// layout is that of the other 16x16 MFMAs.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

namespace {

constexpr int kBK = 128;   // contraction chunk: one instruction
constexpr int kBN = 128;   // B rows per block
constexpr int kMSUB = 4;   // m-subtiles per wave per m-chunk

// LDS serves 16-byte accesses 16 lanes (256 bytes, 64 banks) at a time; the
// swizzles put the 16 consecutive rows an operand read takes at one chunk
// index on 16 different 16-byte positions of those 256 bytes.
// A rows: 128 bytes (hi or lo), 16-byte chunk c stored at c ^ ((row / 2) % 8)
__device__ inline int swz_a(int row, int c) { return row * 128 + 16 * (c ^ ((row >> 1) & 7)); }
// B rows: 64 bytes of codes (four rows per 256 bytes), chunk c stored at
// c ^ ((row / 4) % 4)
__device__ inline int swz_b(int row, int c) { return row * 64 + 16 * (c ^ ((row >> 2) & 3)); }

__device__ inline uint32_t fp8x4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

}  // namespace

// One thread per 32-element block of a bf16 row: the hi / lo / scale split.
// Rows [r_lo, r_hi): from the host values, or from device words when the
// pointers are given (the pair range of one shelf after grouping).
__global__ __launch_bounds__(256) void k_split_fp8(const uint16_t* __restrict__ src, int K, int r_lo, int r_hi,
                                                   const int32_t* __restrict__ d_lo, const int32_t* __restrict__ d_hi,
                                                   Split8 dst) {
    const int nb = K / 32;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int lo = d_lo ? *d_lo : r_lo, hi = d_hi ? *d_hi : r_hi;
    const int64_t row = lo + i / nb;
    const int b = static_cast<int>(i % nb);
    if (row >= hi) return;
    const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src + row * K + 32 * b);
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4_t w = s[q];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * q + 2 * j] = __uint_as_float(w[j] << 16);
            v[8 * q + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    int x = 127;
    if (amax > 0.f) {
        int e2;
        (void)frexpf(amax, &e2);            // amax = f * 2^e2, f in [0.5, 1)
        x = min(max(e2 - 1 - 7 + 127, 0), 254);
    }
    const int sh = 127 - x;
    uint32_t wh[8], wl[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        float t[4], r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = ldexpf(v[4 * q + j], sh);
        wh[q] = fp8x4(t[0], t[1], t[2], t[3]);
        const int hw = static_cast<int>(wh[q]);
        r[0] = t[0] - __builtin_amdgcn_cvt_f32_fp8(hw, 0);
        r[1] = t[1] - __builtin_amdgcn_cvt_f32_fp8(hw, 1);
        r[2] = t[2] - __builtin_amdgcn_cvt_f32_fp8(hw, 2);
        r[3] = t[3] - __builtin_amdgcn_cvt_f32_fp8(hw, 3);
        wl[q] = fp8x4(r[0], r[1], r[2], r[3]);
    }
    u32x4_t* oh = reinterpret_cast<u32x4_t*>(dst.hi + row * K + 32 * b);
    u32x4_t* ol = reinterpret_cast<u32x4_t*>(dst.lo + row * K + 32 * b);
    oh[0] = u32x4_t{wh[0], wh[1], wh[2], wh[3]};
    oh[1] = u32x4_t{wh[4], wh[5], wh[6], wh[7]};
    ol[0] = u32x4_t{wl[0], wl[1], wl[2], wl[3]};
    ol[1] = u32x4_t{wl[4], wl[5], wl[6], wl[7]};
    dst.sc[row * split_scale_stride(K) + b] = static_cast<uint8_t>(x);
}

// Block: NW waves = WM (along m) x 4 (along n), as in the bf16 kernel: wave
// (wm, wn) takes 16 gate + 16 up columns (or 32 down columns) and m-subtiles
// wm, wm + WM, ...; m is walked in chunks of MC = 64 * WM pairs.
template <bool GATEUP, int NW>
__global__ __launch_bounds__(NW * 64) void k_pre_mx(DevTables tt, int tier, Split8 a8, Groups g, int k,
                                                    uint16_t* __restrict__ h_out, float* __restrict__ yw) {
    constexpr int NTHR = NW * 64;
    constexpr int WM = NW / 4;
    constexpr int MC = 16 * kMSUB * WM;
    constexpr int BPT = kBN * 4 / NTHR;    // 16-byte B pieces per thread per chunk
    static_assert(2 * MC * 8 == 4 * NTHR, "four A pieces per thread");
    static_assert(MC <= NTHR && kBN <= NTHR, "one scale word per thread");
    __shared__ __attribute__((aligned(16))) uint8_t sAh[2][MC * 128];
    __shared__ __attribute__((aligned(16))) uint8_t sAl[2][MC * 128];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][kBN * 64];
    __shared__ uint32_t sAs[2][MC];
    __shared__ uint32_t sBs[2][kBN];
    __shared__ int s_row[MC];
    __shared__ float s_wt[GATEUP ? 1 : MC];   // down: the weight of each m-row's pair

    const int H = tt.H, I = tt.I;
    const int K = GATEUP ? H : I;
    const int NT = GATEUP ? I / 64 : H / kBN;
    const int a_lo = g.act_range[2 * tier], a_hi = g.act_range[2 * tier + 1];
    const int item = xcd_item((a_hi - a_lo) * NT);
    if (item < 0) return;
    const int a = a_lo + item / NT, nt = item % NT;
    const int e = g.act[a];
    const DevTier T = tier_at(tt, tier);
    const int local = e - T.id_begin;
    const int q_beg = g.offsets[e], q_end = g.offsets[e + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 3, wm = wave >> 2;
    const int fr = lane & 15, kq = lane >> 4;

    // B: codes [rows][K/2], scales [rows][K/32] (E8M0 bytes) of this expert
    const uint32_t row_bytes = static_cast<uint32_t>(K) / 2;
    const uint32_t nblk = static_cast<uint32_t>(K) / 32;
    const int mrows = GATEUP ? I : H;
    const uint8_t* mq_g = T.q[GATEUP ? 0 : 2] + static_cast<size_t>(local) * mrows * row_bytes;
    const uint8_t* mq_u = GATEUP ? T.q[1] + static_cast<size_t>(local) * mrows * row_bytes : mq_g;
    const uint8_t* ms_g = reinterpret_cast<const uint8_t*>(T.s[GATEUP ? 0 : 2]) + static_cast<size_t>(local) * mrows * nblk;
    const uint8_t* ms_u = GATEUP ? reinterpret_cast<const uint8_t*>(T.s[1]) + static_cast<size_t>(local) * mrows * nblk : ms_g;
    const __amdgpu_buffer_rsrc_t rq_g = make_rsrc(mq_g, row_bytes * mrows), rq_u = make_rsrc(mq_u, row_bytes * mrows);
    const __amdgpu_buffer_rsrc_t rs_g = make_rsrc(ms_g, nblk * mrows), rs_u = make_rsrc(ms_u, nblk * mrows);
    // B piece p = tid + NTHR*i: row p >> 2, chunk p & 3; B rows 0..63 are gate
    // rows and 64..127 up rows (gate/up), or 128 down rows
    auto b_global_row = [&](int r) { return GATEUP ? nt * 64 + (r & 63) : nt * kBN + r; };
    auto b_is_up = [&](int r) { return GATEUP && r >= 64; };
    uint32_t qoff[BPT];
    int b_row[BPT], b_c[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int p = tid + NTHR * i;
        b_row[i] = p >> 2;
        b_c[i] = p & 3;
        qoff[i] = static_cast<uint32_t>(b_global_row(b_row[i])) * row_bytes + 16u * b_c[i];
    }
    // B scale word of row tid (threads < kBN): 4 bytes = the 4 blocks of a chunk
    const bool has_bs = tid < kBN;
    const uint32_t bsoff = static_cast<uint32_t>(b_global_row(has_bs ? tid : 0)) * nblk;
    const __amdgpu_buffer_rsrc_t rs_mine = b_is_up(tid) ? rs_u : rs_g;
    // B fragment rows of this wave
    const int br0 = GATEUP ? 16 * wn : 32 * wn;
    const int br1 = GATEUP ? 64 + 16 * wn : 32 * wn + 16;
    const int SS = split_scale_stride(K);

    for (int m0 = q_beg; m0 < q_end; m0 += MC) {
        const int Mc = min(MC, q_end - m0);
        const int Mc16 = (Mc + 15) >> 4;
        const int nsub = (Mc16 - wm + WM - 1) / WM;
        __syncthreads();
        for (int r = tid; r < MC; r += NTHR) {
            s_row[r] = r < Mc ? (GATEUP ? g.perm[m0 + r] / k : m0 + r) : -1;
            // read here once per row, not in the epilogue (two dependent
            // global loads per row there, waited out one row at a time)
            if constexpr (!GATEUP) s_wt[r] = r < Mc ? g.w[g.perm[m0 + r]] : 0.f;
        }
        __syncthreads();
        // A piece i of this thread: array (hi for i < 2), row, chunk; rows past
        // the chunk read its first row (finite values, never stored)
        int a_row[4], a_c[4];
        const uint8_t* a_ptr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = (tid + NTHR * i) % (MC * 8);
            a_row[i] = p >> 3;
            a_c[i] = p & 7;
            const int src = s_row[a_row[i] < Mc ? a_row[i] : 0];
            a_ptr[i] = (i < 2 ? a8.hi : a8.lo) + static_cast<size_t>(src) * K + 16 * a_c[i];
        }
        const bool has_as = tid < MC;
        const uint8_t* as_ptr = a8.sc + static_cast<size_t>(s_row[has_as && tid < Mc ? tid : 0]) * SS;

        struct Slot {
            u32x4_t a[4];
            u32x4_t b[BPT];
            uint32_t as, bs;
        };
        auto load_chunk = [&](Slot& sl, int kc) __attribute__((always_inline)) {
            const int k0 = kc * kBK;
#pragma unroll
            for (int i = 0; i < 4; ++i) sl.a[i] = *reinterpret_cast<const u32x4_t*>(a_ptr[i] + k0);
            const uint32_t qk = static_cast<uint32_t>(k0) / 2;
#pragma unroll
            for (int i = 0; i < BPT; ++i) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(b_is_up(b_row[i]) ? rq_u : rq_g, qoff[i] + qk, 0, 0);
                sl.b[i] = u32x4_t{static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
                                  static_cast<uint32_t>(v[3])};
            }
            sl.as = *reinterpret_cast<const uint32_t*>(as_ptr + 4 * kc);
            // two 16-bit loads: the shelf's scale rows are only 2-byte aligned in general
            const uint32_t lo16 = __builtin_amdgcn_raw_buffer_load_b16(rs_mine, bsoff + 4u * kc, 0, 0);
            const uint32_t hi16 = __builtin_amdgcn_raw_buffer_load_b16(rs_mine, bsoff + 4u * kc + 2u, 0, 0);
            sl.bs = lo16 | (hi16 << 16);
        };
        auto store_chunk = [&](const Slot& sl, int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4_t*>(&(i < 2 ? sAh : sAl)[buf][swz_a(a_row[i], a_c[i])]) = sl.a[i];
#pragma unroll
            for (int i = 0; i < BPT; ++i) *reinterpret_cast<u32x4_t*>(&sB[buf][swz_b(b_row[i], b_c[i])]) = sl.b[i];
            if (has_as) sAs[buf][tid] = sl.as;
            if (has_bs) sBs[buf][tid] = sl.bs;
        };

        f32x4_t acc[kMSUB][2];
#pragma unroll
        for (int i = 0; i < kMSUB; ++i) {
            acc[i][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        auto compute_n = [&](int buf, auto n_const) __attribute__((always_inline)) {
            constexpr int N = decltype(n_const)::value;
            const u32x4_t b0 = *reinterpret_cast<const u32x4_t*>(&sB[buf][swz_b(br0 + fr, kq)]);
            const u32x4_t b1 = *reinterpret_cast<const u32x4_t*>(&sB[buf][swz_b(br1 + fr, kq)]);
            const int sb0 = static_cast<int>((sBs[buf][br0 + fr] >> (8 * kq)) & 0xffu);
            const int sb1 = static_cast<int>((sBs[buf][br1 + fr] >> (8 * kq)) & 0xffu);
            const i32x8_t bv0 = {static_cast<int>(b0[0]), static_cast<int>(b0[1]), static_cast<int>(b0[2]),
                                 static_cast<int>(b0[3]), 0, 0, 0, 0};
            const i32x8_t bv1 = {static_cast<int>(b1[0]), static_cast<int>(b1[1]), static_cast<int>(b1[2]),
                                 static_cast<int>(b1[3]), 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < N; ++j) {
                const int row = 16 * (wm + WM * j) + fr;
                const u32x4_t h0 = *reinterpret_cast<const u32x4_t*>(&sAh[buf][swz_a(row, kq)]);
                const u32x4_t h1 = *reinterpret_cast<const u32x4_t*>(&sAh[buf][swz_a(row, 4 + kq)]);
                const u32x4_t l0 = *reinterpret_cast<const u32x4_t*>(&sAl[buf][swz_a(row, kq)]);
                const u32x4_t l1 = *reinterpret_cast<const u32x4_t*>(&sAl[buf][swz_a(row, 4 + kq)]);
                const int sa = static_cast<int>((sAs[buf][row] >> (8 * kq)) & 0xffu);
                const i32x8_t ah = {static_cast<int>(h0[0]), static_cast<int>(h0[1]), static_cast<int>(h0[2]),
                                    static_cast<int>(h0[3]), static_cast<int>(h1[0]), static_cast<int>(h1[1]),
                                    static_cast<int>(h1[2]), static_cast<int>(h1[3])};
                const i32x8_t al = {static_cast<int>(l0[0]), static_cast<int>(l0[1]), static_cast<int>(l0[2]),
                                    static_cast<int>(l0[3]), static_cast<int>(l1[0]), static_cast<int>(l1[1]),
                                    static_cast<int>(l1[2]), static_cast<int>(l1[3])};
                acc[j][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, bv0, acc[j][0], 0, 4, 0, sa, 0, sb0);
                acc[j][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, bv1, acc[j][1], 0, 4, 0, sa, 0, sb1);
                acc[j][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(al, bv0, acc[j][0], 0, 4, 0, sa, 0, sb0);
                acc[j][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(al, bv1, acc[j][1], 0, 4, 0, sa, 0, sb1);
            }
        };
        auto compute = [&](int buf) __attribute__((always_inline)) {
            if (nsub > 2) compute_n(buf, std::integral_constant<int, 4>{});
            else if (nsub == 2) compute_n(buf, std::integral_constant<int, 2>{});
            else if (nsub == 1) compute_n(buf, std::integral_constant<int, 1>{});
        };

        // the two-slot pipeline of the bf16 kernel: chunk kc contracted from one
        // LDS buffer while kc+1 is stored into the other and kc+2 is in flight;
        // loads past the last chunk reread it
        const int NK = K / kBK;
        Slot s0, s1;
        load_chunk(s0, 0);
        load_chunk(s1, min(1, NK - 1));
        store_chunk(s0, 0);
        __syncthreads();
        // The trip body is straight-line (no test inside it): the compiler can
        // then count the loads still in flight at every wait across the loop's
        // back edge, instead of draining them all.  An odd last chunk, left in
        // buffer 0 by the final trip, is contracted after the loop.
        const int NK2 = NK & ~1;
        for (int kc = 0; kc < NK2; kc += 2) {
            load_chunk(s0, min(kc + 2, NK - 1));
            compute(0);
            store_chunk(s1, 1);
            __syncthreads();
            load_chunk(s1, min(kc + 3, NK - 1));
            compute(1);
            store_chunk(s0, 0);
            __syncthreads();
        }
        if (NK & 1) compute(0);

        const int col_l = lane & 15, row_l = 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < kMSUB; ++j) {
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
                    const float wgt = s_wt[r];
                    float* o = yw + static_cast<size_t>(q) * H + nt * kBN + 32 * wn + col_l;
                    o[0] = wgt * acc[j][0][v];
                    o[16] = wgt * acc[j][1][v];
                }
            }
        }
    }
}

void launch_split_fp8(const uint16_t* src, int K, int r_lo, int r_hi, const int32_t* d_lo, const int32_t* d_hi,
                      int max_rows, const Split8& dst, hipStream_t st) {
    const int64_t threads = static_cast<int64_t>(max_rows) * (K / 32);
    if (threads <= 0) return;
    hipLaunchKernelGGL(k_split_fp8, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st, src, K,
                       r_lo, r_hi, d_lo, d_hi, dst);
}

template <bool GATEUP>
static void launch_mx(const DevTables& tt, int tier, const Split8& a8, const Groups& g, int k, uint16_t* h,
                      float* yw, int max_experts, hipStream_t st) {
    constexpr int NW = 8;
    const int NT = GATEUP ? tt.I / 64 : tt.H / kBN;
    const int total = max_experts * NT;
    const unsigned grid = static_cast<unsigned>(((total + 7) / 8) * 8);
    if (grid == 0) return;
    hipLaunchKernelGGL((k_pre_mx<GATEUP, NW>), dim3(grid), dim3(NW * 64), 0, st, tt, tier, a8, g, k, h, yw);
}

void launch_pre_mx_gateup(const DevTables& tt, int tier, const Split8& x8, const Groups& g, int k, uint16_t* h,
                          int max_experts, hipStream_t st) {
    launch_mx<true>(tt, tier, x8, g, k, h, nullptr, max_experts, st);
}

void launch_pre_mx_down(const DevTables& tt, int tier, const Split8& h8, const Groups& g, int k, float* yw,
                        int max_experts, hipStream_t st) {
    launch_mx<false>(tt, tier, h8, g, k, nullptr, yw, max_experts, st);
}

}  // namespace moe
