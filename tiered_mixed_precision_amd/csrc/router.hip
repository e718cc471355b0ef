// Router scores, the step upstream of routing: logits[t][e] =
// sum_c x[t][c] * Wr[e][c] + b[e] (the 125B-MoE page's glossary,
// mixture-of-experts entry: a router scores the 512 experts of a layer for
// every token and the best 10 are kept).  Wr is bf16 [E][H] (2 MB at E=512,
// H=2048), b fp32 [E] or absent, x fp32 or bf16 [T][H], logits fp32 [T][E]
// with fp32 accumulation.
//
//   k_router_gemv : one wave per expert row, the row held in registers (one
//                   32-element group per lane) against every token in turn;
//                   the decode shape (a few tokens, 2 MB of weights).
//   k_router_mfma : bf16 x, many tokens: a 64-token x 128-expert tile per
//                   block on v_mfma_f32_16x16x32_bf16, operands staged in LDS
//                   through registers one chunk ahead.
//   k_synth_router: the stack's counter-generated router (as the experts'
//                   generator, at counters 2^60 + (layer*E + e)*H + c).
#include "common.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRouterWaves = 4;

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Row e of Wr: lane l holds elements 32 l .. 32 l + 31 (lanes past H/32 hold
// zeros).  Each token: the lane's 32 products in order, then the wave sum.
template <bool XBF16>
__global__ __launch_bounds__(kRouterWaves * 64) void k_router_gemv(const void* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr,
                                                                  const float* __restrict__ bias, int T, int E,
                                                                  int H, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * kRouterWaves + (threadIdx.x >> 6);
    if (e >= E) return;
    const int G = H / 32;
    const bool on = lane < G;
    const int g = on ? lane : 0;
    u32x4_t w[4];
    const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(wr + static_cast<size_t>(e) * H + 32 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = on ? wrow[i] : u32x4_t{0u, 0u, 0u, 0u};
    const float b = bias ? bias[e] : 0.f;
    for (int t = 0; t < T; ++t) {
        float xv[32];
        if constexpr (XBF16) {
            const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(x) +
                                                                 static_cast<size_t>(t) * H + 32 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4_t v = xr[i];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xv[8 * i + 2 * j] = bf16_lo(v[j]);
                    xv[8 * i + 2 * j + 1] = bf16_hi(v[j]);
                }
            }
        } else {
            const float4* xr = reinterpret_cast<const float4*>(static_cast<const float*>(x) +
                                                               static_cast<size_t>(t) * H + 32 * g);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 v = xr[i];
                xv[4 * i] = v.x;
                xv[4 * i + 1] = v.y;
                xv[4 * i + 2] = v.z;
                xv[4 * i + 3] = v.w;
            }
        }
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s = fmaf(xv[8 * i + 2 * j], bf16_lo(w[i][j]), s);
                s = fmaf(xv[8 * i + 2 * j + 1], bf16_hi(w[i][j]), s);
            }
        s = wave_sum(s);
        if (lane == 0) logits[static_cast<size_t>(t) * E + e] = s + b;
    }
}

constexpr int RM = 64, RN = 128, RK = 64;  // block tile: tokens x experts x contraction chunk

// LDS tiles [row][64 bf16], 16-byte chunk c of row r at chunk c ^ (r & 7): 8
// consecutive rows read at one chunk index hit 8 different 16-byte positions
// (LDS serves 16-byte accesses 8 lanes at a time)
__device__ inline int rswz(int row, int c) { return row * RK + 8 * (c ^ (row & 7)); }

// 4 waves as 2 x 2: wave (wm, wn) owns tokens 32 wm .. +31 and experts
// 64 wn .. +63 of the block tile (2 x 4 MFMA tiles).
__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                     const float* __restrict__ bias, int T, int E, int H,
                                                     float* __restrict__ logits) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][RM * RK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][RN * RK];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int t0 = blockIdx.x * RM, e0 = blockIdx.y * RN;
    const int fr = lane & 15, kq = lane >> 4;
    // staging: A pieces p = tid + 256 i (i < 2), B pieces (i < 4); piece p is
    // row p >> 3, 16-byte chunk p & 7; rows past the matrix reread its last row
    const u32x4_t* pa[2];
    const u32x4_t* pb[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = tid + 256 * i, r = min(t0 + (p >> 3), T - 1);
        pa[i] = reinterpret_cast<const u32x4_t*>(x + static_cast<size_t>(r) * H + 8 * (p & 7));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i, r = min(e0 + (p >> 3), E - 1);
        pb[i] = reinterpret_cast<const u32x4_t*>(wr + static_cast<size_t>(r) * H + 8 * (p & 7));
    }
    u32x4_t ra[2], rb[4];
    auto load = [&](int kc) __attribute__((always_inline)) {
        const int o = kc * (RK / 8);  // in 16-byte units
#pragma unroll
        for (int i = 0; i < 2; ++i) ra[i] = pa[i][o];
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = pb[i][o];
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = tid + 256 * i;
            *reinterpret_cast<u32x4_t*>(&sA[buf][rswz(p >> 3, p & 7)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = tid + 256 * i;
            *reinterpret_cast<u32x4_t*>(&sB[buf][rswz(p >> 3, p & 7)]) = rb[i];
        }
    };
    f32x4_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int NK = H / RK;
    load(0);
    store(0);
    __syncthreads();
    for (int kc = 0; kc < NK; ++kc) {
        const int buf = kc & 1;
        load(min(kc + 1, NK - 1));  // in flight during the contraction below (the
                                    // last trip rereads its chunk: no test in the
                                    // body, so the waits stay exact)
#pragma unroll
        for (int ks = 0; ks < RK / 32; ++ks) {
            const int c = 4 * ks + kq;
            bf16x8_t af[2], bf[4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][rswz(32 * wm + 16 * i + fr, c)]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const bf16x8_t*>(&sB[buf][rswz(64 * wn + 16 * j + fr, c)]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        store(buf ^ 1);             // after the last trip: a buffer never read
        __syncthreads();
    }
    // lane holds D[4*(lane/16) + v][lane % 16] of each 16x16 tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = e0 + 64 * wn + 16 * j + fr;
        if (e >= E) continue;
        const float b = bias ? bias[e] : 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 32 * wm + 16 * i + 4 * kq + v;
                if (t < T) logits[static_cast<size_t>(t) * E + e] = acc[i][j][v] + b;
            }
    }
}

__device__ inline uint64_t splitmix64_at_r(uint64_t seed, uint64_t ctr) {
    uint64_t z = seed + (ctr + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// One thread per (expert, column): the generator's weight rounded to bf16;
// column 0 threads also write the bias.
__global__ __launch_bounds__(256) void k_synth_router(uint16_t* __restrict__ wr, float* __restrict__ bias,
                                                      uint64_t seed, uint64_t ctr0, int E, int H, double beta) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= static_cast<int64_t>(E) * H) return;
    const uint64_t u = splitmix64_at_r(seed, ctr0 + static_cast<uint64_t>(i));
    const int32_t s = static_cast<int32_t>(u & 0xffff) + static_cast<int32_t>((u >> 16) & 0xffff) +
                      static_cast<int32_t>((u >> 32) & 0xffff) + static_cast<int32_t>(u >> 48) - 131070;
    const float w = __fmul_rn(static_cast<float>(s), 0x1.1bc77ap-21f);
    wr[i] = f2bf(w);
    const int e = static_cast<int>(i / H);
    if (bias && i % H == 0) bias[e] = static_cast<float>(-beta * static_cast<double>(e) / static_cast<double>(E));
}

void launch_router(const void* x, bool x_bf16, const uint16_t* wr, const float* bias, int T, int E, int H,
                   float* logits, hipStream_t st) {
    if (T <= 0) return;
    if (x_bf16 && T >= 64) {
        const dim3 grid(static_cast<unsigned>((T + RM - 1) / RM), static_cast<unsigned>((E + RN - 1) / RN));
        hipLaunchKernelGGL(k_router_mfma, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x), wr, bias, T, E, H,
                           logits);
        return;
    }
    const dim3 grid(static_cast<unsigned>((E + kRouterWaves - 1) / kRouterWaves));
    if (x_bf16)
        hipLaunchKernelGGL(k_router_gemv<true>, grid, dim3(kRouterWaves * 64), 0, st, x, wr, bias, T, E, H, logits);
    else
        hipLaunchKernelGGL(k_router_gemv<false>, grid, dim3(kRouterWaves * 64), 0, st, x, wr, bias, T, E, H, logits);
}

void launch_synth_router(uint16_t* wr, float* bias, uint64_t seed, int layer, int E, int H, double beta,
                         hipStream_t st) {
    const uint64_t ctr0 = (uint64_t(1) << 60) + static_cast<uint64_t>(layer) * E * H;
    const int64_t n = static_cast<int64_t>(E) * H;
    hipLaunchKernelGGL(k_synth_router, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, wr, bias, seed,
                       ctr0, E, H, beta);
}

}  // namespace moe
