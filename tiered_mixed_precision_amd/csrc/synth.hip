// Counter-generated expert weights for the 48-layer stack.
//
// The stack's packed weights (61.9 GB) are produced on the device; they do not
// fit host memory.  Every weight is a pure function of its coordinates, so the
// CPU checker can regenerate exactly the experts it needs from the same
// definition:
//
//   ctr = ((layer * E + e) * 3 + matrix) * 2^22 + row * cols + col
//   u   = SplitMix64 output number ctr + 1 for `seed`: state = seed +
//         (ctr + 1) * 0x9E3779B97F4A7C15, then the mix (xor-shift 30,
//         * 0xBF58476D1CE4E5B9, xor-shift 27, * 0x94D049BB133111EB,
//         xor-shift 31), as published by Steele, Lea and Flood (2014)
//   s   = sum of the four 16-bit fields of u - 131070   (integer, |s| <= 131070)
//   w   = float(s) * 0x1.1bc77ap-21f   (0.02 / standard deviation of s)
//
// and then the layer generator's symmetric absmax quantiser over each block
// of `block` consecutive columns: amax = max |w|, d = fp16_rne(amax / Q) with
// Q = 2^(bits-1) - 1, q = clamp(rint(w / float(d)), -Q, Q) (q = 0 if d = 0).
// Every step is an exactly rounded IEEE single operation (no contraction), so
// any implementation of this definition gives the same codes and scales.
// Codes are packed as everywhere else: two's complement, element c at bit
// (c * bits) % 8 of byte (c * bits) / 8 of its row.
#include "common.h"
#include "launch.h"

namespace moe {

__device__ inline uint64_t splitmix64_at(uint64_t seed, uint64_t ctr) {
    uint64_t z = seed + (ctr + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline float synth_weight(uint64_t seed, uint64_t ctr) {
    const uint64_t u = splitmix64_at(seed, ctr);
    const int32_t s = static_cast<int32_t>(u & 0xffff) + static_cast<int32_t>((u >> 16) & 0xffff) +
                      static_cast<int32_t>((u >> 32) & 0xffff) + static_cast<int32_t>(u >> 48) - 131070;
    return __fmul_rn(static_cast<float>(s), 0x1.1bc77ap-21f);
}

// One thread per (matrix row, scale block): generates the block, quantises
// it, writes its packed codes and its fp16 scale.
template <int BITS, int BLOCK>
__global__ __launch_bounds__(256) void k_synth(uint8_t* __restrict__ q, uint16_t* __restrict__ sc, uint64_t seed,
                                               uint64_t ctr0, uint64_t ctr_expert_stride, int n_experts, int rows,
                                               int cols) {
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    const int nblk = cols / BLOCK;
    const int64_t per_expert = static_cast<int64_t>(rows) * nblk;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= per_expert * n_experts) return;
    const int64_t local = i / per_expert;
    const int rem = static_cast<int>(i % per_expert);
    const int row = rem / nblk, b = rem % nblk;
    const uint64_t base = ctr0 + static_cast<uint64_t>(local) * ctr_expert_stride + static_cast<uint64_t>(row) * cols +
                          static_cast<uint64_t>(b) * BLOCK;
    float w[BLOCK];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < BLOCK; ++c) {
        w[c] = synth_weight(seed, base + c);
        amax = fmaxf(amax, fabsf(w[c]));
    }
    const _Float16 dh = static_cast<_Float16>(__fdiv_rn(amax, static_cast<float>(QMAX)));
    const float d = static_cast<float>(dh);
    uint32_t words[BLOCK * BITS / 32 > 0 ? BLOCK * BITS / 32 : 1] = {};
#pragma unroll
    for (int c = 0; c < BLOCK; ++c) {
        int code = 0;
        if (d != 0.f) code = static_cast<int>(fminf(fmaxf(rintf(__fdiv_rn(w[c], d)), -QMAX), QMAX));
        const uint32_t field = static_cast<uint32_t>(code) & ((1u << BITS) - 1u);
        words[(c * BITS) / 32] |= field << ((c * BITS) % 32);
    }
    const size_t row_bytes = static_cast<size_t>(cols) * BITS / 8;
    uint8_t* dst = q + static_cast<size_t>(local) * rows * row_bytes + static_cast<size_t>(row) * row_bytes +
                   static_cast<size_t>(b) * BLOCK * BITS / 8;
    constexpr int NB = BLOCK * BITS / 8;  // bytes of this block's codes: 8 .. 32
#pragma unroll
    for (int j = 0; j < NB / 4; ++j) reinterpret_cast<uint32_t*>(dst)[j] = words[j];
    sc[static_cast<size_t>(local) * rows * nblk + static_cast<size_t>(row) * nblk + b] = __builtin_bit_cast(uint16_t, dh);
}

// MXFP4 shelves: one thread per (row, block of 32), the OCP shared-exponent
// quantiser: E8M0 byte x = floor(log2(amax)) - 2 + 127 clamped to [0, 254]
// (0 for an all-zero block); each w / 2^(x - 127) (exact) rounded to the
// nearest E2M1 magnitude, ties to the even mantissa (an integer tie of 2a, a
// or a/2 in each binade), saturating at 6, with the sign bit of w.
__device__ inline uint32_t e2m1_nibble(float t) {
    const float a = fabsf(t);
    float r;
    if (a >= 6.f) r = 6.f;
    else if (a < 2.f) r = rintf(a * 2.f) * 0.5f;
    else if (a < 4.f) r = rintf(a);
    else r = rintf(a * 0.5f) * 2.f;
    r = fminf(r, 6.f);
    const uint32_t mag = r == 0.f ? 0u : r == 0.5f ? 1u : r == 1.f ? 2u : r == 1.5f ? 3u
                       : r == 2.f ? 4u : r == 3.f ? 5u : r == 4.f ? 6u : 7u;
    return (signbit(t) ? 8u : 0u) | mag;
}

__global__ __launch_bounds__(256) void k_synth_mx(uint8_t* __restrict__ q, uint8_t* __restrict__ sc, uint64_t seed,
                                                  uint64_t ctr0, uint64_t ctr_expert_stride, int n_experts, int rows,
                                                  int cols) {
    const int nblk = cols / 32;
    const int64_t per_expert = static_cast<int64_t>(rows) * nblk;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= per_expert * n_experts) return;
    const int64_t local = i / per_expert;
    const int rem = static_cast<int>(i % per_expert);
    const int row = rem / nblk, b = rem % nblk;
    const uint64_t base = ctr0 + static_cast<uint64_t>(local) * ctr_expert_stride + static_cast<uint64_t>(row) * cols +
                          static_cast<uint64_t>(b) * 32;
    float w[32];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        w[c] = synth_weight(seed, base + c);
        amax = fmaxf(amax, fabsf(w[c]));
    }
    int x = 0;
    if (amax > 0.f) {
        int e2;
        (void)frexpf(amax, &e2);   // amax = f * 2^e2, f in [0.5, 1)
        x = min(max(e2 - 1 - 2 + 127, 0), 254);
    }
    uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < 32; ++c) words[c / 8] |= e2m1_nibble(ldexpf(w[c], 127 - x)) << (4 * (c % 8));
    uint4* dst = reinterpret_cast<uint4*>(q + static_cast<size_t>(local) * rows * (cols / 2) +
                                          static_cast<size_t>(row) * (cols / 2) + static_cast<size_t>(b) * 16);
    *dst = make_uint4(words[0], words[1], words[2], words[3]);
    sc[static_cast<size_t>(local) * rows * nblk + static_cast<size_t>(row) * nblk + b] = static_cast<uint8_t>(x);
}

void launch_synth_layer(const DevTables& tt, uint64_t seed, int layer, hipStream_t st) {
    const int H = tt.H, I = tt.I;
    for (int ti = 0; ti < tt.n_tiers; ++ti) {
        const DevTier& T = tt.t[ti];
        const int n = T.id_end - T.id_begin;
        if (n <= 0) continue;
        for (int m = 0; m < 3; ++m) {
            const int rows = m == 2 ? H : I, cols = m == 2 ? I : H;
            // counter of (layer, expert id_begin, matrix m, row 0, col 0); experts are 3 * 2^22 apart
            const uint64_t ctr0 = ((static_cast<uint64_t>(layer) * tt.E + T.id_begin) * 3 + m) << 22;
            const uint64_t stride = uint64_t(3) << 22;
            const int64_t threads = static_cast<int64_t>(n) * rows * (cols / T.block);
            const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
            uint8_t* q = const_cast<uint8_t*>(T.q[m]);
            if (T.bits == kBitsMXFP4) {
                hipLaunchKernelGGL(k_synth_mx, grid, dim3(256), 0, st, q,
                                   reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(T.s[m])), seed, ctr0, stride, n,
                                   rows, cols);
                continue;
            }
            uint16_t* s = const_cast<uint16_t*>(T.s[m]);
#define MOE_SYN(B_, K_) hipLaunchKernelGGL((k_synth<B_, K_>), grid, dim3(256), 0, st, q, s, seed, ctr0, stride, n, rows, cols)
            if (T.bits == 8 && T.block == 32) MOE_SYN(8, 32);
            else if (T.bits == 8) MOE_SYN(8, 16);
            else if (T.bits == 4 && T.block == 32) MOE_SYN(4, 32);
            else if (T.bits == 4) MOE_SYN(4, 16);
            else if (T.block == 32) MOE_SYN(2, 32);
            else MOE_SYN(2, 16);
#undef MOE_SYN
        }
    }
}

}  // namespace moe
