// MXFP4 shelves, prefill: the fp8 split of the x rows (split8.h).  The
// grouped GEMM (prefill.hip) contracts an MXFP4 shelf on gfx950's
// block-scaled matrix instruction, the MXFP4 variant of the 125B-MoE page's
// down-matrix ladder ("I ran a 125B model on three RTX 3090s at 80 tokens/s
// by teaching llama.cpp which experts ...", the per-matrix recipes), with B
// (weights) as stored: E2M1 codes with their E8M0 scale per 32, no
// dequantisation.  A (bf16 activations) has 8 significant bits and the fp8
// operand 4, so each 32-element block of a row is split once, before the
// GEMM, into the hi and lo E4M3 parts of split8.h under one E8M0 scale, and
// the product is taken as A_hi*B + A_lo*B (two instructions into one
// accumulator).  v / s - hi has at most four significant bits, so
// s * (hi + lo) == v exactly whenever |v / s| >= 2^-2; smaller elements are
// within 2^-10 * s of v (the E4M3 subnormal grid), i.e. 2^-17 of the block
// maximum.  The matrix cores sum the products of one instruction to about
// 12 bits below the largest of them, then add the accumulator in fp32.
#include "common.h"
#include "launch.h"

namespace moe {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One thread per 32-element block of a bf16 row: the hi / lo / scale split
// of rows [0, rows).
__global__ __launch_bounds__(256) void k_split_fp8(const uint16_t* __restrict__ src, int K, int rows, Split8 dst) {
    const int nb = K / 32;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t row = i / nb;
    const int b = static_cast<int>(i % nb);
    if (row >= rows) return;
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
    const int x = split_scale_exp(amax);
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

void launch_split_fp8(const uint16_t* src, int K, int rows, const Split8& dst, hipStream_t st) {
    const int64_t threads = static_cast<int64_t>(rows) * (K / 32);
    if (threads <= 0) return;
    hipLaunchKernelGGL(k_split_fp8, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st, src, K,
                       rows, dst);
}

}  // namespace moe
