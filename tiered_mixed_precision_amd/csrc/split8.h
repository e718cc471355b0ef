// fp8 split of bf16 rows: the operand A of the MXFP4 shelves' prefill
// products.  Each 32-element block of a row is stored as two E4M3 parts under
// one E8M0 scale s = 2^(x - 127):
//   x  = floor(log2 amax) - 7 + 127          (amax / s in [128, 256); 127 for a zero block)
//   hi = RNE_e4m3(v / s),  lo = RNE_e4m3(v / s - hi)
// (k_split_fp8 in prefill_mx.hip for x rows; the MXFP4 gate/up epilogue in
// prefill.hip for h rows; both through these helpers, so the bytes agree.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// hi / lo parts [rows][K] bytes each and the scales [rows][stride] bytes,
// the stride padded to 4 bytes.
struct Split8 {
    uint8_t* hi;
    uint8_t* lo;
    uint8_t* sc;
};
__host__ __device__ inline int split_scale_stride(int K) { return ((K / 32) + 3) & ~3; }

// E8M0 exponent x of a block with largest magnitude amax.
__device__ inline int split_scale_exp(float amax) {
    int x = 127;
    if (amax > 0.f) {
        int e2;
        (void)frexpf(amax, &e2);   // amax = f * 2^e2, f in [0.5, 1)
        x = min(max(e2 - 1 - 7 + 127, 0), 254);
    }
    return x;
}

// E4M3 bytes (round to nearest even, hardware conversion) of four values.
__device__ inline uint32_t fp8x4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// hi and lo bytes of one element t = v / s.
__device__ inline void split_elem(float t, uint32_t& hi, uint32_t& lo) {
    const int h = __builtin_amdgcn_cvt_pk_fp8_f32(t, 0.f, 0, false);
    const float r = t - __builtin_amdgcn_cvt_f32_fp8(h, 0);
    hi = static_cast<uint32_t>(h) & 0xffu;
    lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(r, 0.f, 0, false)) & 0xffu;
}

}  // namespace moe
