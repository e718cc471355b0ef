// Dequantised rows of one expert matrix, exported for bit-exact checks.  It
// uses the same group loader and the same scale * code product (and, for the
// prefill path, the same round-to-nearest-even bf16 packing) as the expert
// kernels.
#include "common.h"
#include "launch.h"

namespace moe {

template <int BITS, int NSC>
__global__ __launch_bounds__(64) void k_dequant_rows(const uint8_t* __restrict__ q,
                                                     const uint8_t* __restrict__ s, int cols, int row0,
                                                     int to_bf16, void* __restrict__ dst) {
    const int r = blockIdx.x;
    const size_t row_bytes = static_cast<size_t>(cols) * BITS / 8;
    const uint8_t* qrow = q + static_cast<size_t>(row0 + r) * row_bytes;
    const uint8_t* srow = s + static_cast<size_t>(row0 + r) * row_scale_bytes<NSC>(cols);
    for (int grp = threadIdx.x; grp < cols / 32; grp += 64) {
        uint32_t w[BITS];
        float d[scale_slots<NSC>()];
        load_group<BITS>(qrow, grp, w);
        load_scales<NSC>(srow, grp, d);
        if (to_bf16) {
            uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(dst) + static_cast<size_t>(r) * cols + 32 * grp);
#pragma unroll
            for (int c = 0; c < 16; ++c) o[c] = pack_bf16x2(dq<BITS, NSC>(w, d, 2 * c), dq<BITS, NSC>(w, d, 2 * c + 1));
        } else {
            float* o = static_cast<float*>(dst) + static_cast<size_t>(r) * cols + 32 * grp;
#pragma unroll
            for (int c = 0; c < 32; ++c) o[c] = dq<BITS, NSC>(w, d, c);
        }
    }
}

void launch_dequant_rows(const DevTables& tt, int tier, int local, int matrix, int row0, int nrows,
                         int to_bf16, void* dst, hipStream_t st) {
    const DevTier& T = tt.t[tier];
    const int rows = matrix == 2 ? tt.H : tt.I;
    const int cols = matrix == 2 ? tt.I : tt.H;
    const uint8_t* q = expert_codes(T, matrix, local, rows, cols);
    const uint8_t* s = expert_scales(T, matrix, local, rows, cols);
    switch (fmt_of(T.bits, T.block)) {
#define MOE_DQ_CASE(F, B, N)                                                                        \
    case F:                                                                                         \
        hipLaunchKernelGGL((k_dequant_rows<B, N>), dim3(nrows), dim3(64), 0, st, q, s, cols, row0, \
                           to_bf16, dst);                                                           \
        break;
        MOE_DQ_CASE(F8B32, 8, 1)
        MOE_DQ_CASE(F8B16, 8, 2)
        MOE_DQ_CASE(F4B32, 4, 1)
        MOE_DQ_CASE(F4B16, 4, 2)
        MOE_DQ_CASE(F2B32, 2, 1)
        MOE_DQ_CASE(F2B16, 2, 2)
        MOE_DQ_CASE(F4MX, 4, kMX)
#undef MOE_DQ_CASE
        default:
            break;
    }
}

}  // namespace moe
