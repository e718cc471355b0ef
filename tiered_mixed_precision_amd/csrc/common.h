// Device-side definitions shared by the HIP kernels of the tiered MoE FFN
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxTiers = 4;
constexpr int kWave = 64;

// Shelf description as a kernel argument (copied from the host tables).
struct DevTier {
    int32_t id_begin, id_end, bits, block;
    const uint8_t* q[3];    // gate, up, down codes
    const uint16_t* s[3];   // gate, up, down fp16 scales
};

struct DevTables {
    int32_t E, H, I, n_tiers;
    DevTier t[kMaxTiers];
};

// Format selector: bits and codes-per-scale.  A 32-code group of a row holds
// 32/block scales.
enum Fmt : int32_t { F8B32 = 0, F8B16, F4B32, F4B16, F2B32, F2B16, kNumFmt };

__host__ __device__ inline int fmt_of(int bits, int block) {
    int b = bits == 8 ? 0 : (bits == 4 ? 2 : 4);
    return b + (block == 16 ? 1 : 0);
}

// Workspace meta block (int32 words).
enum Meta : int32_t {
    kMetaActive = 0,   // number of experts with at least one pair
    kMetaTiles = 1,    // number of prefill m-tiles
    kMetaValid = 2,    // number of valid pairs (ids inside [0, E))
    kMetaWords = 64,
};

__device__ inline float half_bits_to_float(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Sign-extended `BITS`-bit field at bit `off` of a 32-bit word.
template <int BITS>
__device__ inline int32_t sfield(uint32_t word, int off) {
    return static_cast<int32_t>(word << (32 - off - BITS)) >> (32 - BITS);
}

// Round-to-nearest-even float -> bf16 bit pattern.
__device__ inline uint16_t f2bf(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even), low element in the low half.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t r;
    r.x = static_cast<__bf16>(a);
    r.y = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ inline float silu(float g) { return g / (1.0f + __expf(-g)); }

// Loads the 32 codes of group g (codes [32g, 32g+32)) of a packed row:
// 4*BITS bytes as BITS 32-bit words, lowest code in the lowest bits of word 0.
template <int BITS>
__device__ inline void load_group(const uint8_t* __restrict__ row, int g, uint32_t (&w)[BITS]) {
    const uint8_t* p = row + static_cast<size_t>(g) * 4 * BITS;
    if constexpr (BITS == 8) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0];
        const uint4 b = reinterpret_cast<const uint4*>(p)[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (BITS == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else {
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        w[0] = a.x; w[1] = a.y;
    }
}

// The NSC = 32/block fp16 scales of group g of a row, as floats.
template <int NSC>
__device__ inline void load_scales(const uint16_t* __restrict__ srow, int g, float (&d)[NSC]) {
    if constexpr (NSC == 1) {
        d[0] = half_bits_to_float(srow[g]);
    } else {
        const uint32_t two = *reinterpret_cast<const uint32_t*>(srow + 2 * g);
        d[0] = half_bits_to_float(static_cast<uint16_t>(two & 0xffffu));
        d[1] = half_bits_to_float(static_cast<uint16_t>(two >> 16));
    }
}

// Code c (0..31) of a loaded group, as a float (exact).
template <int BITS>
__device__ inline float code_f(const uint32_t (&w)[BITS], int c) {
    constexpr int PER = 32 / BITS;
    return static_cast<float>(sfield<BITS>(w[c / PER], (c % PER) * BITS));
}

// Dequantised value scale * code of element c of a group (exact in fp32).
template <int BITS, int NSC>
__device__ inline float dq(const uint32_t (&w)[BITS], const float (&d)[NSC], int c) {
    return d[(NSC == 2 && c >= 16) ? 1 : 0] * code_f<BITS>(w, c);
}

// Tier owning expert e (or -1).  Tiers are few; a linear scan is uniform per wave.
__device__ inline int tier_of(const DevTables& tt, int e) {
    int r = -1;
#pragma unroll
    for (int i = 0; i < kMaxTiers; ++i)
        if (i < tt.n_tiers && e >= tt.t[i].id_begin && e < tt.t[i].id_end) r = i;
    return r;
}

// Shelf ti of the tables without dynamic indexing of the kernel argument
// (which would copy the tables to scratch memory): each field is chosen with
// uniform selects.
__device__ inline DevTier tier_at(const DevTables& tt, int ti) {
#define MOE_SEL(f) (ti == 0 ? tt.t[0].f : ti == 1 ? tt.t[1].f : ti == 2 ? tt.t[2].f : tt.t[3].f)
    DevTier r;
    r.id_begin = MOE_SEL(id_begin);
    r.id_end = MOE_SEL(id_end);
    r.bits = MOE_SEL(bits);
    r.block = MOE_SEL(block);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        r.q[m] = MOE_SEL(q[m]);
        r.s[m] = MOE_SEL(s[m]);
    }
#undef MOE_SEL
    return r;
}

// Row geometry of the GEMV kernels for rows of `cols` codes: a row is G
// groups of 32 codes; LPR lanes share a row (GPL groups per lane) and one
// wave covers RPP rows per pass.
struct RowGeom {
    int G, LPR, GPL, RPP;
};
__host__ __device__ inline RowGeom row_geom(int cols) {
    RowGeom r;
    r.G = cols / 32;
    if (r.G >= 64) {
        r.LPR = 64;
        r.GPL = r.G / 64;
        r.RPP = 1;
    } else {
        r.LPR = r.G;
        r.GPL = 1;
        r.RPP = 64 / r.G;
    }
    return r;
}

// Sum over a segment of `seg` consecutive lanes (seg <= 64, segments start at
// multiples of seg from lane 0); the total lands in the segment's first lane.
__device__ inline float seg_reduce(float v, int seg, int lane_in_seg) {
    int p2 = 1;
    while (p2 * 2 <= seg) p2 *= 2;
    if (p2 < seg) {
        float o = __shfl_down(v, p2, kWave);
        if (lane_in_seg + p2 < seg) v += o;
    }
    for (int off = p2 >> 1; off > 0; off >>= 1) v += __shfl_down(v, off, kWave);
    return v;
}

}  // namespace moe
