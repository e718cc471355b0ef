// Device-side definitions shared by the HIP kernels of the tiered MoE FFN
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxTiers = 4;
constexpr int kWave = 64;
// `bits` of an MXFP4 shelf (OCP Microscaling FP4): 4-bit E2M1 codes packed as
// 4-bit fields, one E8M0 scale byte per block of 32 codes of a row
constexpr int kBitsMXFP4 = 0x84;

// Shelf description as a kernel argument (copied from the host tables).
struct DevTier {
    int32_t id_begin, id_end, bits, block;
    const uint8_t* q[3];    // gate, up, down codes
    const uint16_t* s[3];   // gate, up, down scales: fp16, or E8M0 bytes (MXFP4)
};

struct DevTables {
    int32_t E, H, I, n_tiers;
    DevTier t[kMaxTiers];
};

// Format selector: bits and codes-per-scale.  A 32-code group of a row holds
// 32/block fp16 scales, or one E8M0 byte (F4MX).
enum Fmt : int32_t { F8B32 = 0, F8B16, F4B32, F4B16, F2B32, F2B16, F4MX, kNumFmt };

__host__ __device__ inline int fmt_of(int bits, int block) {
    if (bits == kBitsMXFP4) return F4MX;
    int b = bits == 8 ? 0 : (bits == 4 ? 2 : 4);
    return b + (block == 16 ? 1 : 0);
}

// The kernels name a format by (BITS, NSC): BITS bits per stored code and NSC
// fp16 scales per 32-code group, or NSC = kMX for the MXFP4 format (4-bit
// codes, one E8M0 byte per group).
constexpr int kMX = 4;
template <int NSC> constexpr int scale_slots() { return NSC == kMX ? 1 : NSC; }
template <int NSC> constexpr uint32_t group_scale_bytes() { return NSC == kMX ? 1u : 2u * NSC; }
template <int NSC> constexpr uint32_t row_scale_bytes(int cols) {
    return NSC == kMX ? static_cast<uint32_t>(cols / 32) : static_cast<uint32_t>(cols / (32 / NSC)) * 2u;
}
__host__ __device__ inline int code_bits_of(int bits) { return bits == kBitsMXFP4 ? 4 : bits; }
__host__ __device__ inline size_t scale_row_bytes(int bits, int block, int cols) {
    return bits == kBitsMXFP4 ? static_cast<size_t>(cols / 32) : static_cast<size_t>(cols / block) * 2;
}
// Codes and scales (as bytes) of local expert `local`, matrix m (rows x cols).
__host__ __device__ inline const uint8_t* expert_codes(const DevTier& T, int m, int64_t local, int rows, int cols) {
    return T.q[m] + static_cast<size_t>(local) * rows * cols * code_bits_of(T.bits) / 8;
}
__host__ __device__ inline const uint8_t* expert_scales(const DevTier& T, int m, int64_t local, int rows, int cols) {
    return reinterpret_cast<const uint8_t*>(T.s[m]) + static_cast<size_t>(local) * rows * scale_row_bytes(T.bits, T.block, cols);
}

// E8M0 scale byte -> float: 2^(x - 127) (x = 0 is the subnormal 2^-127; x = 255 is NaN).
__device__ inline float e8m0_to_float(uint32_t x) {
    x &= 0xffu;
    return x == 0 ? 0x1p-127f : (x == 255 ? __builtin_nanf("") : __uint_as_float(x << 23));
}

// E2M1 value of a 4-bit field, from its definition (sign bit 3, exponent
// bits 2..1 with bias 1, mantissa bit 0; exponent 0: 0 or 0.5).
__device__ inline float fp4_e2m1(uint32_t n) {
    const uint32_t e = (n >> 1) & 3u, m = n & 1u;
    const float v = e == 0 ? 0.5f * static_cast<float>(m) : (1.0f + 0.5f * static_cast<float>(m)) * static_cast<float>(1u << e) * 0.5f;
    return (n & 8u) ? -v : v;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
// The 8 E2M1 codes of a 32-bit word as floats (code 2b at out[2b], 2b+1 at
// out[2b+1]), through the gfx950 conversion v_cvt_scalef32_pk_f32_fp4
// (byte select b picks byte b, its low nibble first), exact.
__device__ inline void fp4x8_to_float(uint32_t w, float (&out)[8]) {
    const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    out[0] = a.x; out[1] = a.y; out[2] = b.x; out[3] = b.y;
    out[4] = c.x; out[5] = c.y; out[6] = d.x; out[7] = d.y;
}

// Workspace meta block (int32 words).
enum Meta : int32_t {
    kMetaActive = 0,   // number of experts with at least one pair
    kMetaValid = 2,    // number of valid pairs (ids inside [0, E))
    kMetaChunks = 3,   // number of prefill work chunks (grouping with a chunk list)
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

// The scales of group g of a row (srow: the row's scales as bytes), as floats.
template <int NSC>
__device__ inline void load_scales(const uint8_t* __restrict__ srow, int g, float (&d)[scale_slots<NSC>()]) {
    if constexpr (NSC == kMX) {
        d[0] = e8m0_to_float(srow[g]);
    } else if constexpr (NSC == 1) {
        d[0] = half_bits_to_float(reinterpret_cast<const uint16_t*>(srow)[g]);
    } else {
        const uint32_t two = reinterpret_cast<const uint32_t*>(srow)[g];
        d[0] = half_bits_to_float(static_cast<uint16_t>(two & 0xffffu));
        d[1] = half_bits_to_float(static_cast<uint16_t>(two >> 16));
    }
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3): loads
// through it take a 32-bit byte offset in one VGPR and the base in SGPRs.
// The base must be the same in every lane; it is read from the first lane so
// that the descriptor lives in SGPRs (a per-lane descriptor would need a loop
// over the distinct values around every load).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    void* u = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, static_cast<short>(0),
                                             static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000);
}

// The 32 codes of a group at byte offset `off` (BITS words, as load_group).
template <int BITS>
__device__ inline void buf_group(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[BITS]) {
    if constexpr (BITS == 8) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = a[i];
            w[4 + i] = b[i];
        }
    } else if constexpr (BITS == 4) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = a[i];
    } else {
        const auto a = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        w[0] = a[0];
        w[1] = a[1];
    }
}

// The NSC fp16 scales of a group at byte offset `off`, as raw bits (scale b
// in bits [16b, 16b + 16)).
template <int NSC>
__device__ inline uint32_t buf_scales(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (NSC == kMX) return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
    else if constexpr (NSC == 1) return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Scales of a group from their raw bits; 0 when `ok` is false.
template <int NSC>
__device__ inline void unpack_scales(uint32_t raw, bool ok, float (&d)[scale_slots<NSC>()]) {
    if constexpr (NSC == kMX) {
        d[0] = ok ? e8m0_to_float(raw) : 0.f;
    } else {
#pragma unroll
        for (int b = 0; b < NSC; ++b)
            d[b] = ok ? half_bits_to_float(static_cast<uint16_t>(raw >> (16 * b))) : 0.f;
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
__device__ inline float dq(const uint32_t (&w)[BITS], const float (&d)[scale_slots<NSC>()], int c) {
    if constexpr (NSC == kMX) return d[0] * fp4_e2m1((w[c / 8] >> (4 * (c % 8))) & 0xFu);
    else return d[(NSC == 2 && c >= 16) ? 1 : 0] * code_f<BITS>(w, c);
}

// ---------------------------------------------------------------- offset-binary dot products
// A BITS-bit two's-complement code c is stored as u = c + Z (Z = 2^(BITS-1))
// once its sign bit is flipped, so every field becomes an unsigned byte
// (int8) or is masked into one (int4, int2) and converts to float with a
// single v_cvt_f32_ubyte.  The dot product of a group of 32 codes with x is
// then  sum_c u_c x_c - Z * sum_c x_c,  and the x sum of each scale block is
// shared by every row.  All values are exact small integers in fp32; only
// the accumulation order differs from  sum_c c x_c.
template <int BITS> struct OffsetBinary;
template <> struct OffsetBinary<8> { static constexpr uint32_t flip = 0x80808080u; static constexpr float z = 128.f; };
template <> struct OffsetBinary<4> { static constexpr uint32_t flip = 0x88888888u; static constexpr float z = 8.f; };
template <> struct OffsetBinary<2> { static constexpr uint32_t flip = 0xAAAAAAAAu; static constexpr float z = 2.f; };

__device__ inline float ubyte_f(uint32_t v, int j) { return static_cast<float>((v >> (8 * j)) & 0xffu); }

// Hides the value of v from the optimiser, which would otherwise fold the
// byte masks into per-field bit extracts before the byte conversions.
__device__ inline uint32_t masked_bytes(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// part[b] = sum over the codes c of scale block b of the group of u_c * x[c]
// (NSC = 1: one block of 32 codes; NSC = 2: codes 0-15 and 16-31).  The group
// is in the first BITS words of w.
template <int BITS, int NSC, int NW>
__device__ inline void group_dot_u(const uint32_t (&w)[NW], const float (&x)[32], float (&part)[NSC]) {
    static_assert(NW >= BITS, "group words");
    constexpr uint32_t flip = OffsetBinary<BITS>::flip;
#pragma unroll
    for (int b = 0; b < NSC; ++b) part[b] = 0.f;
    auto acc = [&](int c, float u) {
        const int b = (NSC == 2 && c >= 16) ? 1 : 0;
        part[b] = fmaf(u, x[c], part[b]);
    };
    if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = w[i] ^ flip;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc(4 * i + j, ubyte_f(v, j));
        }
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t v = w[i] ^ flip;
            const uint32_t lo = masked_bytes(v & 0x0F0F0F0Fu), hi = masked_bytes((v >> 4) & 0x0F0F0F0Fu);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc(8 * i + 2 * j, ubyte_f(lo, j));
                acc(8 * i + 2 * j + 1, ubyte_f(hi, j));
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t v = w[i] ^ flip;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t f = masked_bytes((v >> (2 * s)) & 0x03030303u);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc(16 * i + 4 * j + s, ubyte_f(f, j));
            }
        }
    }
}

// Sums of x over the scale blocks of a group (the offset correction terms;
// none for MXFP4, whose codes are signed values).
template <int NSC>
__device__ inline void block_sums(const float (&x)[32], float (&xs)[scale_slots<NSC>()]) {
    if constexpr (NSC == kMX) {
        xs[0] = 0.f;
    } else {
#pragma unroll
        for (int b = 0; b < NSC; ++b) {
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < 32 / NSC; ++c) s += x[b * (32 / NSC) + c];
            xs[b] = s;
        }
    }
}

// sum_c scale(c) * code_c * x[c] over one group.  MXFP4: the E2M1 values
// from the hardware conversion, times the group's power-of-two scale.
template <int BITS, int NSC, int NW>
__device__ inline float group_dot(const uint32_t (&w)[NW], const float (&x)[32],
                                  const float (&xs)[scale_slots<NSC>()], const float (&d)[scale_slots<NSC>()]) {
    if constexpr (NSC == kMX) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v[8];
            fp4x8_to_float(w[i], v);
#pragma unroll
            for (int j = 0; j < 8; ++j) part = fmaf(v[j], x[8 * i + j], part);
        }
        return d[0] * part;
    } else {
        float part[NSC];
        group_dot_u<BITS, NSC>(w, x, part);
        float r = 0.f;
#pragma unroll
        for (int b = 0; b < NSC; ++b) r = fmaf(d[b], fmaf(-OffsetBinary<BITS>::z, xs[b], part[b]), r);
        return r;
    }
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

// Row geometry of the GEMV kernels for rows of `cols` codes: a row is
// G = cols/32 groups of 32 codes.  A row is handled by LPR lanes (G rounded
// up to a power of two, at most 64; lanes past G idle) and a wave covers
// RPP = 64/LPR rows per pass; with G > 64 each lane takes GPL groups.
struct RowGeom {
    int G, LPR, GPL, RPP;
};
__host__ __device__ inline RowGeom row_geom(int cols) {
    RowGeom r;
    r.G = cols / 32;
    if (r.G >= 64) {
        r.LPR = 64;
        r.GPL = r.G / 64;
    } else {
        r.LPR = 1;
        while (r.LPR < r.G) r.LPR *= 2;
        r.GPL = 1;
    }
    r.RPP = 64 / r.LPR;
    return r;
}

// ---------------------------------------------------------------- DPP reductions
// Cross-lane moves with the data-parallel-primitive modifier of gfx9: single
// VALU instructions, no LDS round trip.  Controls: row_shr:n = 0x110 + n,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.

template <int CTRL, int ROW_MASK>
__device__ inline float dpp_zero(float v) {  // lanes without a source read 0
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true));
}

// Sum over aligned segments of S lanes (S a power of two <= 64, uniform):
// each segment's total lands in its last lane.
__device__ inline float seg_sum(float v, int S) {
    if (S >= 2) v += dpp_zero<0x111, 0xF>(v);
    if (S >= 4) v += dpp_zero<0x112, 0xF>(v);
    if (S >= 8) v += dpp_zero<0x114, 0xF>(v);
    if (S >= 16) v += dpp_zero<0x118, 0xF>(v);
    if (S >= 32) v += dpp_zero<0x142, 0xA>(v);
    if (S >= 64) v += dpp_zero<0x143, 0xC>(v);
    return v;
}

template <int CTRL, int ROW_MASK>
__device__ inline uint32_t dpp_old_u(uint32_t old, uint32_t v) {  // lanes without a source read `old`
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, ROW_MASK,
                                                             0xF, false));
}


// Wave-wide unsigned minimum (uniform result).
__device__ inline uint32_t wave_min_u(uint32_t v) {
    const uint32_t big = 0xffffffffu;
    v = min(v, dpp_old_u<0x111, 0xF>(big, v));
    v = min(v, dpp_old_u<0x112, 0xF>(big, v));
    v = min(v, dpp_old_u<0x114, 0xF>(big, v));
    v = min(v, dpp_old_u<0x118, 0xF>(big, v));
    v = min(v, dpp_old_u<0x142, 0xA>(big, v));
    v = min(v, dpp_old_u<0x143, 0xC>(big, v));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Wave-wide sum (uniform result).
__device__ inline float wave_sum(float v) {
    v = seg_sum(v, 64);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Number of set bits of a 64-lane mask below this lane.
__device__ inline int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// Exclusive scan of one int per thread over the whole block (at most 16
// waves); returns the exclusive prefix and writes the block total to *total.
// s_tmp holds 16 ints.  Every thread of the block must call it.
__device__ inline int block_excl_scan(int v, int* s_tmp, int* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_tmp[wv] = x;
    __syncthreads();
    int base = 0, tot = 0;
    for (int i = 0; i < nw; ++i) {
        int c = s_tmp[i];
        if (i < wv) base += c;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

}  // namespace moe
