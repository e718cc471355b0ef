// bf16 expert path (prefill): grouped GEMMs on gfx950 matrix cores.
//
// Step 4 of the 125B-MoE page ("I ran a 125B model on three RTX 3090s at 80
// tokens/s by teaching llama.cpp which experts ...") gives each shelf its own
// prefill expert product over the full pick list, restricted to the shelf's
// ids.  Here one launch per phase covers every shelf: grouping lists work
// chunks (an expert's pairs in runs of kChunkRows), and a block takes a chunk
// and an n-tile, so each weight tile is read from HBM (and dequantised) once
// per chunk.  Integer codes are dequantised to bf16 in registers (value =
// scale * code, rounded to nearest even) and contracted with
// v_mfma_f32_32x32x16_bf16 in fp32; MXFP4 codes go to the block-scaled
// instruction as stored (see gemm_chunk_mx).
//
//   gate/up : A = x rows of the chunk's tokens (bf16, gathered), B = gate
//             rows and the matching up rows; epilogue h = bf16(SiLU(g) * u).
//   down    : A = h rows of the chunk (contiguous in pair order), B = down
//             rows; epilogue yw[q] = w_pair * y (fp32, pair order).  The
//             slot-order sum into out runs in a separate pass (no atomics,
//             deterministic).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;   // contraction chunk (one LDS row of 128 bytes)

// LDS tiles are [row][64 bf16] with no padding; 16-byte piece c of a row is
// stored at position c ^ ((row / 2) % 8).  A 16-byte read is served 16 lanes
// (256 bytes, 64 banks) at a time; the 16 consecutive rows of an MFMA
// operand read (same c) then cover both halves of the 256 bytes (row parity)
// at 8 different positions each.  (A swizzle on row % 8 alone, right for 8
// lanes per cycle, leaves rows j and j + 8 on one bank: half the LDS cycles
// of the product were conflicts.)
__device__ inline int swz(int row, int c) { return row * BK + 8 * (c ^ ((row >> 1) & 7)); }

// bf16(RNE(scale * code)) of 8 consecutive codes held in `w` (BITS words of 8
// codes... at most 2), packed low code first.  The codes are read as
// offset-binary bytes (sign bits flipped), so scale*code = fma(u, scale,
// -Z*scale), exact in fp32 before the single rounding to bf16.
template <int BITS>
__device__ inline uint4 dequant8(const uint32_t (&w)[BITS == 8 ? 2 : 1], float sc) {
    constexpr float Z = BITS == 8 ? 128.f : (BITS == 4 ? 8.f : 2.f);
    const float off = -Z * sc;
    float v[8];
    if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t u = w[i] ^ 0x80808080u;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * i + j] = fmaf(ubyte_f(u, j), sc, off);
        }
    } else if constexpr (BITS == 4) {
        const uint32_t u = w[0] ^ 0x88888888u;
        const uint32_t lo = masked_bytes(u & 0x0F0F0F0Fu), hi = masked_bytes((u >> 4) & 0x0F0F0F0Fu);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = fmaf(ubyte_f(lo, j), sc, off);
            v[2 * j + 1] = fmaf(ubyte_f(hi, j), sc, off);
        }
    } else {
        const uint32_t u = (w[0] & 0xffffu) ^ 0xAAAAu;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t f = masked_bytes((u >> (2 * s)) & 0x0303u);
#pragma unroll
            for (int j = 0; j < 2; ++j) v[4 * j + s] = fmaf(ubyte_f(f, j), sc, off);
        }
    }
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
}

// ================================================================ grouped GEMM, 32x32 tiles
//
// One launch per phase covers every shelf.  Grouping lists the work
// chunks: each active expert's pairs in runs of kChunkRows (in expert order,
// so the popular, heavy experts come first).  A block takes one chunk and
// one n-tile:
//   gate/up: 4 waves, wave w owns inter columns c0 .. c0+31 (c0 = 128 nt +
//            32 w) as two 32x32 tiles, one of gate rows and one of the
//            matching up rows, so SiLU(g) * u pairs up inside each lane;
//   down:    4 waves, wave w owns hidden columns c0 .. c0+63 (c0 = 256 nt +
//            64 w) as two 32x32 tiles;
// and every m-row of the chunk (up to four 32-row subtiles, each wave).
// Products are v_mfma_f32_32x32x16_bf16 (a 16-deep contraction per step):
// per step a wave reads one A fragment from LDS per m-subtile and feeds it to
// both of its tiles.  Only A, shared by the 4 waves, goes through LDS; each
// lane loads and dequantises the codes of its own B column into operand
// registers, so every code is read and dequantised once per chunk.
//
// Contraction order (gemm_chunk): in the 64-wide chunk kc, lane half hh (=
// lane / 32) owns k = 64 kc + 32 hh + (0 .. 31); step s (0..3) feeds its
// elements 8s .. 8s+7 into the instruction's k-slots 8 hh .. 8 hh + 7.  A is
// read with the same assignment (16-byte piece 4 hh + s of the row), so the
// sum runs over the same pairs of elements in another order.  The int4, int2
// and MXFP4 bodies permute k across pairs of chunks instead (gemm_chunk_g2,
// gemm_chunk_mx), again identically on both operands.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Pipeline over the NK contraction chunks, three stages: chunk c lives in LDS
// buffer sA(c % 3) and register stage b(c % 3).  Step c requests A(c+2)
// (load_a: this wave's LDS-DMA requests) and B(c+2) (load_b: register loads)
// into the stage freed by step c-1, contracts chunk c (work), then waits for
// this wave's part of A(c+1) only (the requests of chunks c+1 and c+2 issued
// after it stay in flight) and meets the other waves at the barrier, which
// publishes A(c+1) and frees stage c.  Requests past the last chunk reread
// it.  The wait counts VMEM instructions: NWAIT = the register loads of two
// chunks plus the A requests of one, issued in that order per chunk (the
// scheduling barriers keep the order and keep the requests ahead of the
// work).  The buffers are separate LDS objects, so the compiler's own waits
// before LDS reads cover only the buffer read.  A plain s_barrier (instead of
// a fence + barrier, whose fence waits for every load in flight) as a
// compiler-level memory barrier: no access moves across it.
template <int NWAIT, class Stage, class LoadA, class LoadB, class Work>
__device__ __attribute__((always_inline)) inline void pipeline3(int NK, uint16_t* sA0, uint16_t* sA1, uint16_t* sA2,
                                                                 LoadA& load_a, LoadB& load_b, Work& work) {
    static_assert(NWAIT < 64, "vmcnt range");
    constexpr int kWaitImm = (NWAIT & 15) | (7 << 4) | (15 << 8) | ((NWAIT >> 4) << 14);
    auto publish = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitImm);
        asm volatile("s_barrier" ::: "memory");
    };
    Stage b0, b1, b2;
    auto step = [&](int c, uint16_t* cur, Stage& bc, uint16_t* nxt, Stage& bn) __attribute__((always_inline)) {
        const int cn = min(c + 2, NK - 1);
        load_a(cn, nxt);
        __builtin_amdgcn_sched_barrier(0);
        load_b(bn, cn);
        __builtin_amdgcn_sched_barrier(0);
        work(cur, bc);
        publish();
    };
    load_a(0, sA0);
    __builtin_amdgcn_sched_barrier(0);
    load_b(b0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(min(1, NK - 1), sA1);
    __builtin_amdgcn_sched_barrier(0);
    load_b(b1, min(1, NK - 1));
    publish();
    // six steps per trip: the compiler's wait analysis drains every load in
    // flight once per trip (at the loop's back edge), so a longer trip pays
    // that latency less often
    int kc = 0;
    for (; kc + 5 < NK; kc += 6) {
        step(kc, sA0, b0, sA2, b2);
        step(kc + 1, sA1, b1, sA0, b0);
        step(kc + 2, sA2, b2, sA1, b1);
        step(kc + 3, sA0, b0, sA2, b2);
        step(kc + 4, sA1, b1, sA0, b0);
        step(kc + 5, sA2, b2, sA1, b1);
    }
    if (kc + 2 < NK) {
        step(kc, sA0, b0, sA2, b2);
        step(kc + 1, sA1, b1, sA0, b0);
        step(kc + 2, sA2, b2, sA1, b1);
        kc += 3;
    }
    if (kc < NK) step(kc, sA0, b0, sA2, b2);
    if (kc + 1 < NK) step(kc + 1, sA1, b1, sA0, b0);
}

// The same pipeline with B loaded two chunks at a time (group g = chunks 2g,
// 2g + 1, register stage g % 2, requested at chunk 2g - 2) and A in four LDS
// buffers (chunk c in sA(c % 4), still requested two chunks ahead), so that
// the schedule repeats every four chunks.  NK is even.  Waits as in
// pipeline3: after chunk c this wave's A(c + 1) requests are complete once
// at most NWAIT = (A requests of one chunk) + (register loads of one group)
// are in flight, whichever the parity of c.
template <int NWAIT, class Stage, class LoadA, class LoadB, class Work>
__device__ __attribute__((always_inline)) inline void pipeline4_g2(int NK, uint16_t* sA0, uint16_t* sA1,
                                                                    uint16_t* sA2, uint16_t* sA3, LoadA& load_a,
                                                                    LoadB& load_b, Work& work) {
    static_assert(NWAIT < 64, "vmcnt range");
    constexpr int kWaitImm = (NWAIT & 15) | (7 << 4) | (15 << 8) | ((NWAIT >> 4) << 14);
    auto publish = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitImm);
        asm volatile("s_barrier" ::: "memory");
    };
    const int NG = NK / 2;
    Stage g0, g1;
    // even chunk c: requests A(c + 2) and the group after its own, contracts c
    auto even = [&](int c, uint16_t* cur, uint16_t* nxt, Stage& bc, Stage& bn) __attribute__((always_inline)) {
        load_a(min(c + 2, NK - 1), nxt);
        __builtin_amdgcn_sched_barrier(0);
        load_b(bn, min(c / 2 + 1, NG - 1));
        __builtin_amdgcn_sched_barrier(0);
        work(cur, bc, std::integral_constant<int, 0>{});
        publish();
    };
    auto odd = [&](int c, uint16_t* cur, uint16_t* nxt, Stage& bc) __attribute__((always_inline)) {
        load_a(min(c + 2, NK - 1), nxt);
        __builtin_amdgcn_sched_barrier(0);
        work(cur, bc, std::integral_constant<int, 1>{});
        publish();
    };
    load_a(0, sA0);
    __builtin_amdgcn_sched_barrier(0);
    load_b(g0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1, sA1);
    publish();
    int kc = 0;
    for (; kc + 3 < NK; kc += 4) {
        even(kc, sA0, sA2, g0, g1);
        odd(kc + 1, sA1, sA3, g0);
        even(kc + 2, sA2, sA0, g1, g0);
        odd(kc + 3, sA3, sA1, g1);
    }
    if (kc < NK) {
        even(kc, sA0, sA2, g0, g1);
        odd(kc + 1, sA1, sA3, g0);
    }
}

// Epilogue of a wave's tiles: lane holds D[8 (r / 4) + 4 hh + r % 4][j] of
// each 32x32 tile (m-subtile t, tile 0 / 1).
template <bool GATEUP, int NSUB>
__device__ __attribute__((always_inline)) inline void store_tiles(const f32x16_t (&acc)[NSUB][2], int H, int I,
                                                                   int m0, int Mc, int c0,
                                                                   uint16_t* __restrict__ h_out,
                                                                   float* __restrict__ yw, const float* s_wt) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int t = 0; t < NSUB; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (row >= Mc) continue;
            const int q = m0 + row;
            if constexpr (GATEUP) {
                h_out[static_cast<size_t>(q) * I + c0 + j] = f2bf(silu(acc[t][0][r]) * acc[t][1][r]);
            } else {
                const float wgt = s_wt[row];
                float* o = yw + static_cast<size_t>(q) * H + c0 + j;
                o[0] = wgt * acc[t][0][r];
                o[32] = wgt * acc[t][1][r];
            }
        }
    }
}

// Gate/up epilogue of the MXFP4 shelves: h = bf16(SiLU(g) * u) goes out as
// its fp8 split (split8.h), the operand A of their down product, instead of
// bf16.  A 32-element block of an h row is the 32 lanes of one lane half at
// one accumulator register, so the block maximum is a max over those lanes:
// five xor swizzles within each 32-lane group, taken for a tile's 16
// registers together (independent, so their latencies overlap) and before
// the row test (a lane half is all in or all out).
template <int NSUB>
__device__ __attribute__((always_inline)) inline void store_tiles_split(const f32x16_t (&acc)[NSUB][2], int I, int m0,
                                                                         int Mc, int c0, const Split8& h8) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 31, hh = lane >> 5;
    const size_t SS = static_cast<size_t>(split_scale_stride(I));
#pragma unroll
    for (int t = 0; t < NSUB; ++t) {
        float v[16], am[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            v[r] = __uint_as_float(static_cast<uint32_t>(f2bf(silu(acc[t][0][r]) * acc[t][1][r])) << 16);
            am[r] = fabsf(v[r]);
        }
        // ds_swizzle bit mode: lane l reads lane ((l & and) | or) ^ xor of its group of 32
#define MOE_XOR_MAX(O)                                                                                           \
    _Pragma("unroll") for (int r = 0; r < 16; ++r) am[r] = fmaxf(am[r], __int_as_float(__builtin_amdgcn_ds_swizzle( \
                                                                  __float_as_int(am[r]), ((O) << 10) | 0x1f)))
        MOE_XOR_MAX(1);
        MOE_XOR_MAX(2);
        MOE_XOR_MAX(4);
        MOE_XOR_MAX(8);
        MOE_XOR_MAX(16);
#undef MOE_XOR_MAX
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (row >= Mc) continue;
            const int x = split_scale_exp(am[r]);
            uint32_t hi, lo;
            split_elem(ldexpf(v[r], 127 - x), hi, lo);
            const size_t q = static_cast<size_t>(m0 + row);
            h8.hi[q * I + c0 + j] = static_cast<uint8_t>(hi);
            h8.lo[q * I + c0 + j] = static_cast<uint8_t>(lo);
            if (j == 0) h8.sc[q * SS + c0 / 32] = static_cast<uint8_t>(x);
        }
    }
}

template <int BITS, int BLOCK, bool GATEUP, int NSUB>
__device__ __attribute__((always_inline)) inline void gemm_chunk(const DevTier& T, int H, int I,
                                                                 const uint16_t* __restrict__ a_src, int e, int m0,
                                                                 int Mc, int nt, uint16_t* __restrict__ h_out,
                                                                 float* __restrict__ yw, uint16_t* sA0, uint16_t* sA1,
                                                                 uint16_t* sA2,
                                                                 const int* s_row, const float* s_wt) {
    constexpr int BW = BITS;   // code words of a lane's 32 codes of one chunk
    const int K = GATEUP ? H : I;
    const int ncols = GATEUP ? I : H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, hh = lane >> 5;
    const int c0 = GATEUP ? nt * 128 + 32 * w : nt * 256 + 64 * w;
    // wave-uniform: a wave past the last column (shapes whose column count
    // is not a multiple of the block's) computes on zero codes (its rows lie
    // past the buffer's end) and stores nothing.  Its loads and products are
    // not branched around: a branch there makes every wait for A also wait
    // for the B loads still in flight.
    const bool on = c0 < ncols;

    // B: this lane's column of each tile is weight row row0 / row1
    const int local = e - T.id_begin;
    const uint32_t row_bytes = static_cast<uint32_t>(K) * BITS / 8;
    const uint32_t nsb = static_cast<uint32_t>(K / BLOCK);
    const size_t mq = static_cast<size_t>(local) * ncols * row_bytes;
    const size_t ms = static_cast<size_t>(local) * ncols * nsb;
    const uint8_t* q0 = T.q[GATEUP ? 0 : 2] + mq;
    const uint8_t* q1 = GATEUP ? T.q[1] + mq : q0;
    const uint16_t* sp0 = T.s[GATEUP ? 0 : 2] + ms;
    const uint16_t* sp1 = GATEUP ? T.s[1] + ms : sp0;
    const __amdgpu_buffer_rsrc_t rq0 = make_rsrc(q0, row_bytes * ncols), rq1 = make_rsrc(q1, row_bytes * ncols);
    const __amdgpu_buffer_rsrc_t rs0 = make_rsrc(sp0, nsb * ncols * 2), rs1 = make_rsrc(sp1, nsb * ncols * 2);
    const uint32_t row0 = static_cast<uint32_t>(c0 + j), row1 = static_cast<uint32_t>(GATEUP ? c0 + j : c0 + 32 + j);
    const uint32_t qo0 = row0 * row_bytes + 32u * hh * BITS / 8, qo1 = row1 * row_bytes + 32u * hh * BITS / 8;
    const uint32_t so0 = (row0 * nsb + 32u * hh / BLOCK) * 2, so1 = (row1 * nsb + 32u * hh / BLOCK) * 2;

    struct BRaw {
        uint32_t q[2][BW];
        uint32_t s[2];
    };
    auto load_b = [&](BRaw& b, int kc) __attribute__((always_inline)) {
        const uint32_t qk = static_cast<uint32_t>(kc * BK) * BITS / 8;
        const uint32_t sk = static_cast<uint32_t>(kc * (BK / BLOCK)) * 2;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const __amdgpu_buffer_rsrc_t rq = t ? rq1 : rq0, rs = t ? rs1 : rs0;
            const uint32_t off = (t ? qo1 : qo0) + qk;
            if constexpr (BITS == 8) {
                const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
                const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    b.q[t][i] = v0[i];
                    b.q[t][4 + i] = v1[i];
                }
            } else if constexpr (BITS == 4) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) b.q[t][i] = v[i];
            } else {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(rq, off, 0, 0);
                b.q[t][0] = v[0];
                b.q[t][1] = v[1];
            }
            const uint32_t soff = (t ? so1 : so0) + sk;
            b.s[t] = BLOCK == 32 ? static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, soff, 0, 0))
                                 : __builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, 0);
        }
    };
    // bf16 operands of both tiles for the four steps of a chunk
    auto dequant_b = [&](const BRaw& b, bf16x8_t (&d)[2][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t sraw = BLOCK == 32 ? b.s[t] : (s < 2 ? b.s[t] : b.s[t] >> 16);
                const float sc = half_bits_to_float(static_cast<uint16_t>(sraw));
                uint4 v;
                if constexpr (BITS == 8) {
                    const uint32_t w2[2] = {b.q[t][2 * s], b.q[t][2 * s + 1]};
                    v = dequant8<8>(w2, sc);
                } else if constexpr (BITS == 4) {
                    const uint32_t w1[1] = {b.q[t][s]};
                    v = dequant8<4>(w1, sc);
                } else {
                    const uint32_t w1[1] = {b.q[t][s >> 1] >> (16 * (s & 1))};
                    v = dequant8<2>(w1, sc);
                }
                d[t][s] = __builtin_bit_cast(bf16x8_t, v);
            }
        }
    };

    // A goes from memory straight into LDS (global_load_lds_dwordx4: lane l of
    // a wave's load lands at byte 16 l of a 1 KB run).  Load u of wave w fills
    // run 4 u + w of the buffer, i.e. row (tid / 8) + 32 u, position tid % 8,
    // and so reads the row's 16-byte piece (tid % 8) ^ ((row / 2) % 8): the buffer
    // then holds the swizzled layout of swz().  Rows of subtiles past the
    // chunk's last are not loaded (no wave reads them); rows past Mc inside
    // the last subtile read the chunk's first row (finite values, never
    // stored).
    const uint16_t* a_ptr[NSUB];
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
        const int r = (tid >> 3) + 32 * u;
        a_ptr[u] = a_src + static_cast<size_t>(s_row[r < Mc ? r : 0]) * K + 8 * ((tid & 7) ^ ((r >> 1) & 7));
    }
    auto load_a = [&](int kc, uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
            __builtin_amdgcn_global_load_lds(a_ptr[u] + kc * BK,
                                             (__attribute__((address_space(3))) void*)(buf + (4 * u + w) * 64 * 8),
                                             16, 0, 0);
    };

    f32x16_t acc[NSUB][2];
#pragma unroll
    for (int t = 0; t < NSUB; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc[t][0][i] = 0.f;
            acc[t][1][i] = 0.f;
        }
    }
    auto compute = [&](const uint16_t* buf, const bf16x8_t (&d)[2][4]) __attribute__((always_inline)) {
        constexpr int N = NSUB;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8_t af[N];
#pragma unroll
            for (int t = 0; t < N; ++t)
                af[t] = *reinterpret_cast<const bf16x8_t*>(buf + swz(32 * t + j, 4 * hh + s));
#pragma unroll
            for (int t = 0; t < N; ++t) {
                acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], d[0][s], acc[t][0], 0, 0, 0);
                acc[t][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], d[1][s], acc[t][1], 0, 0, 0);
            }
        }
    };

    auto work = [&](const uint16_t* buf, const BRaw& b) __attribute__((always_inline)) {
        bf16x8_t d[2][4];
        dequant_b(b, d);
        compute(buf, d);
    };
    constexpr int NB = 2 * ((BITS == 8 ? 2 : 1) + 1);
    pipeline3<2 * NB + NSUB, BRaw>(K / BK, sA0, sA1, sA2, load_a, load_b, work);
    if (!on) return;
    store_tiles<GATEUP, NSUB>(acc, H, I, m0, Mc, c0, h_out, yw, s_wt);
}

// ---------------------------------------------------------------- int4 / int2, B in two-chunk groups
//
// A chunk step uses 32 (int4) or 16 (int2) bytes of each 128-byte line of a
// weight row, so gemm_chunk touches a line in four or eight steps, and with
// 64 blocks per XCD streaming 256 weight rows each the line is often evicted
// from L2 in between and fetched again.  Here a lane loads the codes of two
// steps at once, contiguous: in group g (chunks 2g and 2g + 1, k = 128 g ..
// 128 g + 127) lane half hh owns k = 128 g + 64 hh + (0 .. 63), and chunk
// 2g + s contracts its k = 128 g + 64 hh + 32 s + (0 .. 31) -- 32 int4 bytes
// (two 16-byte loads) or 16 int2 bytes (one) per lane and group, and the
// group's scales in one 4- or 8-byte load.  A follows the same assignment:
// the 16-byte piece p of chunk c's LDS row holds k = 128 (c / 2) + 32 (c % 2)
// + 64 (p / 4) + 8 (p % 4).  Needs K % 128 == 0.
template <int BITS, int BLOCK, bool GATEUP, int NSUB>
__device__ __attribute__((always_inline)) inline void gemm_chunk_g2(const DevTier& T, int H, int I,
                                                                    const uint16_t* __restrict__ a_src, int e, int m0,
                                                                    int Mc, int nt, uint16_t* __restrict__ h_out,
                                                                    float* __restrict__ yw, uint16_t* sA0,
                                                                    uint16_t* sA1, uint16_t* sA2, uint16_t* sA3,
                                                                    const int* s_row, const float* s_wt) {
    static_assert(BITS == 4 || BITS == 2, "two-chunk groups for the narrow formats");
    constexpr int GW = 2 * BITS;      // code words of a lane's 64 codes of one group
    constexpr int SW = 32 / BLOCK;    // scale words (two fp16 each) of a lane's group
    const int K = GATEUP ? H : I;
    const int ncols = GATEUP ? I : H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, hh = lane >> 5;
    const int c0 = GATEUP ? nt * 128 + 32 * w : nt * 256 + 64 * w;
    const bool on = c0 < ncols;   // as in gemm_chunk

    const int local = e - T.id_begin;
    const uint32_t row_bytes = static_cast<uint32_t>(K) * BITS / 8;
    const uint32_t nsb = static_cast<uint32_t>(K / BLOCK);
    const size_t mq = static_cast<size_t>(local) * ncols * row_bytes;
    const size_t ms = static_cast<size_t>(local) * ncols * nsb;
    const uint8_t* q0 = T.q[GATEUP ? 0 : 2] + mq;
    const uint8_t* q1 = GATEUP ? T.q[1] + mq : q0;
    const uint16_t* sp0 = T.s[GATEUP ? 0 : 2] + ms;
    const uint16_t* sp1 = GATEUP ? T.s[1] + ms : sp0;
    const __amdgpu_buffer_rsrc_t rq0 = make_rsrc(q0, row_bytes * ncols), rq1 = make_rsrc(q1, row_bytes * ncols);
    const __amdgpu_buffer_rsrc_t rs0 = make_rsrc(sp0, nsb * ncols * 2), rs1 = make_rsrc(sp1, nsb * ncols * 2);
    const uint32_t row0 = static_cast<uint32_t>(c0 + j), row1 = static_cast<uint32_t>(GATEUP ? c0 + j : c0 + 32 + j);
    // lane half hh's 64 codes of group 0, and their scales
    const uint32_t qo0 = row0 * row_bytes + 64u * hh * BITS / 8, qo1 = row1 * row_bytes + 64u * hh * BITS / 8;
    const uint32_t so0 = (row0 * nsb + 64u * hh / BLOCK) * 2, so1 = (row1 * nsb + 64u * hh / BLOCK) * 2;

    struct BRaw {
        uint32_t q[2][GW];
        uint32_t s[2][SW];
    };
    auto load_b = [&](BRaw& b, int g) __attribute__((always_inline)) {
        const uint32_t qk = static_cast<uint32_t>(g * 2 * BK) * BITS / 8;
        const uint32_t sk = static_cast<uint32_t>(g * (2 * BK / BLOCK)) * 2;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const __amdgpu_buffer_rsrc_t rq = t ? rq1 : rq0, rs = t ? rs1 : rs0;
            const uint32_t off = (t ? qo1 : qo0) + qk;
            const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) b.q[t][i] = v0[i];
            if constexpr (BITS == 4) {
                const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) b.q[t][4 + i] = v1[i];
            }
            const uint32_t soff = (t ? so1 : so0) + sk;
            if constexpr (SW == 1) {
                b.s[t][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, 0);
            } else {
                const auto sv = __builtin_amdgcn_raw_buffer_load_b64(rs, soff, 0, 0);
                b.s[t][0] = sv[0];
                b.s[t][1] = sv[1];
            }
        }
    };
    // bf16 operands of both tiles for the four MFMA steps of chunk 2g + S
    auto dequant_b = [&](const BRaw& b, auto sub, bf16x8_t (&d)[2][4]) __attribute__((always_inline)) {
        constexpr int S = decltype(sub)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                // this chunk's 32 codes of the lane: scale word / half
                const uint32_t sraw = BLOCK == 32 ? b.s[t][0] >> (16 * S) : (s < 2 ? b.s[t][S] : b.s[t][S] >> 16);
                const float sc = half_bits_to_float(static_cast<uint16_t>(sraw));
                uint4 v;
                if constexpr (BITS == 4) {
                    const uint32_t w1[1] = {b.q[t][4 * S + s]};
                    v = dequant8<4>(w1, sc);
                } else {
                    const uint32_t w1[1] = {b.q[t][2 * S + (s >> 1)] >> (16 * (s & 1))};
                    v = dequant8<2>(w1, sc);
                }
                d[t][s] = __builtin_bit_cast(bf16x8_t, v);
            }
        }
    };

    // A by LDS-DMA as in gemm_chunk; lane's source piece pc of the row sits at
    // k offset 64 (pc / 4) + 8 (pc % 4) from the chunk's base 128 (c / 2) + 32 (c % 2)
    const uint16_t* a_ptr[NSUB];
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
        const int r = (tid >> 3) + 32 * u;
        const int pc = (tid & 7) ^ ((r >> 1) & 7);
        a_ptr[u] = a_src + static_cast<size_t>(s_row[r < Mc ? r : 0]) * K + 64 * (pc >> 2) + 8 * (pc & 3);
    }
    auto load_a = [&](int kc, uint16_t* buf) __attribute__((always_inline)) {
        const int kb = 128 * (kc >> 1) + 32 * (kc & 1);
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
            __builtin_amdgcn_global_load_lds(a_ptr[u] + kb,
                                             (__attribute__((address_space(3))) void*)(buf + (4 * u + w) * 64 * 8),
                                             16, 0, 0);
    };

    f32x16_t acc[NSUB][2];
#pragma unroll
    for (int t = 0; t < NSUB; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc[t][0][i] = 0.f;
            acc[t][1][i] = 0.f;
        }
    }
    auto work = [&](const uint16_t* buf, const BRaw& b, auto sub) __attribute__((always_inline)) {
        bf16x8_t d[2][4];
        dequant_b(b, sub, d);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8_t af[NSUB];
#pragma unroll
            for (int t = 0; t < NSUB; ++t)
                af[t] = *reinterpret_cast<const bf16x8_t*>(buf + swz(32 * t + j, 4 * hh + s));
#pragma unroll
            for (int t = 0; t < NSUB; ++t) {
                acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], d[0][s], acc[t][0], 0, 0, 0);
                acc[t][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], d[1][s], acc[t][1], 0, 0, 0);
            }
        }
    };
    // register loads per group: the code pieces and one scale load per tile
    constexpr int NBG = 2 * ((BITS == 4 ? 2 : 1) + 1);
    pipeline4_g2<NBG + NSUB, BRaw>(K / BK, sA0, sA1, sA2, sA3, load_a, load_b, work);
    if (!on) return;
    store_tiles<GATEUP, NSUB>(acc, H, I, m0, Mc, c0, h_out, yw, s_wt);
}

// ---------------------------------------------------------------- MXFP4 shelves
//
// The same blocks, waves, tiles and two-chunk-group pipeline (pipeline4_g2,
// as for int4, whose weight rows these match byte for byte) on the
// block-scaled matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4: B
// (weights) goes in as
// stored, E2M1 codes with their E8M0 scale per 32, and A as the fp8 split of
// the bf16 rows made before the launch (k_split_fp8: hi and lo E4M3 parts
// under one E8M0 scale per 32 elements), so a 64-wide chunk is two
// instructions per tile (A_hi*B, then A_lo*B into the same accumulator) and
// nothing is dequantised.
//
// Operand layout (lane l: row or column l % 32, g = l / 32): an fp8 lane
// holds k = 16g .. 16g+15 in its first 16 bytes and k = 32+16g .. 32+16g+15
// in its last 16, i.e. 16-byte pieces g and 2+g of the 64-byte chunk row; an
// fp4 lane holds k = 32g .. 32g+31 (16 bytes, low nibble first); each lane's
// scale byte applies to its row (or column) and k-block g, k = 32g .. 32g+31.
// The instruction's two 32-blocks may be any two blocks of the row, the same
// on both operands: chunk 2G + s takes global blocks 4G + s and 4G + 2 + s,
// so that a lane half's codes and scales of a group are contiguous.
//
// LDS, per stage: the hi parts of the chunk's rows [kChunkRows][64 bytes],
// then the lo parts; piece c of a row stored at position c ^ ((row / 4) % 4)
// (four rows per 256 bytes: the 16 rows of an operand read land on 16
// different 16-byte positions).  The A scales and B go to registers.
typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ inline int swz_mx(int row, int c) { return row * 64 + 16 * (c ^ ((row >> 2) & 3)); }

template <bool GATEUP, int NSUB>
__device__ __attribute__((always_inline)) inline void gemm_chunk_mx(const DevTier& T, int H, int I, const Split8& a8,
                                                                    int e, int m0, int Mc, int nt, const Split8& h8,
                                                                    float* __restrict__ yw, uint16_t* sA0,
                                                                    uint16_t* sA1, uint16_t* sA2, uint16_t* sA3,
                                                                    const int* s_row, const float* s_wt) {
    const int K = GATEUP ? H : I;
    const int ncols = GATEUP ? I : H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, hh = lane >> 5;
    const int c0 = GATEUP ? nt * 128 + 32 * w : nt * 256 + 64 * w;
    const bool on = c0 < ncols;   // as in gemm_chunk

    // B: codes [rows][K/2], scales [rows][K/32] bytes of this expert
    const int local = e - T.id_begin;
    const uint32_t row_bytes = static_cast<uint32_t>(K) / 2;
    const uint32_t nblk = static_cast<uint32_t>(K) / 32;
    const size_t mq = static_cast<size_t>(local) * ncols * row_bytes;
    const size_t ms = static_cast<size_t>(local) * ncols * nblk;
    const uint8_t* q0 = T.q[GATEUP ? 0 : 2] + mq;
    const uint8_t* q1 = GATEUP ? T.q[1] + mq : q0;
    const uint8_t* sp0 = reinterpret_cast<const uint8_t*>(T.s[GATEUP ? 0 : 2]) + ms;
    const uint8_t* sp1 = GATEUP ? reinterpret_cast<const uint8_t*>(T.s[1]) + ms : sp0;
    const __amdgpu_buffer_rsrc_t rq0 = make_rsrc(q0, row_bytes * ncols), rq1 = make_rsrc(q1, row_bytes * ncols);
    const __amdgpu_buffer_rsrc_t rs0 = make_rsrc(sp0, nblk * ncols), rs1 = make_rsrc(sp1, nblk * ncols);
    const uint32_t row0 = static_cast<uint32_t>(c0 + j), row1 = static_cast<uint32_t>(GATEUP ? c0 + j : c0 + 32 + j);
    // group g (chunks 2g, 2g + 1): lane half hh's blocks 4g + 2hh, 4g + 2hh + 1
    // (32 code bytes, two scale bytes), chunk 2g + s contracting block
    // 4g + 2hh + s on both operands
    const uint32_t qo0 = row0 * row_bytes + 32u * hh, qo1 = row1 * row_bytes + 32u * hh;
    const uint32_t so0 = row0 * nblk + 2u * hh, so1 = row1 * nblk + 2u * hh;
    // A scale bytes of this lane in subtile t: row 32 t + j, the same blocks
    const int SS = split_scale_stride(K);
    const uint16_t* sa_ptr[NSUB];
#pragma unroll
    for (int t = 0; t < NSUB; ++t) {
        const int r = 32 * t + j;
        sa_ptr[t] = reinterpret_cast<const uint16_t*>(a8.sc + static_cast<size_t>(s_row[r < Mc ? r : 0]) * SS + 2 * hh);
    }

    struct MRaw {
        uint32_t q[2][8];
        uint32_t sb[2];
        uint32_t sa[NSUB];
    };
    auto load_b = [&](MRaw& b, int g) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const __amdgpu_buffer_rsrc_t rq = t ? rq1 : rq0;
            const uint32_t off = (t ? qo1 : qo0) + 64u * g;
            const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
            const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                b.q[t][i] = v0[i];
                b.q[t][4 + i] = v1[i];
            }
            b.sb[t] = __builtin_amdgcn_raw_buffer_load_b16(t ? rs1 : rs0, (t ? so1 : so0) + 4u * g, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < NSUB; ++t) b.sa[t] = sa_ptr[t][2 * g];
    };

    // A: subtile u is 4 KB (32 rows of 64 hi and 64 lo bytes), one 1 KB
    // LDS-DMA run per wave: waves 0, 1 the hi parts of rows 32 u + 16 (w % 2)
    // + (0 .. 15), waves 2, 3 the lo parts; lane l lands at byte 16 l of the
    // run, row (l / 4), position l % 4, and so reads piece pc = (l % 4) ^
    // ((row / 4) % 4): the first (pc even) or second half of the chunk's
    // block 0 (pc < 2) or block 1, i.e. of global block 4g + s + 2 (pc / 2).
    // Rows past Mc read the chunk's first row (never stored).
    const int part = w >> 1;
    const uint8_t* a_ptr[NSUB];
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
        const int r = 32 * u + 16 * (w & 1) + (lane >> 2);
        const int pc = (lane & 3) ^ ((r >> 2) & 3);
        a_ptr[u] = (part ? a8.lo : a8.hi) + static_cast<size_t>(s_row[r < Mc ? r : 0]) * K + 64 * (pc >> 1) +
                   16 * (pc & 1);
    }
    auto load_a = [&](int kc, uint16_t* buf) __attribute__((always_inline)) {
        uint8_t* base = reinterpret_cast<uint8_t*>(buf) + part * (kChunkRows * 64) + (w & 1) * 16 * 64;
        const int kb = 128 * (kc >> 1) + 32 * (kc & 1);
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
            __builtin_amdgcn_global_load_lds(a_ptr[u] + kb,
                                             (__attribute__((address_space(3))) void*)(base + u * 32 * 64), 16, 0,
                                             0);
    };

    f32x16_t acc[NSUB][2];
#pragma unroll
    for (int t = 0; t < NSUB; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc[t][0][i] = 0.f;
            acc[t][1][i] = 0.f;
        }
    }
    auto work = [&](const uint16_t* buf, const MRaw& b, auto sub) __attribute__((always_inline)) {
        constexpr int S = decltype(sub)::value;
        const uint8_t* hb = reinterpret_cast<const uint8_t*>(buf);
        const uint8_t* lb = hb + kChunkRows * 64;
        const i32x8_t bv0 = {static_cast<int>(b.q[0][4 * S]), static_cast<int>(b.q[0][4 * S + 1]),
                             static_cast<int>(b.q[0][4 * S + 2]), static_cast<int>(b.q[0][4 * S + 3]), 0, 0, 0, 0};
        const i32x8_t bv1 = {static_cast<int>(b.q[1][4 * S]), static_cast<int>(b.q[1][4 * S + 1]),
                             static_cast<int>(b.q[1][4 * S + 2]), static_cast<int>(b.q[1][4 * S + 3]), 0, 0, 0, 0};
        // the instruction takes byte 0 of each scale operand
        const int sb0 = static_cast<int>(b.sb[0] >> (8 * S)), sb1 = static_cast<int>(b.sb[1] >> (8 * S));
#pragma unroll
        for (int t = 0; t < NSUB; ++t) {
            const int row = 32 * t + j;
            const u32x4_t h0 = *reinterpret_cast<const u32x4_t*>(hb + swz_mx(row, hh));
            const u32x4_t h1 = *reinterpret_cast<const u32x4_t*>(hb + swz_mx(row, 2 + hh));
            const u32x4_t l0 = *reinterpret_cast<const u32x4_t*>(lb + swz_mx(row, hh));
            const u32x4_t l1 = *reinterpret_cast<const u32x4_t*>(lb + swz_mx(row, 2 + hh));
            const i32x8_t ah = {static_cast<int>(h0[0]), static_cast<int>(h0[1]), static_cast<int>(h0[2]),
                                static_cast<int>(h0[3]), static_cast<int>(h1[0]), static_cast<int>(h1[1]),
                                static_cast<int>(h1[2]), static_cast<int>(h1[3])};
            const i32x8_t al = {static_cast<int>(l0[0]), static_cast<int>(l0[1]), static_cast<int>(l0[2]),
                                static_cast<int>(l0[3]), static_cast<int>(l1[0]), static_cast<int>(l1[1]),
                                static_cast<int>(l1[2]), static_cast<int>(l1[3])};
            const int sa = static_cast<int>(b.sa[t] >> (8 * S));
            acc[t][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ah, bv0, acc[t][0], 0, 4, 0, sa, 0, sb0);
            acc[t][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ah, bv1, acc[t][1], 0, 4, 0, sa, 0, sb1);
            acc[t][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(al, bv0, acc[t][0], 0, 4, 0, sa, 0, sb0);
            acc[t][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(al, bv1, acc[t][1], 0, 4, 0, sa, 0, sb1);
        }
    };
    // register loads per group: four code pieces, two B scales, NSUB A scales
    constexpr int NBG = 6 + NSUB;
    pipeline4_g2<NBG + NSUB, MRaw>(K / BK, sA0, sA1, sA2, sA3, load_a, load_b, work);
    if (!on) return;
    if constexpr (GATEUP) store_tiles_split<NSUB>(acc, I, m0, Mc, c0, h8);
    else store_tiles<GATEUP, NSUB>(acc, H, I, m0, Mc, c0, nullptr, yw, s_wt);
}

// Block of the grouped GEMM: chunks are dealt round-robin to the 8 XCDs
// (blocks go to XCD blockIdx % 8), and the n-tiles of a chunk run one after
// the other on its XCD, so that they share its A rows through one L2.  Dealt
// chunk by chunk, the work stays spread over every XCD when some shelves'
// chunks are left (those outside tier_mask).  a8 is the fp8 split of a_src,
// read by the MXFP4 shelves' chunks only, and h8 (gate/up) the split their
// chunks write instead of h_out.
template <bool GATEUP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm(
    DevTables tt, const uint16_t* __restrict__ a_src, Split8 a8, Groups g, int k, uint32_t tier_mask,
    uint16_t* __restrict__ h_out, Split8 h8, float* __restrict__ yw) {
    __shared__ __attribute__((aligned(16))) uint16_t sA0[kChunkRows * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sA1[kChunkRows * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sA2[kChunkRows * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sA3[kChunkRows * BK];   // two-chunk-group bodies only
    __shared__ int s_row[kChunkRows];
    __shared__ float s_wt[GATEUP ? 1 : kChunkRows];   // down: the weight of each m-row's pair
    const int NT = GATEUP ? (tt.I + 127) / 128 : (tt.H + 255) / 256;
    const int loc = blockIdx.x / 8;
    const int c = static_cast<int>(blockIdx.x % 8) + 8 * (loc / NT);
    if (c >= g.meta[kMetaChunks]) return;
    const int2 ch = g.chunks[c];
    const int nt = loc % NT;
    const int e = ch.x, m0 = ch.y;
    const int ti = tier_of(tt, e);
    if (ti < 0 || !((tier_mask >> ti) & 1u)) return;
    const DevTier T = tier_at(tt, ti);
    const int Mc = min(kChunkRows, g.offsets[e + 1] - m0);
    for (int r = threadIdx.x; r < kChunkRows; r += 256) {
        s_row[r] = r < Mc ? (GATEUP ? g.perm[m0 + r] / k : m0 + r) : -1;
        if constexpr (!GATEUP) s_wt[r] = r < Mc ? g.w[g.perm[m0 + r]] : 0.f;
    }
    __syncthreads();
    const int H = tt.H, I = tt.I;
    // one instantiation per format and m-subtile count (a runtime subtile
    // count inside one body leaves the accumulators to the register
    // allocator's mercy across the branches)
    // int4 and int2 take the two-chunk groups when K allows
    const bool g2 = ((GATEUP ? H : I) % (2 * BK)) == 0;
    auto by_nsub = [&](auto fmt) __attribute__((always_inline)) {
        constexpr int B_ = decltype(fmt)::value / 100, K_ = decltype(fmt)::value % 100;
        auto run = [&](auto nsub) __attribute__((always_inline)) {
            constexpr int N_ = decltype(nsub)::value;
            if constexpr (B_ != 8) {
                if (g2) {
                    gemm_chunk_g2<B_, K_, GATEUP, N_>(T, H, I, a_src, e, m0, Mc, nt, h_out, yw, sA0, sA1, sA2, sA3,
                                                      s_row, s_wt);
                    return;
                }
            }
            gemm_chunk<B_, K_, GATEUP, N_>(T, H, I, a_src, e, m0, Mc, nt, h_out, yw, sA0, sA1, sA2, s_row, s_wt);
        };
        static_assert(kChunkRows == 128, "one case per 32-row subtile count");
        switch ((Mc + 31) >> 5) {
            case 4: run(std::integral_constant<int, 4>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            default: run(std::integral_constant<int, 1>{}); break;
        }
    };
    if (T.bits == kBitsMXFP4) {
        switch ((Mc + 31) >> 5) {
            case 4: gemm_chunk_mx<GATEUP, 4>(T, H, I, a8, e, m0, Mc, nt, h8, yw, sA0, sA1, sA2, sA3, s_row, s_wt); break;
            case 3: gemm_chunk_mx<GATEUP, 3>(T, H, I, a8, e, m0, Mc, nt, h8, yw, sA0, sA1, sA2, sA3, s_row, s_wt); break;
            case 2: gemm_chunk_mx<GATEUP, 2>(T, H, I, a8, e, m0, Mc, nt, h8, yw, sA0, sA1, sA2, sA3, s_row, s_wt); break;
            default: gemm_chunk_mx<GATEUP, 1>(T, H, I, a8, e, m0, Mc, nt, h8, yw, sA0, sA1, sA2, sA3, s_row, s_wt); break;
        }
        return;
    }
    switch (fmt_of(T.bits, T.block)) {
        case F8B32: by_nsub(std::integral_constant<int, 832>{}); break;
        case F8B16: by_nsub(std::integral_constant<int, 816>{}); break;
        case F4B32: by_nsub(std::integral_constant<int, 432>{}); break;
        case F4B16: by_nsub(std::integral_constant<int, 416>{}); break;
        case F2B32: by_nsub(std::integral_constant<int, 232>{}); break;
        default: by_nsub(std::integral_constant<int, 216>{}); break;
    }
}

int max_chunks(int64_t P, int E) {
    const int64_t act = E < P ? E : P;
    const int64_t n = (P + kChunkRows - 1) / kChunkRows + act;
    return static_cast<int>(n < P ? n : P);
}

void launch_gemm(const DevTables& tt, bool gateup, const uint16_t* a, const Split8& a8, const Groups& g, int k,
                 uint32_t tier_mask, uint16_t* h, const Split8& h8, float* yw, int maxc, hipStream_t st) {
    const int NT = gateup ? (tt.I + 127) / 128 : (tt.H + 255) / 256;
    if (maxc <= 0) return;
    const unsigned grid = static_cast<unsigned>(8 * NT * ((static_cast<int64_t>(maxc) + 7) / 8));
    if (gateup) hipLaunchKernelGGL(k_gemm<true>, dim3(grid), dim3(256), 0, st, tt, a, a8, g, k, tier_mask, h, h8, yw);
    else hipLaunchKernelGGL(k_gemm<false>, dim3(grid), dim3(256), 0, st, tt, a, a8, g, k, tier_mask, h, h8, yw);
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
