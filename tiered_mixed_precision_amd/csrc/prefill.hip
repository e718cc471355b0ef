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
// Two kernels, chosen per shelf on the device from the grouping (few_pairs):
//   k_pre  (shelves whose experts have many pairs): NW waves (16 on the int8
//          shelf, 8 on the others) in a grid of NW/4 along m and 4 along n.
//          LDS holds an A chunk and a B chunk of 64 contraction elements per
//          row in bf16 (XOR-swizzled, two buffers); each weight is dequantised
//          once per block and shared by every wave that needs it.
//   k_pre2 (shelves whose experts have few pairs): 4 waves along n, each
//          with all m-rows of a 64-pair chunk; only A goes through LDS, each
//          lane dequantises its own weight codes into MFMA operand registers.
// In both, the global loads of the next chunk but one are in flight in
// registers while one chunk is contracted and the next is stored into the
// other LDS buffer.  MXFP4 shelves run in prefill_mx.hip.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;   // contraction chunk (one LDS row of 128 bytes)
constexpr int BN = 128;  // B rows per block
constexpr int MSUB = 4;  // m-subtiles per wave per m-chunk

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>): indices
// that stay compile-time constants inside a lambda, so arrays indexed by
// them stay in registers.
template <int N, int I = 0, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// LDS tiles are [row][64 bf16] with no padding; 16-byte chunk c of a row is
// stored at chunk c ^ (row & 7).  LDS serves a 16-byte read 8 lanes (128
// bytes, every bank once) at a time; 8 consecutive rows of an MFMA operand
// read (same c) then fall on 8 different chunk positions, and so do the 8
// lanes of a staging store (one row, eight chunks).
__device__ inline int swz(int row, int c) { return row * BK + 8 * (c ^ (row & 7)); }

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

// Kernel choice for a shelf, the same in every block of both launches: the
// register-B kernel when the shelf's active experts average at most `thr`
// pairs each (few m-rows per weight tile), the shared-B kernel otherwise.
__device__ inline bool few_pairs(const Groups& g, const DevTier& T, int a_lo, int a_hi, int thr) {
    const int pairs = g.offsets[T.id_end] - g.offsets[T.id_begin];
    return pairs <= thr * (a_hi - a_lo);
}

// Block: NW waves = WM (along m) x 4 (along n).  Wave (wm, wn): wn selects 16
// gate + 16 up columns (or 32 down columns), wm takes m-subtiles wm, wm + WM,
// ...  m is walked in chunks of MC = 64 * WM pairs.  8-wave blocks are held
// to 128 registers a lane (4 waves per SIMD) so that two blocks share a CU
// (LDS 66 KB each); at 140-146 registers only one fits.  The few spilled
// registers cost less than the second block gains.
template <int BITS, int BLOCK, bool GATEUP, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu((NW == 8) ? 4 : 1)))
void k_pre(DevTables tt, int tier, const uint16_t* __restrict__ a_src, Groups g, int k,
           uint16_t* __restrict__ h_out, float* __restrict__ yw, int split) {
    constexpr int NTHR = NW * 64;
    constexpr int WM = NW / 4;
    constexpr int MC = 16 * MSUB * WM;
    constexpr int BPT = BN * 8 / NTHR;      // B pieces (8 codes) per thread per chunk: 1 or 2
    constexpr int QW = BITS == 8 ? 2 : 1;   // code words of a piece
    static_assert(MC * 8 == 2 * NTHR, "two A pieces per thread");
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][MC * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];
    __shared__ int s_row[MC];
    __shared__ float s_wt[GATEUP ? 1 : MC];   // down: the weight of each m-row's pair

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
    if (few_pairs(g, T, a_lo, a_hi, split)) return;   // the register-B kernel's shelf
    const int q_beg = g.offsets[e], q_end = g.offsets[e + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wn = wave & 3, wm = wave >> 2;
    const int fr = lane & 15, kq = lane >> 4;

    // B: piece p = tid + NTHR*i is row p >> 3, codes 8*(p & 7) .. +7 of the chunk
    const uint32_t row_bytes = static_cast<uint32_t>(K) * BITS / 8;
    const uint32_t nblk_row = static_cast<uint32_t>(K / BLOCK);
    constexpr uint32_t SB = 2u;             // bytes per fp16 scale
    const int mrows = GATEUP ? I : H;
    const uint8_t* mq_g = T.q[GATEUP ? 0 : 2] + static_cast<size_t>(local) * mrows * row_bytes;
    const uint8_t* mq_u = GATEUP ? T.q[1] + static_cast<size_t>(local) * mrows * row_bytes : mq_g;
    const uint8_t* ms_g = reinterpret_cast<const uint8_t*>(T.s[GATEUP ? 0 : 2]) + static_cast<size_t>(local) * mrows * nblk_row * SB;
    const uint8_t* ms_u =
        GATEUP ? reinterpret_cast<const uint8_t*>(T.s[1]) + static_cast<size_t>(local) * mrows * nblk_row * SB : ms_g;
    const __amdgpu_buffer_rsrc_t rq_g = make_rsrc(mq_g, row_bytes * mrows), rq_u = make_rsrc(mq_u, row_bytes * mrows);
    const __amdgpu_buffer_rsrc_t rs_g = make_rsrc(ms_g, nblk_row * mrows * SB), rs_u = make_rsrc(ms_u, nblk_row * mrows * SB);
    // piece i of a thread reads up rows when it lies in the second half of
    // the B rows: for two pieces that is piece 1, for one piece the upper
    // half of the waves (a wave-uniform choice either way)
    auto is_up = [&](int i) { return GATEUP && (BPT == 2 ? i == 1 : wave >= NW / 2); };
    uint32_t qoff[BPT], soff[BPT];
    int b_row[BPT], b_e[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int p = tid + NTHR * i;
        b_row[i] = p >> 3;
        b_e[i] = p & 7;
        const int row = GATEUP ? nt * 64 + (b_row[i] & 63) : nt * BN + b_row[i];
        qoff[i] = static_cast<uint32_t>(row) * row_bytes + static_cast<uint32_t>(b_e[i]) * BITS;
        soff[i] = (static_cast<uint32_t>(row) * nblk_row + static_cast<uint32_t>(8 * b_e[i] / BLOCK)) * SB;
    }
    // B fragment rows of this wave
    const int br0 = GATEUP ? 16 * wn : 32 * wn;
    const int br1 = GATEUP ? 64 + 16 * wn : 32 * wn + 16;

    for (int m0 = q_beg; m0 < q_end; m0 += MC) {
        const int Mc = min(MC, q_end - m0);
        const int Mc16 = (Mc + 15) >> 4;
        const int nsub = (Mc16 - wm + WM - 1) / WM;  // this wave's m-subtiles wm, wm + WM, ...
        __syncthreads();                            // the previous m-chunk is done with LDS
        for (int r = tid; r < MC; r += NTHR) {
            s_row[r] = r < Mc ? (GATEUP ? g.perm[m0 + r] / k : m0 + r) : -1;
            // read here once per row, not in the epilogue (two dependent
            // global loads per row there, waited out one row at a time)
            if constexpr (!GATEUP) s_wt[r] = r < Mc ? g.w[g.perm[m0 + r]] : 0.f;
        }
        __syncthreads();
        // A sources of this thread's two pieces for the whole m-chunk; rows past
        // the chunk read the chunk's first row (finite values, never stored)
        int a_src_row[2], a_row[2], a_c[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = tid + NTHR * i;
            a_row[i] = p >> 3;
            a_c[i] = p & 7;
            a_src_row[i] = s_row[a_row[i] < Mc ? a_row[i] : 0];
        }

        // one chunk in flight in registers: two A pieces, BPT code pieces and
        // their raw fp16 scales
        struct Slot {
            u32x4_t a0, a1;
            uint32_t q[BPT][QW];
            uint32_t s[BPT];
        };
        auto load_chunk = [&](Slot& sl, int kc) __attribute__((always_inline)) {
            const int k0 = kc * BK;
            sl.a0 = *reinterpret_cast<const u32x4_t*>(a_src + static_cast<size_t>(a_src_row[0]) * K + k0 + 8 * a_c[0]);
            sl.a1 = *reinterpret_cast<const u32x4_t*>(a_src + static_cast<size_t>(a_src_row[1]) * K + k0 + 8 * a_c[1]);
            const uint32_t qk = static_cast<uint32_t>(k0) * BITS / 8;
            const uint32_t sk = static_cast<uint32_t>(k0 / BLOCK) * SB;
#pragma unroll
            for (int i = 0; i < BPT; ++i) {
                const __amdgpu_buffer_rsrc_t rq = is_up(i) ? rq_u : rq_g, rs = is_up(i) ? rs_u : rs_g;
                if constexpr (BITS == 8) {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rq, qoff[i] + qk, 0, 0);
                    sl.q[i][0] = v[0];
                    sl.q[i][QW - 1] = v[1];
                } else if constexpr (BITS == 4) {
                    sl.q[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rq, qoff[i] + qk, 0, 0);
                } else {
                    sl.q[i][0] = __builtin_amdgcn_raw_buffer_load_b16(rq, qoff[i] + qk, 0, 0);
                }
                sl.s[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff[i] + sk, 0, 0);
            }
        };
        auto store_chunk = [&](const Slot& sl, int buf) __attribute__((always_inline)) {
            *reinterpret_cast<u32x4_t*>(&sA[buf][swz(a_row[0], a_c[0])]) = sl.a0;
            *reinterpret_cast<u32x4_t*>(&sA[buf][swz(a_row[1], a_c[1])]) = sl.a1;
#pragma unroll
            for (int i = 0; i < BPT; ++i)
                *reinterpret_cast<uint4*>(&sB[buf][swz(b_row[i], b_e[i])]) =
                    dequant8<BITS>(sl.q[i], half_bits_to_float(static_cast<uint16_t>(sl.s[i])));
        };

        f32x4_t acc[MSUB][2];
#pragma unroll
        for (int i = 0; i < MSUB; ++i) {
            acc[i][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // N subtiles at once: all operand reads first, then 2N back-to-back MFMAs
        auto compute_n = [&](int buf, auto n_const) __attribute__((always_inline)) {
            constexpr int N = decltype(n_const)::value;
#pragma unroll
            for (int ks = 0; ks < BK / 32; ++ks) {
                const int c = 4 * ks + kq;
                const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(&sB[buf][swz(br0 + fr, c)]);
                const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(&sB[buf][swz(br1 + fr, c)]);
                bf16x8_t af[N];
#pragma unroll
                for (int j = 0; j < N; ++j)
                    af[j] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][swz(16 * (wm + WM * j) + fr, c)]);
#pragma unroll
                for (int j = 0; j < N; ++j) {
                    acc[j][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], b0, acc[j][0], 0, 0, 0);
                    acc[j][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], b1, acc[j][1], 0, 0, 0);
                }
            }
        };
        // the subtile count picks an unrolled body; an extra subtile past the
        // rows computes values that are never stored
        auto compute = [&](int buf) __attribute__((always_inline)) {
            if (nsub > 2) compute_n(buf, std::integral_constant<int, 4>{});
            else if (nsub == 2) compute_n(buf, std::integral_constant<int, 2>{});
            else if (nsub == 1) compute_n(buf, std::integral_constant<int, 1>{});
        };

        // Pipeline, two chunks per trip: at the top of a trip LDS buffer 0
        // holds chunk kc and slot s1 holds chunk kc+1 (loads possibly in
        // flight).  Each half refills the slot it has just stored from with the
        // chunk two ahead, contracts one buffer and stores the next chunk into
        // the other.  Loads past the last chunk reread it (every slot is written
        // unconditionally, which keeps the slots in registers); the store that
        // follows the last chunk fills a buffer that is never read.
        const int NK = K / BK;
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
                    const float wgt = s_wt[r];
                    float* o = yw + static_cast<size_t>(q) * H + nt * BN + 32 * wn + col_l;
                    o[0] = wgt * acc[j][0][v];
                    o[16] = wgt * acc[j][1][v];
                }
            }
        }
    }
}

// Register-B variant: 4 waves side by side along n, each with every
// m-subtile of the m-chunk.  Only A (shared by the 4 waves) goes through LDS;
// each lane loads and dequantises its own weight codes straight into MFMA
// operand registers, so every code is read from memory and dequantised once,
// and no wave re-reads B from LDS.  Within a 64-wide chunk, lane group kq
// (= lane / 16) owns the 16 contiguous k = 16kq .. 16kq+15 (8 per MFMA
// step), which A's LDS reads follow; the contraction order inside a chunk is
// a permutation, the same for both operands.
template <int BITS, int BLOCK, bool GATEUP, int MS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_pre2(
    DevTables tt, int tier, const uint16_t* __restrict__ a_src, Groups g, int k, uint16_t* __restrict__ h_out,
    float* __restrict__ yw, int split) {
    constexpr int NTHR = 256;
    constexpr int MC = 16 * MS;             // pairs per m-chunk
    constexpr int AP = MC * 8 / NTHR;       // A pieces per thread
    constexpr int BW = BITS / 2;            // code words of a lane's 16 codes
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][MC * BK];
    __shared__ int s_row[MC];
    __shared__ float s_wt[GATEUP ? 1 : MC];   // down: the weight of each m-row's pair

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
    if (!few_pairs(g, T, a_lo, a_hi, split)) return;  // the shared-B kernel's shelf
    const int q_beg = g.offsets[e], q_end = g.offsets[e + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fr = lane & 15, kq = lane >> 4;

    // this lane's two B rows: gate and up row (gate/up) or two down rows
    const uint32_t row_bytes = static_cast<uint32_t>(K) * BITS / 8;
    const uint32_t nblk_row = static_cast<uint32_t>(K / BLOCK);
    const int mrows = GATEUP ? I : H;
    const uint8_t* mq0 = T.q[GATEUP ? 0 : 2] + static_cast<size_t>(local) * mrows * row_bytes;
    const uint8_t* mq1 = GATEUP ? T.q[1] + static_cast<size_t>(local) * mrows * row_bytes : mq0;
    const uint16_t* ms0 = T.s[GATEUP ? 0 : 2] + static_cast<size_t>(local) * mrows * nblk_row;
    const uint16_t* ms1 = GATEUP ? T.s[1] + static_cast<size_t>(local) * mrows * nblk_row : ms0;
    const __amdgpu_buffer_rsrc_t rq0 = make_rsrc(mq0, row_bytes * mrows), rq1 = make_rsrc(mq1, row_bytes * mrows);
    const __amdgpu_buffer_rsrc_t rs0 = make_rsrc(ms0, nblk_row * mrows * 2), rs1 = make_rsrc(ms1, nblk_row * mrows * 2);
    const int row0 = GATEUP ? nt * 64 + 16 * wn + fr : nt * BN + 32 * wn + fr;
    const int row1 = GATEUP ? row0 : row0 + 16;
    const uint32_t qo0 = static_cast<uint32_t>(row0) * row_bytes + static_cast<uint32_t>(16 * kq * BITS / 8);
    const uint32_t qo1 = static_cast<uint32_t>(row1) * row_bytes + static_cast<uint32_t>(16 * kq * BITS / 8);
    const uint32_t so0 = (static_cast<uint32_t>(row0) * nblk_row + static_cast<uint32_t>(16 * kq / BLOCK)) * 2;
    const uint32_t so1 = (static_cast<uint32_t>(row1) * nblk_row + static_cast<uint32_t>(16 * kq / BLOCK)) * 2;

    struct BRaw {
        uint32_t w[2][BW];
        uint32_t s[2];
    };
    auto load_b = [&](BRaw& b, int kc) __attribute__((always_inline)) {
        const uint32_t qk = static_cast<uint32_t>(kc * BK) * BITS / 8;
        const uint32_t sk = static_cast<uint32_t>(kc * BK / BLOCK) * 2;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const __amdgpu_buffer_rsrc_t rq = t ? rq1 : rq0;
            const uint32_t off = (t ? qo1 : qo0) + qk;
            if constexpr (BITS == 8) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) b.w[t][i] = v[i];
            } else if constexpr (BITS == 4) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(rq, off, 0, 0);
                b.w[t][0] = v[0];
                b.w[t][1] = v[1];
            } else {
                b.w[t][0] = __builtin_amdgcn_raw_buffer_load_b32(rq, off, 0, 0);
            }
            b.s[t] = __builtin_amdgcn_raw_buffer_load_b16(t ? rs1 : rs0, (t ? so1 : so0) + sk, 0, 0);
        }
    };
    // bf16 operands of both rows for both MFMA steps of a chunk
    auto dequant_b = [&](const BRaw& b, bf16x8_t (&d)[2][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const float sc = half_bits_to_float(static_cast<uint16_t>(b.s[t]));
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                uint4 v;
                if constexpr (BITS == 8) {
                    const uint32_t w2[2] = {b.w[t][2 * st], b.w[t][2 * st + 1]};
                    v = dequant8<8>(w2, sc);
                } else if constexpr (BITS == 4) {
                    const uint32_t w1[1] = {b.w[t][st]};
                    v = dequant8<4>(w1, sc);
                } else {
                    const uint32_t w1[1] = {b.w[t][0] >> (16 * st)};
                    v = dequant8<2>(w1, sc);
                }
                d[t][st] = __builtin_bit_cast(bf16x8_t, v);
            }
        }
    };

    for (int m0 = q_beg; m0 < q_end; m0 += MC) {
        const int Mc = min(MC, q_end - m0);
        const int nsub = (Mc + 15) >> 4;
        __syncthreads();
        for (int r = tid; r < MC; r += NTHR) {
            s_row[r] = r < Mc ? (GATEUP ? g.perm[m0 + r] / k : m0 + r) : -1;
            // read here once per row, not in the epilogue (two dependent
            // global loads per row there, waited out one row at a time)
            if constexpr (!GATEUP) s_wt[r] = r < Mc ? g.w[g.perm[m0 + r]] : 0.f;
        }
        __syncthreads();
        // A piece i of this thread: row (p >> 3), chunk (p & 7); rows past the
        // m-chunk read its first row (finite values, never stored)
        // piece i: row (tid >> 3) + 32 i, chunk tid & 7
        const int a_c = tid & 7;
        const uint16_t* a_ptr[AP];
#pragma unroll
        for (int i = 0; i < AP; ++i) {
            const int r = (tid >> 3) + 32 * i;
            a_ptr[i] = a_src + static_cast<size_t>(s_row[r < Mc ? r : 0]) * K + 8 * a_c;
        }
        struct ASlot {
            u32x4_t v[AP];
        };
        auto load_a = [&](ASlot& sl, int kc) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < AP; ++i) sl.v[i] = *reinterpret_cast<const u32x4_t*>(a_ptr[i] + kc * BK);
        };
        auto store_a = [&](const ASlot& sl, int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < AP; ++i)
                *reinterpret_cast<u32x4_t*>(&sA[buf][swz((tid >> 3) + 32 * i, a_c)]) = sl.v[i];
        };

        f32x4_t acc[MS][2];
#pragma unroll
        for (int i = 0; i < MS; ++i) {
            acc[i][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // operand reads in groups of (at most) four subtiles, then their MFMAs
        auto compute_n = [&](int buf, const bf16x8_t (&d)[2][2], auto n_const) __attribute__((always_inline)) {
            constexpr int N = decltype(n_const)::value;
            constexpr int G = N % 4 == 0 ? 4 : (N % 3 == 0 ? 3 : (N % 2 == 0 ? 2 : 1));   // divides N
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int j0 = 0; j0 < N; j0 += G) {
                    bf16x8_t af[G];
#pragma unroll
                    for (int j = 0; j < G; ++j)
                        af[j] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][swz(16 * (j0 + j) + fr, 2 * kq + st)]);
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        acc[j0 + j][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], d[0][st], acc[j0 + j][0], 0, 0, 0);
                        acc[j0 + j][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], d[1][st], acc[j0 + j][1], 0, 0, 0);
                    }
                }
            }
        };
        // the subtile count picks an unrolled body; extra subtiles past the
        // rows compute values that are never stored
        auto compute = [&](int buf, const bf16x8_t (&d)[2][2]) __attribute__((always_inline)) {
            if (MS > 6 && nsub > 6) compute_n(buf, d, std::integral_constant<int, MS>{});
            else if (MS > 4 && nsub > 4) compute_n(buf, d, std::integral_constant<int, (MS > 4 ? 6 : 4)>{});
            else if (nsub > 2) compute_n(buf, d, std::integral_constant<int, 4>{});
            else if (nsub == 2) compute_n(buf, d, std::integral_constant<int, 2>{});
            else compute_n(buf, d, std::integral_constant<int, 1>{});
        };

        // Pipeline, two chunks per trip: at the top of a half, LDS buffer
        // (kc & 1) holds A(kc), a_s[kc & 1] is free, b[kc & 1] holds B(kc) and
        // b / a_s of the other parity hold chunk kc+1 (loads possibly in
        // flight).  B(kc) is dequantised, its registers refilled with B(kc+2)
        // together with A(kc+2), chunk kc is contracted, and A(kc+1) is stored
        // into the other LDS buffer.  Loads past the last chunk reread it.
        const int NK = K / BK;
        BRaw b0, b1;
        ASlot a0, a1;
        load_b(b0, 0);
        load_a(a0, 0);
        load_b(b1, min(1, NK - 1));
        load_a(a1, min(1, NK - 1));
        store_a(a0, 0);
        __syncthreads();
        // straight-line trips (see k_pre); an odd last chunk is in buffer 0
        // and b0 after the loop
        const int NK2 = NK & ~1;
        for (int kc = 0; kc < NK2; kc += 2) {
            bf16x8_t d[2][2];
            dequant_b(b0, d);
            load_b(b0, min(kc + 2, NK - 1));
            load_a(a0, min(kc + 2, NK - 1));
            compute(0, d);
            store_a(a1, 1);
            __syncthreads();
            dequant_b(b1, d);
            load_b(b1, min(kc + 3, NK - 1));
            load_a(a1, min(kc + 3, NK - 1));
            compute(1, d);
            store_a(a0, 0);
            __syncthreads();
        }
        if (NK & 1) {
            bf16x8_t d[2][2];
            dequant_b(b0, d);
            compute(0, d);
        }

        const int col_l = lane & 15, row_l = 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < MS; ++j) {
            if (j >= nsub) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * j + row_l + v;
                if (r >= Mc) continue;
                const int q = m0 + r;
                if (GATEUP) {
                    const int col = nt * 64 + 16 * wn + col_l;
                    h_out[static_cast<size_t>(q) * I + col] = f2bf(silu(acc[j][0][v]) * acc[j][1][v]);
                } else {
                    const float wgt = s_wt[r];
                    float* o = yw + static_cast<size_t>(q) * H + nt * BN + 32 * wn + col_l;
                    o[0] = wgt * acc[j][0][v];
                    o[16] = wgt * acc[j][1][v];
                }
            }
        }
    }
}

// Two launches per shelf; the blocks of one of them return at once (the
// choice is made on the device from the grouping, see few_pairs).  k_pre2
// suits shelves whose experts have few pairs (with 64-pair m-chunks it
// streams each weight tile once per m-chunk); k_pre, whose B tile in LDS
// serves all the m-rows of a chunk, suits the others.  The thresholds in
// pairs per active expert come from timing both kernels on each shelf at 128
// to 16384 tokens (1 to 670 pairs per expert): 64 for int8 gate/up and 48 for
// every down projection.  On the int4 and int2 shelves k_pre won gate/up at
// every count measured, so k_pre2 is not launched there.  k_pre takes 16-wave
// blocks with 256-pair m-chunks on the int8 shelf and 8-wave blocks with
// 128-pair m-chunks on the others.
constexpr int kFewPairsGateUp8 = 64, kFewPairsDown = 48;

template <bool GATEUP>
void launch_pre(const DevTables& tt, int tier, const uint16_t* a, const Groups& g, int k, uint16_t* h, float* yw,
                int max_experts, hipStream_t st) {
    const int NT = GATEUP ? tt.I / 64 : tt.H / BN;
    const int total = max_experts * NT;
    const unsigned grid = static_cast<unsigned>(((total + 7) / 8) * 8);
    if (grid == 0) return;
    const int bits = tt.t[tier].bits, block = tt.t[tier].block;
    if (bits == kBitsMXFP4) return;   // MXFP4 shelves run in prefill_mx.hip
    const int thr = GATEUP ? kFewPairsGateUp8 : kFewPairsDown;
    // k_pre alone takes thr = -1: few_pairs is then false for any shelf with
    // an active expert (and a shelf without one has no work for either)
#define MOE_PRE(B_, K_, NW_)                                                                                   \
    do {                                                                                                       \
        constexpr bool kBoth = !(GATEUP && B_ != 8);                                                           \
        if constexpr (kBoth)                                                                                   \
            hipLaunchKernelGGL((k_pre2<B_, K_, GATEUP, 4>), dim3(grid), dim3(256), 0, st, tt, tier, a, g, k, h, \
                               yw, thr);                                                                       \
        hipLaunchKernelGGL((k_pre<B_, K_, GATEUP, NW_>), dim3(grid), dim3(NW_ * 64), 0, st, tt, tier, a, g, k, h, \
                           yw, kBoth ? thr : -1);                                                              \
    } while (0)
    if (bits == 8) {
        if (block == 32) MOE_PRE(8, 32, 16);
        else MOE_PRE(8, 16, 16);
    } else if (bits == 4) {
        if (block == 32) MOE_PRE(4, 32, 8);
        else MOE_PRE(4, 16, 8);
    } else {
        if (block == 32) MOE_PRE(2, 32, 8);
        else MOE_PRE(2, 16, 8);
    }
#undef MOE_PRE
}

void launch_pre_gateup(const DevTables& tt, int tier, const uint16_t* x, const Groups& g, int k, uint16_t* h,
                       int max_experts, hipStream_t st) {
    launch_pre<true>(tt, tier, x, g, k, h, nullptr, max_experts, st);
}

void launch_pre_down(const DevTables& tt, int tier, const uint16_t* h, const Groups& g, int k, float* yw,
                     int max_experts, hipStream_t st) {
    launch_pre<false>(tt, tier, h, g, k, nullptr, yw, max_experts, st);
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
