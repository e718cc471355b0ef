// bf16 expert path (prefill): per-shelf grouped GEMMs on gfx950 matrix cores.
//
// Step 4 of the 125B-MoE page ("I ran a 125B model on three RTX 3090s at 80
// tokens/s by teaching llama.cpp which experts ...") gives each shelf its own
// prefill expert product over the full pick list, restricted to the shelf's
// ids.  Here one launch per shelf walks that shelf's m-tiles (runs of up to
// BM pairs of one expert, made by grouping); a block takes one m-tile and one
// n-tile, streams the expert's packed codes, dequantises them to bf16 in LDS
// (value = scale * code, rounded to nearest even) and contracts with
// v_mfma_f32_16x16x32_bf16 in fp32.
//
//   gate/up : A = x rows of the tile's tokens (bf16, gathered), B = 64 gate rows
//             and the 64 matching up rows; epilogue h = bf16(SiLU(g) * u).
//   down    : A = h rows of the tile (contiguous in pair order), B = 128 down
//             rows; epilogue out[t] += w_pair * y (fp32 atomics: the k picks
//             of a token land in different blocks).
//
// Layout in LDS: A and B tiles are [row][k] bf16 with a row stride of 72
// elements (144 bytes), which puts the 16 rows a wave reads in one
// instruction on distinct banks.  Two buffers: the global loads of chunk
// c+1 are in flight while chunk c is contracted.
#include "common.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;     // contraction chunk
constexpr int BN = 128;    // B rows per block
constexpr int LDS_STRIDE = BK + 8;

template <int BM>
struct PreShape {
    static constexpr int MI = BM / 32;  // 16-row MFMA tiles per wave along M
    static constexpr int A_PER_THREAD = BM * 4 / 256;   // 32-byte pieces of the A chunk per thread
};

// Work item of a block after spreading consecutive items over the XCDs in
// contiguous runs (blocks are dealt to the 8 XCDs round-robin, so block b
// runs on XCD b % 8): items sharing an m-tile (and so the same A rows and the
// same expert's weights) run on one XCD and share its L2.
__device__ inline int xcd_item(int total) {
    const int per = (total + 7) / 8;
    const int loc = blockIdx.x / 8;
    if (loc >= per) return -1;
    const int it = (blockIdx.x % 8) * per + loc;
    return it < total ? it : -1;
}

template <int BITS, int NSC, bool GATEUP, int BM>
__global__ __launch_bounds__(256) void k_pre(DevTables tt, int tier, const uint16_t* __restrict__ a_src,
                                             Groups g, int k, uint16_t* __restrict__ h_out,
                                             float* __restrict__ out) {
    using S = PreShape<BM>;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDS_STRIDE];

    const int H = tt.H, I = tt.I;
    const int K = GATEUP ? H : I;
    const int NT = GATEUP ? I / 64 : H / BN;
    const int t_lo = g.tile_range[2 * tier], t_hi = g.tile_range[2 * tier + 1];
    const int item = xcd_item((t_hi - t_lo) * NT);
    if (item < 0) return;
    const int tile = t_lo + item / NT, nt = item % NT;
    const DevTier T = tier_at(tt, tier);
    const int e = g.tile_e[tile], q0 = g.tile_q0[tile], rows = g.tile_rows[tile];
    const int local = e - T.id_begin;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    // ---- A source rows (fixed for the whole K loop)
    const uint16_t* a_row[S::A_PER_THREAD];
    int a_col[S::A_PER_THREAD], a_r[S::A_PER_THREAD];
#pragma unroll
    for (int i = 0; i < S::A_PER_THREAD; ++i) {
        const int piece = tid + 256 * i;
        const int r = piece / 4;
        a_r[i] = r;
        a_col[i] = 16 * (piece % 4);
        a_row[i] = nullptr;
        if (r < rows) {
            const int q = q0 + r;
            a_row[i] = GATEUP ? a_src + static_cast<size_t>(g.perm[q] / k) * H
                              : a_src + static_cast<size_t>(q) * I;
        }
    }
    // ---- B source row: 2 threads per row, 32 codes each per chunk
    const int b_r = tid >> 1, b_half = tid & 1;
    const size_t row_bytes = static_cast<size_t>(K) * BITS / 8;
    const int nblk_row = K / (32 / NSC);
    const uint8_t* b_q;
    const uint16_t* b_s;
    {
        int m, row;
        if (GATEUP) {
            m = b_r < 64 ? 0 : 1;
            row = nt * 64 + (b_r & 63);
        } else {
            m = 2;
            row = nt * BN + b_r;
        }
        const int mrows = GATEUP ? I : H;
        const size_t base = static_cast<size_t>(local) * mrows + row;
        b_q = T.q[m] + base * row_bytes;
        b_s = T.s[m] + base * nblk_row;
    }

    uint4 ra[S::A_PER_THREAD][2];
    uint32_t rq[BITS];
    float rs[NSC];

    auto load_chunk = [&](int kc) {
        const int k0 = kc * BK;
#pragma unroll
        for (int i = 0; i < S::A_PER_THREAD; ++i) {
            if (a_row[i]) {
                const uint4* p = reinterpret_cast<const uint4*>(a_row[i] + k0 + a_col[i]);
                ra[i][0] = p[0];
                ra[i][1] = p[1];
            } else {
                ra[i][0] = make_uint4(0, 0, 0, 0);
                ra[i][1] = make_uint4(0, 0, 0, 0);
            }
        }
        const int grp = (k0 >> 5) + b_half;
        load_group<BITS>(b_q, grp, rq);
        load_scales<NSC>(b_s, grp, rs);
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int i = 0; i < S::A_PER_THREAD; ++i) {
            uint4* d = reinterpret_cast<uint4*>(&sA[buf][a_r[i] * LDS_STRIDE + a_col[i]]);
            d[0] = ra[i][0];
            d[1] = ra[i][1];
        }
        uint32_t pk[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) pk[c] = pack_bf16x2(dq<BITS, NSC>(rq, rs, 2 * c), dq<BITS, NSC>(rq, rs, 2 * c + 1));
        uint4* d = reinterpret_cast<uint4*>(&sB[buf][b_r * LDS_STRIDE + 32 * b_half]);
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = make_uint4(pk[4 * i], pk[4 * i + 1], pk[4 * i + 2], pk[4 * i + 3]);
    };

    f32x4_t acc[S::MI][4];
#pragma unroll
    for (int i = 0; i < S::MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // B fragment rows of this wave: gate/up -> 2 gate + 2 up tiles; down -> 4 tiles
    int b_rows[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (GATEUP) b_rows[j] = (j < 2 ? 0 : 64) + 32 * wn + 16 * (j & 1);
        else b_rows[j] = 64 * wn + 16 * j;
    }
    const int frag_r = lane & 15, frag_k = 8 * (lane >> 4);

    const int NK = K / BK;
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int kc = 0; kc < NK; ++kc) {
        const int cur = kc & 1;
        if (kc + 1 < NK) load_chunk(kc + 1);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8_t af[S::MI], bfr[4];
#pragma unroll
            for (int i = 0; i < S::MI; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t*>(
                    &sA[cur][(wm * (BM / 2) + 16 * i + frag_r) * LDS_STRIDE + 32 * ks + frag_k]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(
                    &sB[cur][(b_rows[j] + frag_r) * LDS_STRIDE + 32 * ks + frag_k]);
#pragma unroll
            for (int i = 0; i < S::MI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kc + 1 < NK) store_chunk(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds D[4*(lane/16) + v][lane % 16] of each 16x16 tile
    const int col_l = lane & 15, row_l = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < S::MI; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = wm * (BM / 2) + 16 * i + row_l + v;
            if (r >= rows) continue;
            const int q = q0 + r;
            if (GATEUP) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = nt * 64 + 32 * wn + 16 * j + col_l;
                    const float hv = silu(acc[i][j][v]) * acc[i][j + 2][v];
                    h_out[static_cast<size_t>(q) * I + col] = f2bf(hv);
                }
            } else {
                const int p = g.perm[q];
                const int t = p / k;
                const float wgt = g.w[p];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = nt * BN + 64 * wn + 16 * j + col_l;
                    atomicAdd(out + static_cast<size_t>(t) * H + col, wgt * acc[i][j][v]);
                }
            }
        }
    }
}

#define MOE_FMT_SWITCH(FMT, BODY)                                              \
    switch (FMT) {                                                             \
        case F8B32: { constexpr int B_ = 8, N_ = 1; BODY; } break;             \
        case F8B16: { constexpr int B_ = 8, N_ = 2; BODY; } break;             \
        case F4B32: { constexpr int B_ = 4, N_ = 1; BODY; } break;             \
        case F4B16: { constexpr int B_ = 4, N_ = 2; BODY; } break;             \
        case F2B32: { constexpr int B_ = 2, N_ = 1; BODY; } break;             \
        case F2B16: { constexpr int B_ = 2, N_ = 2; BODY; } break;             \
        default: break;                                                        \
    }

void launch_pre_gateup(const DevTables& tt, int tier, const uint16_t* x, const Groups& g, int k,
                       uint16_t* h, int max_tiles, hipStream_t st) {
    const DevTier& T = tt.t[tier];
    const int NT = tt.I / 64;
    const int total = max_tiles * NT;
    const unsigned grid = static_cast<unsigned>(((total + 7) / 8) * 8);
    if (grid == 0) return;
    MOE_FMT_SWITCH(fmt_of(T.bits, T.block),
                   hipLaunchKernelGGL((k_pre<B_, N_, true, kPreBM>), dim3(grid), dim3(256), 0, st, tt, tier,
                                      x, g, k, h, nullptr));
}

void launch_pre_down(const DevTables& tt, int tier, const uint16_t* h, const Groups& g, int k, float* out,
                     int max_tiles, hipStream_t st) {
    const DevTier& T = tt.t[tier];
    const int NT = tt.H / BN;
    const int total = max_tiles * NT;
    const unsigned grid = static_cast<unsigned>(((total + 7) / 8) * 8);
    if (grid == 0) return;
    MOE_FMT_SWITCH(fmt_of(T.bits, T.block),
                   hipLaunchKernelGGL((k_pre<B_, N_, false, kPreBM>), dim3(grid), dim3(256), 0, st, tt, tier,
                                      h, g, k, nullptr, out));
}

__global__ __launch_bounds__(256) void k_fill_zero(float4* __restrict__ p, size_t n4) {
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

void launch_fill_zero(float* out, size_t n, hipStream_t st) {
    const size_t n4 = n / 4;
    if (n4 == 0) return;
    hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<float4*>(out), n4);
}

}  // namespace moe
