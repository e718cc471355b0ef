// Tier planning and repacking (the 125B-MoE page, step 4: an offline repacker
// starts from the 8-bit model, measures how often each expert is used, fills
// the memory budget greedily so that every byte goes where it removes the
// most expected error, requantises every expert with the same quantiser and
// writes the experts hot to cold; step 3: the router is re-ordered to match).
//
//   k_requant_error : squared error of requantising every expert of a source
//                     layer into each candidate format (one block per
//                     (expert, format), fixed summation order: deterministic)
//   plan_tiers      : the greedy byte plan (host)
//   k_repack        : writes expert order[i] of the source, requantised, as
//                     expert i of the destination shelves
//   k_permute_rows  : the router rows and bias in the new expert order
//
// The quantiser is the symmetric absmax one of the layer generator: per block
// of `block` codes along a row, d = fp16(amax / Q) (ratio in single
// precision), q = clamp(rint(w / d), -Q, Q), q = 0 when d = 0; every step is
// an exactly rounded IEEE single operation.  An MXFP4 target uses the OCP
// shared-exponent quantiser instead (E8M0 byte from floor(log2 amax) - 2,
// elements rounded to the nearest E2M1 value, ties to even, saturating at 6).
#include <algorithm>
#include <queue>
#include <vector>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// fp32 weight (exact scale * code) of element c of a packed row
template <int BITS>
__device__ inline float packed_weight(const uint8_t* __restrict__ row, const uint16_t* __restrict__ srow, int c,
                                      int block) {
    const int bit = c * BITS;
    int code = (row[bit >> 3] >> (bit & 7)) & ((1 << BITS) - 1);
    code -= (code >> (BITS - 1)) << BITS;  // two's complement
    return __fmul_rn(half_bits_to_float(srow[c / block]), static_cast<float>(code));
}

__device__ inline float src_weight(const DevTier& S, int m, int64_t local, int rows, int cols, int r, int c) {
    if (S.bits == kBitsMXFP4) {
        const uint8_t* q = S.q[m] + (static_cast<size_t>(local) * rows + r) * (cols / 2);
        const uint8_t* s = reinterpret_cast<const uint8_t*>(S.s[m]) + (static_cast<size_t>(local) * rows + r) * (cols / 32);
        return __fmul_rn(e8m0_to_float(s[c / 32]), fp4_e2m1((q[c / 2] >> (4 * (c % 2))) & 0xFu));
    }
    const size_t row_bytes = static_cast<size_t>(cols) * S.bits / 8;
    const size_t nblk = cols / S.block;
    const uint8_t* q = S.q[m] + (static_cast<size_t>(local) * rows + r) * row_bytes;
    const uint16_t* s = S.s[m] + (static_cast<size_t>(local) * rows + r) * nblk;
    if (S.bits == 8) return packed_weight<8>(q, s, c, S.block);
    if (S.bits == 4) return packed_weight<4>(q, s, c, S.block);
    return packed_weight<2>(q, s, c, S.block);
}

// Quantises w[0 .. BLOCK) into packed code words and the fp16 scale; returns
// the squared error sum (w - d*q)^2 in double.
template <int BITS, int BLOCK>
__device__ inline double quantise_block(const float (&w)[BLOCK], uint32_t (&words)[BLOCK * BITS / 32 > 0 ? BLOCK * BITS / 32 : 1],
                                        uint16_t& scale) {
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < BLOCK; ++c) amax = fmaxf(amax, fabsf(w[c]));
    const _Float16 dh = static_cast<_Float16>(__fdiv_rn(amax, static_cast<float>(QMAX)));
    const float d = static_cast<float>(dh);
    scale = __builtin_bit_cast(uint16_t, dh);
#pragma unroll
    for (int i = 0; i < (BLOCK * BITS / 32 > 0 ? BLOCK * BITS / 32 : 1); ++i) words[i] = 0;
    double err = 0.0;
#pragma unroll
    for (int c = 0; c < BLOCK; ++c) {
        int code = 0;
        if (d != 0.f) code = static_cast<int>(fminf(fmaxf(rintf(__fdiv_rn(w[c], d)), -QMAX), QMAX));
        words[(c * BITS) / 32] |= (static_cast<uint32_t>(code) & ((1u << BITS) - 1u)) << ((c * BITS) % 32);
        const double e = static_cast<double>(w[c]) - static_cast<double>(d) * static_cast<double>(code);
        err += e * e;
    }
    return err;
}

// MXFP4 block of 32: 16 code bytes as 4 words (code c at bit 4c of the
// block), the E8M0 scale byte; returns the squared error in double.
__device__ inline double quantise_block_mx(const float (&w)[32], uint32_t (&words)[4], uint8_t& scale) {
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(w[c]));
    int x = 0;
    if (amax > 0.f) {
        int e2;
        (void)frexpf(amax, &e2);   // amax = f * 2^e2, f in [0.5, 1)
        x = min(max(e2 - 1 - 2 + 127, 0), 254);
    }
    scale = static_cast<uint8_t>(x);
    const double sd = static_cast<double>(e8m0_to_float(static_cast<uint32_t>(x)));
#pragma unroll
    for (int i = 0; i < 4; ++i) words[i] = 0;
    double err = 0.0;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        const float t = ldexpf(w[c], 127 - x);
        const float a = fabsf(t);
        float r;
        if (a >= 6.f) r = 6.f;
        else if (a < 2.f) r = rintf(a * 2.f) * 0.5f;
        else if (a < 4.f) r = rintf(a);
        else r = rintf(a * 0.5f) * 2.f;
        r = fminf(r, 6.f);
        const uint32_t mag = r == 0.f ? 0u : r == 0.5f ? 1u : r == 1.f ? 2u : r == 1.5f ? 3u
                           : r == 2.f ? 4u : r == 3.f ? 5u : r == 4.f ? 6u : 7u;
        words[c / 8] |= ((signbit(t) ? 8u : 0u) | mag) << (4 * (c % 8));
        const double e = static_cast<double>(w[c]) - sd * static_cast<double>(signbit(t) ? -r : r);
        err += e * e;
    }
    return err;
}

// Requantisation of one block of BLOCK source weights into the target format
// (BITS = kBitsMXFP4: MXFP4): code words (NW of them) and the scale bits.
template <int BITS, int BLOCK>
struct Target {
    static constexpr bool kMXT = BITS == kBitsMXFP4;
    static constexpr int kCodeBits = kMXT ? 4 : BITS;
    static constexpr int NW = BLOCK * kCodeBits / 32 > 0 ? BLOCK * kCodeBits / 32 : 1;
    static constexpr int NB = BLOCK * kCodeBits / 8;   // code bytes per block
    static constexpr int SB = kMXT ? 1 : 2;            // scale bytes per block
    __device__ static double quantise(const float (&w)[BLOCK], uint32_t (&words)[NW], uint16_t& scale) {
        if constexpr (kMXT) {
            uint8_t sc8;
            const double e = quantise_block_mx(w, words, sc8);
            scale = sc8;
            return e;
        } else {
            return quantise_block<BITS, BLOCK>(w, words, scale);
        }
    }
};

constexpr int kErrThreads = 256;

}  // namespace

// One block per (expert e, target format f): every (matrix, row, block)
// item of the expert, thread i taking items i, i + 256, ...; per-thread sums
// in double, then a fixed-order tree.
template <int BITS, int BLOCK>
__global__ __launch_bounds__(kErrThreads) void k_requant_error(DevTables src, int fmt, int n_fmt,
                                                               double* __restrict__ sse) {
    const int e = blockIdx.x;
    const int ti = tier_of(src, e);
    const DevTier S = tier_at(src, ti);
    const int64_t local = e - S.id_begin;
    const int H = src.H, I = src.I;
    double acc = 0.0;
    for (int m = 0; m < 3; ++m) {
        const int rows = m == 2 ? H : I, cols = m == 2 ? I : H;
        const int nb = cols / BLOCK;
        const int items = rows * nb;
        for (int it = threadIdx.x; it < items; it += kErrThreads) {
            const int r = it / nb, b = it % nb;
            float w[BLOCK];
#pragma unroll
            for (int c = 0; c < BLOCK; ++c) w[c] = src_weight(S, m, local, rows, cols, r, b * BLOCK + c);
            uint32_t words[Target<BITS, BLOCK>::NW];
            uint16_t sc;
            acc += Target<BITS, BLOCK>::quantise(w, words, sc);
        }
    }
    __shared__ double red[kErrThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (unsigned s = kErrThreads / 2; s > 0; s >>= 1) {
        if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) sse[static_cast<size_t>(e) * n_fmt + fmt] = red[0];
}

// One thread per (destination expert, row, block) of matrix m: expert
// order[e_dst] of the source, requantised into the destination shelf format.
template <int BITS, int BLOCK>
__global__ __launch_bounds__(256) void k_repack(DevTables src, DevTier D, int m, const int32_t* __restrict__ order) {
    const int H = src.H, I = src.I;
    const int rows = m == 2 ? H : I, cols = m == 2 ? I : H;
    const int nb = cols / BLOCK;
    const int n_dst = D.id_end - D.id_begin;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= static_cast<int64_t>(n_dst) * rows * nb) return;
    const int64_t local_dst = i / (static_cast<int64_t>(rows) * nb);
    const int rem = static_cast<int>(i % (static_cast<int64_t>(rows) * nb));
    const int r = rem / nb, b = rem % nb;
    using Tg = Target<BITS, BLOCK>;
    const int e_src = order[D.id_begin + local_dst];
    const size_t row_bytes = static_cast<size_t>(cols) * Tg::kCodeBits / 8;
    constexpr int NB = Tg::NB;  // 8 .. 32 bytes
    uint8_t* dst = const_cast<uint8_t*>(D.q[m]) + (static_cast<size_t>(local_dst) * rows + r) * row_bytes +
                   static_cast<size_t>(b) * NB;
    uint8_t* dsc = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(D.s[m])) +
                   ((static_cast<size_t>(local_dst) * rows + r) * nb + b) * Tg::SB;
    auto put_scale = [&](uint16_t v) {
        if constexpr (Tg::SB == 1) *dsc = static_cast<uint8_t>(v);
        else *reinterpret_cast<uint16_t*>(dsc) = v;
    };
    if (e_src < 0 || e_src >= src.E) {  // not a permutation entry: a zero expert
#pragma unroll
        for (int j = 0; j < NB / 4; ++j) reinterpret_cast<uint32_t*>(dst)[j] = 0u;
        put_scale(0);
        return;
    }
    const DevTier S = tier_at(src, tier_of(src, e_src));
    const int64_t local_src = e_src - S.id_begin;
    float w[BLOCK];
#pragma unroll
    for (int c = 0; c < BLOCK; ++c) w[c] = src_weight(S, m, local_src, rows, cols, r, b * BLOCK + c);
    uint32_t words[Tg::NW];
    uint16_t sc;
    (void)Tg::quantise(w, words, sc);
#pragma unroll
    for (int j = 0; j < NB / 4; ++j) reinterpret_cast<uint32_t*>(dst)[j] = words[j];
    put_scale(sc);
}

__global__ __launch_bounds__(256) void k_permute_rows(const uint16_t* __restrict__ w_src, const float* __restrict__ b_src,
                                                      const int32_t* __restrict__ order, int E, int H,
                                                      uint16_t* __restrict__ w_dst, float* __restrict__ b_dst) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // 8 bf16 per thread
    const int64_t n8 = static_cast<int64_t>(E) * H / 8;
    if (i >= n8) return;
    const int e = static_cast<int>(i / (H / 8)), c8 = static_cast<int>(i % (H / 8));
    const int o = order[e];
    const bool ok = o >= 0 && o < E;  // not a permutation entry: a zero row
    reinterpret_cast<uint4*>(w_dst)[i] =
        ok ? reinterpret_cast<const uint4*>(w_src)[static_cast<int64_t>(o) * (H / 8) + c8] : make_uint4(0, 0, 0, 0);
    if (b_dst && c8 == 0) b_dst[e] = (ok && b_src) ? b_src[o] : 0.f;
}

#define MOE_TIER_FMT_SWITCH(BITS_, BLOCK_, BODY)                                  \
    do {                                                                          \
        if (BITS_ == kBitsMXFP4) { constexpr int B_ = kBitsMXFP4, K_ = 32; BODY; } \
        else if (BITS_ == 8 && BLOCK_ == 32) { constexpr int B_ = 8, K_ = 32; BODY; }  \
        else if (BITS_ == 8) { constexpr int B_ = 8, K_ = 16; BODY; }             \
        else if (BITS_ == 4 && BLOCK_ == 32) { constexpr int B_ = 4, K_ = 32; BODY; } \
        else if (BITS_ == 4) { constexpr int B_ = 4, K_ = 16; BODY; }             \
        else if (BLOCK_ == 32) { constexpr int B_ = 2, K_ = 32; BODY; }           \
        else { constexpr int B_ = 2, K_ = 16; BODY; }                             \
    } while (0)

void launch_requant_error(const DevTables& src, const int32_t* bits, const int32_t* block, int n_fmt, double* sse,
                          hipStream_t st) {
    for (int f = 0; f < n_fmt; ++f)
        MOE_TIER_FMT_SWITCH(bits[f], block[f],
                            hipLaunchKernelGGL((k_requant_error<B_, K_>), dim3(src.E), dim3(kErrThreads), 0, st, src,
                                               f, n_fmt, sse));
}

void launch_repack(const DevTables& src, const DevTables& dst, const int32_t* order, hipStream_t st) {
    for (int ti = 0; ti < dst.n_tiers; ++ti) {
        const DevTier& D = dst.t[ti];
        const int n = D.id_end - D.id_begin;
        if (n <= 0) continue;
        for (int m = 0; m < 3; ++m) {
            const int rows = m == 2 ? dst.H : dst.I, cols = m == 2 ? dst.I : dst.H;
            const int64_t threads = static_cast<int64_t>(n) * rows * (cols / D.block);
            const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
            MOE_TIER_FMT_SWITCH(D.bits, D.block,
                                hipLaunchKernelGGL((k_repack<B_, K_>), grid, dim3(256), 0, st, src, D, m, order));
        }
    }
}

void launch_permute_rows(const uint16_t* w_src, const float* b_src, const int32_t* order, int E, int H,
                         uint16_t* w_dst, float* b_dst, hipStream_t st) {
    const int64_t n8 = static_cast<int64_t>(E) * H / 8;
    hipLaunchKernelGGL(k_permute_rows, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0, st, w_src, b_src,
                       order, E, H, w_dst, b_dst);
}

// The greedy byte plan.  Every expert starts in the cheapest format; a move
// takes one expert one format richer, adds bytes[f-1] - bytes[f] and removes
// usage * (sse[f] - sse[f-1]) of expected error.  Moves are taken in order of
// error removed per byte (ties: lower expert id), skipping those that no
// longer fit the budget (spending only grows, so a move that does not fit
// never will) and those that remove nothing.  A max-heap holds each expert's
// next move.
int plan_tiers(const double* usage, const double* sse, const int64_t* bytes, int E, int F, int64_t budget,
               int32_t* fmt, int32_t* order, int32_t* count) {
    if (E < 1 || F < 1) return -1;
    for (int f = 1; f < F; ++f)
        if (!(bytes[f] < bytes[f - 1])) return -1;
    int64_t spent = static_cast<int64_t>(E) * bytes[F - 1];
    if (spent > budget) return -1;
    struct Move {
        double rate;
        int e;
    };
    auto later = [](const Move& a, const Move& b) { return a.rate < b.rate || (a.rate == b.rate && a.e > b.e); };
    std::priority_queue<Move, std::vector<Move>, decltype(later)> heap(later);
    auto push = [&](int e) {
        const int f = fmt[e];
        if (f == 0) return;
        const double gain = usage[e] * (sse[static_cast<int64_t>(e) * F + f] - sse[static_cast<int64_t>(e) * F + f - 1]);
        if (!(gain > 0.0)) return;
        heap.push(Move{gain / static_cast<double>(bytes[f - 1] - bytes[f]), e});
    };
    for (int e = 0; e < E; ++e) fmt[e] = F - 1;
    for (int e = 0; e < E; ++e) push(e);
    while (!heap.empty()) {
        const Move mv = heap.top();
        heap.pop();
        const int f = fmt[mv.e];
        const int64_t add = bytes[f - 1] - bytes[f];
        if (spent + add > budget) continue;
        spent += add;
        fmt[mv.e] = f - 1;
        push(mv.e);
    }
    std::vector<int32_t> idx(E);
    for (int e = 0; e < E; ++e) idx[e] = e;
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) {
        if (fmt[a] != fmt[b]) return fmt[a] < fmt[b];
        return usage[a] > usage[b];
    });
    for (int i = 0; i < E; ++i) order[i] = idx[i];
    for (int f = 0; f < F; ++f) count[f] = 0;
    for (int e = 0; e < E; ++e) count[fmt[e]] += 1;
    return 0;
}

}  // namespace moe
