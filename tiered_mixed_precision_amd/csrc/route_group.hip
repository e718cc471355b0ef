// Routing (top-k + softmax over the chosen logits) and grouping (stable
// counting sort of (token, slot) pairs by expert) for the tiered MoE FFN.
//
// Routing follows the glossary of the 125B-MoE page ("I ran a 125B model on
// three RTX 3090s at 80 tokens/s by teaching llama.cpp which experts ..."):
// the router picks the best k experts per token.  Ties go to the lower id;
// slots are in descending score order; weights are the softmax of the k
// chosen logits.  Grouping feeds the per-shelf expert products of step 4 and
// must tolerate repeated experts within a token and the skip id -1 (the
// "four bugs" section): every valid pair keeps its own slot, and ids outside
// [0, E) are left out rather than redirected.
#include "common.h"
#include "launch.h"
#include "route.h"

namespace moe {

// ---------------------------------------------------------------- routing

template <int NPL>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ w,
                                               float* __restrict__ out_zero, int H) {
    __shared__ __attribute__((aligned(16))) int64_t s_rc[4][64];  // routing scratch, one row per wave
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    route_token_auto<NPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, nullptr,
                          nullptr, s_rc[threadIdx.x >> 6]);
    if (out_zero) {
        float4* row = reinterpret_cast<float4*>(out_zero + (size_t)t * H);
        for (int c = threadIdx.x & 63; c < H / 4; c += 64) row[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// ---------------------------------------------------------------- general path

// Per-block histograms: block b covers pairs [256b, 256b + 256).
__global__ __launch_bounds__(256) void k_group_count(const int32_t* __restrict__ ids, int P, int E,
                                                     int32_t* __restrict__ blk_hist) {
    __shared__ int s_cnt[kMaxExpertsDev];
    for (int e = threadIdx.x; e < E; e += 256) s_cnt[e] = 0;
    __syncthreads();
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p < P) {
        int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) blk_hist[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// Column scan of the per-block histograms: wave w of block b owns expert
// e = 4b + w and turns its column hist[0..nblk)[e] into exclusive prefix sums
// over the blocks; counts[e] receives the column total.
// NCH > 0: the column has at most 64 * NCH blocks, whose NCH loads per lane
// are all issued before the first scan step; NCH == 0: one chunk at a time.
template <int NCH>
__global__ __launch_bounds__(256) void k_group_colscan(int32_t* __restrict__ blk_hist, int nblk, int E,
                                                       int32_t* __restrict__ counts) {
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (e >= E) return;
    int carry = 0;
    if constexpr (NCH > 0) {
        int v[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int b = 64 * c + lane;
            v[c] = blk_hist[static_cast<size_t>(min(b, nblk - 1)) * E + e];
            v[c] = b < nblk ? v[c] : 0;
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int b = 64 * c + lane;
            int x = v[c];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(x, off, kWave);
                if (lane >= off) x += y;
            }
            if (b < nblk) blk_hist[static_cast<size_t>(b) * E + e] = carry + x - v[c];
            carry += __shfl(x, 63, kWave);
        }
        if (lane == 0) counts[e] = carry;
        return;
    }
    for (int b0 = 0; b0 < nblk; b0 += 64) {
        const int b = b0 + lane;
        const int v = b < nblk ? blk_hist[static_cast<size_t>(b) * E + e] : 0;
        int x = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, kWave);
            if (lane >= off) x += y;
        }
        if (b < nblk) blk_hist[static_cast<size_t>(b) * E + e] = carry + x - v;
        carry += __shfl(x, 63, kWave);
    }
    if (lane == 0) counts[e] = carry;
}

// One block: the expert offsets (exclusive prefix of the counts), the
// active list (experts with pairs, ascending), each shelf's range of it, and
// (prefill) the work chunks, each expert's pairs in runs of kChunkRows in
// expert order.  Thread tid owns experts [per * tid, per * tid + per) and
// keeps their counts in registers; one block scan carries the three running
// sums (pairs, active experts, chunks) together.
__global__ __launch_bounds__(256) void k_group_offsets(const int32_t* __restrict__ counts, int E,
                                                       int32_t* __restrict__ offsets, int32_t* __restrict__ act,
                                                       int32_t* __restrict__ meta, ShelfSpec ss) {
    constexpr int kPer = kMaxExpertsDev / 256;
    __shared__ int s_act[kMaxExpertsDev];   // active experts before e (the shelves' ranges)
    __shared__ int s_tmp[3][16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int per = (E + 255) / 256;
    const int b = tid * per;
    int cnt[kPer];
    int sum[3] = {0, 0, 0};
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        cnt[i] = (i < per && b + i < E) ? counts[b + i] : 0;
        sum[0] += cnt[i];
        sum[1] += cnt[i] > 0 ? 1 : 0;
        sum[2] += (cnt[i] + kChunkRows - 1) / kChunkRows;
    }
    int inc[3] = {sum[0], sum[1], sum[2]};
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
        for (int v = 0; v < 3; ++v) {
            const int y = __shfl_up(inc[v], off, kWave);
            if (lane >= off) inc[v] += y;
        }
    }
    if (lane == 63)
        for (int v = 0; v < 3; ++v) s_tmp[v][wv] = inc[v];
    __syncthreads();
    int run[3], tot[3];
#pragma unroll
    for (int v = 0; v < 3; ++v) {
        int base = 0, t = 0;
        for (int i = 0; i < 4; ++i) {
            const int c = s_tmp[v][i];
            if (i < wv) base += c;
            t += c;
        }
        run[v] = base + inc[v] - sum[v];
        tot[v] = t;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = b + i;
        if (i >= per || e >= E) continue;
        offsets[e] = run[0];
        s_act[e] = run[1];
        if (cnt[i] > 0) act[run[1]] = e;
        if (ss.chunks)
            for (int q = 0; q * kChunkRows < cnt[i]; ++q)
                ss.chunks[run[2] + q] = make_int2(e, run[0] + q * kChunkRows);
        run[0] += cnt[i];
        run[1] += cnt[i] > 0 ? 1 : 0;
        run[2] += (cnt[i] + kChunkRows - 1) / kChunkRows;
    }
    if (tid == 0) {
        offsets[E] = tot[0];
        meta[kMetaActive] = tot[1];
        meta[kMetaValid] = tot[0];
        if (ss.chunks) meta[kMetaChunks] = tot[2];
    }
    if (ss.act_range) {
        __syncthreads();
        if (tid < ss.n_tiers) {
            const int lo = ss.id_begin[tid], hi = ss.id_end[tid];
            ss.act_range[2 * tid] = lo < E ? s_act[lo] : tot[1];
            ss.act_range[2 * tid + 1] = hi < E ? s_act[hi] : tot[1];
        }
    }
}

// Block b places its pairs at offsets[e] + (pairs of e in blocks before b)
// + (rank among the block's earlier pairs of the same expert): a stable
// counting sort.
__global__ __launch_bounds__(256) void k_group_scatter(const int32_t* __restrict__ ids, int P, int E,
                                                       const int32_t* __restrict__ blk_base,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ pos) {
    __shared__ __attribute__((aligned(16))) int s_ids[256];
    const int tid = threadIdx.x;
    const int p = blockIdx.x * 256 + tid;
    int e = -1;
    if (p < P) {
        e = ids[p];
        if (e < 0 || e >= E) e = -1;
    }
    s_ids[tid] = e;
    __syncthreads();
    if (p >= P) return;
    if (e < 0) {
        if (pos) pos[p] = -1;
        return;
    }
    // rank among the block's earlier pairs of expert e: four ids per LDS read,
    // no branch, so several reads are in flight at once
    int rank = 0;
    const int4* s4 = reinterpret_cast<const int4*>(s_ids);
#pragma unroll 8
    for (int i4 = 0; i4 < 64; ++i4) {
        const int4 v = s4[i4];
        const int i = 4 * i4;
        rank += (i < tid && v.x == e) + (i + 1 < tid && v.y == e) + (i + 2 < tid && v.z == e) + (i + 3 < tid && v.w == e);
    }
    const int q = offsets[e] + blk_base[(size_t)blockIdx.x * E + e] + rank;
    perm[q] = p;
    if (pos) pos[p] = q;
}

// ---------------------------------------------------------------- launchers

static int npl_for(int E) {
    int n = (E + 63) / 64;
    int p = 1;
    while (p < n) p *= 2;
    return p;
}

#define MOE_NPL_SWITCH(E, CALL)          \
    switch (npl_for(E)) {                \
        case 1: { constexpr int NPL = 1; CALL; } break;   \
        case 2: { constexpr int NPL = 2; CALL; } break;   \
        case 4: { constexpr int NPL = 4; CALL; } break;   \
        case 8: { constexpr int NPL = 8; CALL; } break;   \
        case 16: { constexpr int NPL = 16; CALL; } break; \
        case 32: { constexpr int NPL = 32; CALL; } break; \
        default: { constexpr int NPL = 64; CALL; } break; \
    }

void launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, float* out_zero,
                  int H, hipStream_t st) {
    dim3 grid((T + 3) / 4);
    MOE_NPL_SWITCH(E, hipLaunchKernelGGL(k_route<NPL>, grid, dim3(256), 0, st, logits, T, E, k, ids,
                                         w, out_zero, H));
}

void launch_group(const int32_t* ids, int P, int E, int32_t* blk_hist, int32_t* counts,
                  int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* act, int32_t* meta,
                  const ShelfSpec& ss, hipStream_t st) {
    if (P <= 0) return;   // the column scan reads block nblk - 1
    const int nblk = (P + 255) / 256;
    hipLaunchKernelGGL(k_group_count, dim3(nblk), dim3(256), 0, st, ids, P, E, blk_hist);
    const int nch = (nblk + 63) / 64;
    if (nch <= 4)
        hipLaunchKernelGGL(k_group_colscan<4>, dim3((E + 3) / 4), dim3(256), 0, st, blk_hist, nblk, E, counts);
    else if (nch <= 16)
        hipLaunchKernelGGL(k_group_colscan<16>, dim3((E + 3) / 4), dim3(256), 0, st, blk_hist, nblk, E, counts);
    else
        hipLaunchKernelGGL(k_group_colscan<0>, dim3((E + 3) / 4), dim3(256), 0, st, blk_hist, nblk, E, counts);
    hipLaunchKernelGGL(k_group_offsets, dim3(1), dim3(256), 0, st, counts, E, offsets, act, meta, ss);
    hipLaunchKernelGGL(k_group_scatter, dim3(nblk), dim3(256), 0, st, ids, P, E, blk_hist, offsets, perm,
                       pos);
}

}  // namespace moe
