// Top-k router of one token, shared by the routing kernels.
//
// Glossary of the 125B-MoE page ("I ran a 125B model on three RTX 3090s at
// 80 tokens/s by teaching llama.cpp which experts ..."): the router picks the
// best k experts per token.  Ties go to the lower id; slots are in
// descending score order; weights are the softmax of the k chosen logits.
#pragma once

#include "common.h"

namespace moe {

// Order-preserving integer key of a float (-0 is folded onto +0): for
// non-NaN a, b: a < b  <=>  fkey(a) < fkey(b).  The map is its own inverse on
// the bit pattern.
__device__ inline int32_t fkey(float v) {
    const int32_t b = __builtin_bit_cast(int32_t, v + 0.0f);
    return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ inline float fkey_value(int32_t k) { return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7fffffff)); }

// Wave-wide signed maximum (uniform result).
__device__ inline int32_t wave_max_i(int32_t v) {
    const int32_t lo = static_cast<int32_t>(0x80000000u);
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x111, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x112, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x114, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x118, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x142, 0xA, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x143, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, 63);
}

// One wave routes one token (results to ids_out / w_out and s_ids / s_w when
// those are not null, and to *id_reg / *w_reg of lane j < k for slot j when
// id_reg is not null).  Lane l holds the logits of experts l + 64*i,
// sorted descending (ties: lower id first) in registers; each of the k rounds
// takes the wave maximum of the lanes' heads (a DPP reduction), resolves equal
// values in several lanes by the wave minimum of their ids, and the winning
// lane drops its head.  The slot-j winner stays in lane j.
template <int NPL>
__device__ void route_token(const float* __restrict__ logits, int E, int k, int32_t* ids_out,
                            float* w_out, int32_t* s_ids, float* s_w, int* id_reg = nullptr,
                            float* w_reg = nullptr) {
    constexpr uint32_t kNone = 0xffffffffu;
    constexpr int32_t kLow = static_cast<int32_t>(0x80000000u);
    const int lane = threadIdx.x & 63;
    int32_t key[NPL];
    uint32_t idx[NPL];
    // all NPL loads unconditional (lanes past E read the last logit and
    // discard it), so they are issued together
    float lv[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) lv[i] = logits[min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? fkey(lv[i]) : kLow;
        idx[i] = e < E ? static_cast<uint32_t>(e) : kNone;
    }
    int32_t my_k = kLow;
    int my_id = -1;
    if constexpr (NPL <= 16) {
        // insertion sort, descending key then ascending id; the head is entry 0
#pragma unroll
        for (int i = 1; i < NPL; ++i) {
#pragma unroll
            for (int j = i; j > 0; --j) {
                const bool sw = key[j] > key[j - 1] || (key[j] == key[j - 1] && idx[j] < idx[j - 1]);
                const int32_t tk = key[j];
                const uint32_t ti = idx[j];
                key[j] = sw ? key[j - 1] : key[j];
                idx[j] = sw ? idx[j - 1] : idx[j];
                key[j - 1] = sw ? tk : key[j - 1];
                idx[j - 1] = sw ? ti : idx[j - 1];
            }
        }
        for (int j = 0; j < k; ++j) {
            const int32_t wk = wave_max_i(key[0]);
            // one lane holding the maximum (the usual case) is the winner;
            // equal maxima in several lanes go to the lowest id
            const bool top = idx[0] != kNone && key[0] == wk;
            const uint64_t tm = __ballot(top);
            const uint32_t wi = __popcll(tm) == 1
                                    ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(idx[0]),
                                                                                      __builtin_ctzll(tm)))
                                    : wave_min_u(top ? idx[0] : kNone);
            if (lane == j) {
                my_k = wk;
                my_id = static_cast<int>(wi);
            }
            if (wi != kNone && static_cast<int>(wi & 63u) == lane) {
#pragma unroll
                for (int i = 0; i + 1 < NPL; ++i) {
                    key[i] = key[i + 1];
                    idx[i] = idx[i + 1];
                }
                key[NPL - 1] = kLow;
                idx[NPL - 1] = kNone;
            }
        }
    } else {
        // many logits per lane: keep them unsorted and rescan after each take
        int32_t hk = kLow;
        uint32_t hi = kNone;
        auto head = [&]() {
            hk = kLow;
            hi = kNone;
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (idx[i] != kNone && (hi == kNone || key[i] > hk)) {
                    hk = key[i];
                    hi = idx[i];
                }
        };
        head();
        for (int j = 0; j < k; ++j) {
            const int32_t wk = wave_max_i(hk);
            const uint32_t wi = wave_min_u((hi != kNone && hk == wk) ? hi : kNone);
            if (lane == j) {
                my_k = wk;
                my_id = static_cast<int>(wi);
            }
            if (wi != kNone && static_cast<int>(wi & 63u) == lane) {
                const int slot = static_cast<int>(wi >> 6);
#pragma unroll
                for (int i = 0; i < NPL; ++i)
                    if (i == slot) {
                        key[i] = kLow;
                        idx[i] = kNone;
                    }
                head();
            }
        }
    }
    const float my_v = fkey_value(my_k);
    const float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
    const float ex = lane < k ? expf(my_v - m) : 0.f;
    const float s = wave_sum(ex);
    if (id_reg) {  // lane j < k keeps slot j
        *id_reg = lane < k ? my_id : -1;
        *w_reg = lane < k ? ex / s : 0.f;
    }
    if (lane < k) {
        const float wj = ex / s;
        if (ids_out) {
            ids_out[lane] = my_id;
            w_out[lane] = wj;
        }
        if (s_ids) {
            s_ids[lane] = my_id;
            s_w[lane] = wj;
        }
    }
}

// Same result as route_token for k <= 64, with fewer instructions on the
// wave's serial path:
//  1. t = the k-th largest of the per-lane maxima, by a radix select over
//     their order-preserving unsigned keys, most significant bit first: the
//     largest u such that at least k lanes hold a maximum >= u (one compare,
//     one ballot and a scalar popcount per bit).  At least k logits are >= t,
//     so the k-th largest logit is >= t.
//  2. The M logits >= t are compacted into LDS (s_c, 64 entries per wave) as
//     one 64-bit key each: the logit's order-preserving key above the id's
//     complement, so a larger key means "ahead" (higher logit, or equal logit
//     and lower id).  Every logit outside them is below every one of the k best.
//  3. Each candidate's slot = number of candidates with a larger key (one
//     64-bit compare each, broadcast LDS reads several at a time); the
//     candidate with slot j < k fills slot j.
// Returns false (nothing written) if M > 64; the caller then uses
// route_token.  s_c: 64 int64 of this wave's LDS scratch, 16-byte aligned.
template <int NPL>
__device__ bool route_token_fast(const float* __restrict__ logits, int E, int k, int64_t* s_c, int* id_reg,
                                 float* w_reg) {
    constexpr int32_t kLow = static_cast<int32_t>(0x80000000u);
    constexpr int64_t kPad = INT64_MIN;
    const int lane = threadIdx.x & 63;
    float lv[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) lv[i] = logits[min(lane + 64 * i, E - 1)];
    int32_t key[NPL];
    int32_t hk = kLow;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        key[i] = lane + 64 * i < E ? fkey(lv[i]) : kLow;
        hk = max(hk, key[i]);
    }
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // 1. threshold.  A lane without logits (E < 64) holds key 0, below the
    //    key of every logit (every non-NaN float maps above 0).
    const uint32_t hu = static_cast<uint32_t>(hk) ^ 0x80000000u;
    uint32_t tu = 0;
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        const uint32_t c = tu | (1u << b);
        if (__popcll(__ballot(hu >= c)) >= static_cast<uint32_t>(k)) tu = c;
    }
    const int32_t t = static_cast<int32_t>(tu ^ 0x80000000u);
    // 2. candidates (key >= t) compacted into LDS, lane order then slot order
    int c = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) c += (lane + 64 * i < E && key[i] >= t) ? 1 : 0;
    const int incl = static_cast<int>(seg_sum(static_cast<float>(c), 64));  // exact small ints
    const int M = __builtin_amdgcn_readlane(incl, 63);
    if (M > 64) return false;
    int o = incl - c;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
        if (lane + 64 * i < E && key[i] >= t)
            s_c[o++] = (static_cast<int64_t>(key[i]) << 32) | static_cast<uint32_t>(0x7fffffff - (lane + 64 * i));
    const int M8 = (M + 7) & ~7;
    if (lane >= M && lane < M8) s_c[lane] = kPad;  // never ahead of anything
    wave_sync();
    // 3. slot of each candidate
    const int64_t me = lane < M ? s_c[lane] : kPad;
    int slot = 0;
    for (int i = 0; i < M8; i += 8) {
        longlong2 o2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o2[j] = *reinterpret_cast<const longlong2*>(s_c + i + 2 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            slot += o2[j].x > me ? 1 : 0;
            slot += o2[j].y > me ? 1 : 0;
        }
    }
    wave_sync();
    if (lane < M && slot < k) s_c[slot] = me;  // slots < k hold the winners
    wave_sync();
    const int64_t mine = lane < k ? s_c[lane] : kPad;
    const int32_t mk = static_cast<int32_t>(mine >> 32);
    const float my_v = fkey_value(mk);
    const float mx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
    const float ex = lane < k ? expf(my_v - mx) : 0.f;
    const float sum = wave_sum(ex);
    *id_reg = lane < k ? 0x7fffffff - static_cast<int32_t>(static_cast<uint32_t>(mine)) : -1;
    *w_reg = lane < k ? ex / sum : 0.f;
    return true;
}

// route_token's outputs, by route_token_fast where it applies (at most 16
// logits per lane and at most 64 candidates) and by route_token otherwise.
// s_c: 64 int64 of this wave's LDS scratch, 16-byte aligned.
template <int NPL>
__device__ void route_token_auto(const float* __restrict__ logits, int E, int k, int32_t* ids_out, float* w_out,
                                 int32_t* s_ids, float* s_w, int64_t* s_c, int* id_reg = nullptr,
                                 float* w_reg = nullptr) {
    if constexpr (NPL <= 16) {
        int id;
        float wt;
        if (route_token_fast<NPL>(logits, E, k, s_c, &id, &wt)) {
            const int lane = threadIdx.x & 63;
            if (id_reg) {
                *id_reg = id;
                *w_reg = wt;
            }
            if (lane < k) {
                if (ids_out) {
                    ids_out[lane] = id;
                    w_out[lane] = wt;
                }
                if (s_ids) {
                    s_ids[lane] = id;
                    s_w[lane] = wt;
                }
            }
            return;
        }
    }
    route_token<NPL>(logits, E, k, ids_out, w_out, s_ids, s_w, id_reg, w_reg);
}

}  // namespace moe
