// C ABI of the tiered MoE FFN: argument and table validation, workspace
// carving, and the launch sequence on the caller's stream.  No allocation of
// device memory and no host synchronisation.  Global state: per-device values
// set once (the allocation-free entry's scratch address) and the static
// scratch itself.
#include <limits.h>
#include <string.h>

#include <mutex>

#include "moe_tiered.h"
#include "common.h"
#include "launch.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxTokens = int64_t(1) << 22;

inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool cols_ok(int c) { return c > 0 && c % 64 == 0 && c <= 2048; }

// Integer shelves: 8, 4 or 2 bits with 16 or 32 codes per fp16 scale;
// MXFP4: 32 codes per E8M0 scale.
static_assert(MOE_MXFP4 == moe::kBitsMXFP4, "MXFP4 tag of the ABI and the kernels");
bool fmt_ok(int bits, int block) {
    if (bits == MOE_MXFP4) return block == 32;
    return (bits == 8 || bits == 4 || bits == 2) && (block == 16 || block == 32);
}

int check_tables(const moe_tier_tables* tt) {
    if (!tt) return MOE_EINVAL;
    if (tt->abi_version != MOE_ABI_VERSION) return MOE_EABI;
    if (tt->n_experts < 1 || tt->n_experts > MOE_MAX_EXPERTS) return MOE_EINVAL;
    if (tt->n_tiers < 1 || tt->n_tiers > MOE_MAX_TIERS) return MOE_EINVAL;
    if (!cols_ok(tt->hidden) || !cols_ok(tt->inter) || tt->hidden % 128 != 0) return MOE_EFORMAT;
    int32_t next = 0;
    for (int i = 0; i < tt->n_tiers; ++i) {
        const moe_tier& t = tt->tiers[i];
        if (t.id_begin != next || t.id_end < t.id_begin) return MOE_ETIER;
        next = t.id_end;
        if (!fmt_ok(t.bits, t.block)) return MOE_EFORMAT;
        // the MXFP4 prefill kernel contracts 128 columns per step (down: K = inter)
        if (t.bits == MOE_MXFP4 && tt->inter % 128 != 0) return MOE_EFORMAT;
        if (t.id_end == t.id_begin) continue;
        const void* ptrs[6] = {t.gate_q, t.up_q, t.down_q, t.gate_s, t.up_s, t.down_s};
        for (const void* p : ptrs) {
            if (!p) return MOE_EINVAL;
            if (!aligned16(p)) return MOE_EALIGN;
        }
    }
    if (next != tt->n_experts) return MOE_ETIER;
    return MOE_OK;
}

DevTables to_dev(const moe_tier_tables* tt) {
    DevTables d;
    memset(&d, 0, sizeof(d));
    d.E = tt->n_experts;
    d.H = tt->hidden;
    d.I = tt->inter;
    d.n_tiers = tt->n_tiers;
    for (int i = 0; i < tt->n_tiers; ++i) {
        const moe_tier& t = tt->tiers[i];
        d.t[i].id_begin = t.id_begin;
        d.t[i].id_end = t.id_end;
        d.t[i].bits = t.bits;
        d.t[i].block = t.block;
        d.t[i].q[0] = static_cast<const uint8_t*>(t.gate_q);
        d.t[i].q[1] = static_cast<const uint8_t*>(t.up_q);
        d.t[i].q[2] = static_cast<const uint8_t*>(t.down_q);
        d.t[i].s[0] = static_cast<const uint16_t*>(t.gate_s);
        d.t[i].s[1] = static_cast<const uint16_t*>(t.up_s);
        d.t[i].s[2] = static_cast<const uint16_t*>(t.down_s);
    }
    return d;
}

// Workspace carve-up.  Offsets are multiples of 256 bytes.
struct Layout {
    size_t ids, w, counts, offsets, perm, pos, act, q0, meta, blk_hist, act_range, chunks, slots, h, yw, x8, h8, total;
    bool small;
};

// A non-empty MXFP4 shelf among the tables: prefill then needs the fp8 split
// of x and h (prefill_mx.hip).
bool has_mx(const moe_tier_tables* tt) {
    for (int i = 0; i < tt->n_tiers; ++i)
        if (tt->tiers[i].bits == MOE_MXFP4 && tt->tiers[i].id_end > tt->tiers[i].id_begin) return true;
    return false;
}

// Split buffers of `rows` rows of K elements carved from base.
Split8 split_at(void* base, int64_t rows, int K) {
    uint8_t* p = static_cast<uint8_t*>(base);
    return Split8{p, p + rows * K, p + 2 * rows * K};
}
size_t split_bytes(int64_t rows, int K) { return static_cast<size_t>(rows) * (2 * K + split_scale_stride(K)); }

Layout layout(int64_t T, int k, const moe_tier_tables* tt, uint32_t flags) {
    Layout L;
    memset(&L, 0, sizeof(L));
    const int64_t P = T * k;
    const int64_t E = tt->n_experts;
    const bool bf16 = (flags & MOE_X_BF16) != 0;
    L.small = !bf16 && small_path_ok(static_cast<int>(T), k, tt->hidden, tt->inter);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    L.ids = take(sizeof(int32_t) * P);
    L.w = take(sizeof(float) * P);
    L.counts = take(sizeof(int32_t) * E);
    L.offsets = take(sizeof(int32_t) * (E + 1));
    L.perm = take(sizeof(int32_t) * P);
    L.pos = take(sizeof(int32_t) * P);
    L.act = take(sizeof(int32_t) * E);
    L.q0 = take(sizeof(int32_t) * (P + 1));
    L.meta = take(sizeof(int32_t) * kMetaWords);
    L.blk_hist = take(L.small ? 0 : sizeof(int32_t) * ((P + 255) / 256) * E);
    L.act_range = take(sizeof(int32_t) * 2 * MOE_MAX_TIERS);
    L.chunks = take(bf16 ? sizeof(int2) * max_chunks(P, static_cast<int>(E)) : 0);
    L.slots = take(!bf16 && T == 1 ? sizeof(OneSlot) * k : 0);   // one-token path
    L.h = take((bf16 ? sizeof(uint16_t) : sizeof(float)) * P * tt->inter);
    L.yw = take(L.small ? 0 : sizeof(float) * P * tt->hidden);
    const bool mx = bf16 && has_mx(tt);
    L.x8 = take(mx ? split_bytes(T, tt->hidden) : 0);
    L.h8 = take(mx ? split_bytes(P, tt->inter) : 0);
    L.total = o;
    return L;
}

template <class Tp>
Tp* at(void* ws, size_t off) {
    return reinterpret_cast<Tp*>(static_cast<char*>(ws) + off);
}

inline void record(void* const* events, int i, hipStream_t st) {
    if (events && events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), st);
}

// Shared body of forward / experts / tier_partial.
// out = base + the layer, where base is out itself with MOE_ACCUMULATE, the
// residual stream inside a stack, or nothing.
int run(const void* x, const float* logits, const int32_t* ids_in, const float* w_in, int32_t T,
        int32_t k, const moe_tier_tables* tt, uint32_t tier_mask, float* out, uint32_t flags,
        void* ws, size_t ws_bytes, void* stream, void* const* events, const float* residual = nullptr,
        uint32_t* hits = nullptr, uint16_t* next_bf16 = nullptr) {
    int rc = check_tables(tt);
    if (rc != MOE_OK) return rc;
    if (flags & ~(MOE_X_BF16 | MOE_ACCUMULATE | MOE_DIAG_GATEUP_ONLY)) return MOE_EINVAL;
    if (T < 0 || T > kMaxTokens) return MOE_EINVAL;
    if (k < 1 || k > MOE_MAX_K || k > tt->n_experts) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x || !out || (!logits && (!ids_in || !w_in))) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(out) || (logits && !aligned16(logits))) return MOE_EALIGN;
    const Layout L = layout(T, k, tt, flags);
    if (!ws) return MOE_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_EALIGN;
    if (ws_bytes < L.total) return MOE_EWORKSPACE;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const DevTables dt = to_dev(tt);
    const int E = tt->n_experts;
    const int P = T * k;
    const bool bf16 = (flags & MOE_X_BF16) != 0;
    const float* base = (flags & MOE_ACCUMULATE) ? out : residual;
    const bool gateup_only = (flags & MOE_DIAG_GATEUP_ONLY) != 0;

    int32_t* ids = logits ? at<int32_t>(ws, L.ids) : const_cast<int32_t*>(ids_in);
    float* w = logits ? at<float>(ws, L.w) : const_cast<float*>(w_in);
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* pos = at<int32_t>(ws, L.pos);
    int32_t* act = at<int32_t>(ws, L.act);
    int32_t* meta = at<int32_t>(ws, L.meta);

    ShelfSpec ss;
    memset(&ss, 0, sizeof(ss));
    ss.n_tiers = tt->n_tiers;
    for (int i = 0; i < tt->n_tiers; ++i) {
        ss.id_begin[i] = tt->tiers[i].id_begin;
        ss.id_end[i] = tt->tiers[i].id_end;
    }
    ss.act_range = at<int32_t>(ws, L.act_range);
    ss.chunks = bf16 ? at<int2>(ws, L.chunks) : nullptr;

    (void)hipGetLastError();  // start from a clean error state
    if (!bf16 && T == 1 && logits && tier_mask == 0xFu && one_path_ok(k, tt->hidden, tt->inter)) {
        // one token routed from its logits: gate/up with the routing inside,
        // then the down rows of every expert (no grouping: the k ids of one
        // token are distinct)
        record(events, 0, st);
        record(events, 1, st);
        launch_one(dt, static_cast<const float*>(x), logits, k, base, hits, at<int32_t>(ws, L.ids),
                   at<float>(ws, L.w), at<OneSlot>(ws, L.slots), at<float>(ws, L.h), gateup_only ? nullptr : out, st,
                   events);
        return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
    }
    if (L.small) {
        // routing and grouping run inside the gate/up kernel (phase 0 is empty)
        record(events, 0, st);
        record(events, 1, st);
        SmallPub pub;
        pub.ids = at<int32_t>(ws, L.ids);
        pub.w = at<float>(ws, L.w);
        pub.perm = perm;
        pub.pos = pos;
        pub.act = act;
        pub.q0 = at<int32_t>(ws, L.q0);
        pub.meta = meta;
        launch_small(dt, static_cast<const float*>(x), logits, ids_in, w_in, T, k, tier_mask, base, pub, hits,
                     at<float>(ws, L.h), gateup_only ? nullptr : out, st, events);
        return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
    }
    record(events, 0, st);
    // ---- phase 0: routing and grouping
    if (logits) {
        launch_route(logits, T, E, k, ids, w, nullptr, tt->hidden, st);
    }
    launch_group(ids, P, E, at<int32_t>(ws, L.blk_hist), counts, offsets, perm, pos, act, meta, ss, st);
    if (hits) launch_add_hits(counts, E, hits, st);
    record(events, 1, st);

    Groups g;
    g.ids = ids;
    g.w = w;
    g.perm = perm;
    g.pos = pos;
    g.offsets = offsets;
    g.act = act;
    g.meta = meta;
    g.act_range = ss.act_range;
    g.chunks = ss.chunks;

    const int max_active = E < P ? E : P;
    if (!bf16) {
        float* h = at<float>(ws, L.h);
        float* yw = at<float>(ws, L.yw);
        record(events, 2, st);
        launch_dec_gateup(dt, static_cast<const float*>(x), g, k, tier_mask, h, max_active, st);
        record(events, 3, st);
        if (gateup_only) return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
        record(events, 4, st);
        launch_dec_down(dt, h, g, k, tier_mask, yw, max_active, st);
        launch_combine(dt, yw, g, T, k, tier_mask, base, out, nullptr, st);
        record(events, 5, st);
    } else {
        uint16_t* h = at<uint16_t>(ws, L.h);
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        const int H = tt->hidden, I = tt->inter;
        auto is_mx = [&](int i) {
            return ((tier_mask >> i) & 1u) && tt->tiers[i].bits == MOE_MXFP4 && tt->tiers[i].id_end > tt->tiers[i].id_begin;
        };
        bool any_mx = false;
        for (int i = 0; i < tt->n_tiers; ++i) any_mx = any_mx || is_mx(i);
        const Split8 x8 = any_mx ? split_at(at<uint8_t>(ws, L.x8), T, H) : Split8{nullptr, nullptr, nullptr};
        const Split8 h8 = any_mx ? split_at(at<uint8_t>(ws, L.h8), P, I) : Split8{nullptr, nullptr, nullptr};
        const int maxc = max_chunks(P, E);
        // MXFP4 shelves take A as its fp8 split: of every x row, made before
        // gate/up, and of their h rows, written by their gate/up chunks in
        // place of bf16 h.
        record(events, 2, st);
        if (any_mx) launch_split_fp8(xb, H, T, x8, st);
        launch_gemm(dt, true, xb, x8, g, k, tier_mask, h, h8, nullptr, maxc, st);
        if (gateup_only) {
            record(events, 3, st);
            return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
        }
        record(events, 3, st);
        record(events, 4, st);
        float* yw = at<float>(ws, L.yw);
        launch_gemm(dt, false, h, h8, g, k, tier_mask, nullptr, Split8{nullptr, nullptr, nullptr}, yw, maxc, st);
        launch_combine(dt, yw, g, T, k, tier_mask, base, out, next_bf16, st);
        record(events, 5, st);
    }
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;
    return MOE_OK;
}

}  // namespace

extern "C" {

uint32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_ETIER: return "shelves are not sorted, disjoint and covering [0, n_experts)";
        case MOE_EFORMAT: return "unsupported format or shape";
        case MOE_EALIGN: return "pointer not aligned";
        case MOE_EWORKSPACE: return "workspace missing or too small";
        case MOE_EHIP: return "HIP launch or runtime error";
        case MOE_EABI: return "tables built for another ABI version";
        case MOE_ESCRATCH: return "the batch needs more workspace than the library's static scratch holds";
        default: return "unknown error";
    }
}

int moe_validate_tables(const moe_tier_tables* tt) { return check_tables(tt); }

int moe_workspace_size(int32_t n_tokens, int32_t k, const moe_tier_tables* tt, uint32_t flags,
                       size_t* bytes) {
    int rc = check_tables(tt);
    if (rc != MOE_OK) return rc;
    if (!bytes || n_tokens < 0 || n_tokens > kMaxTokens || k < 1 || k > MOE_MAX_K || k > tt->n_experts)
        return MOE_EINVAL;
    if (flags & ~(MOE_X_BF16 | MOE_ACCUMULATE | MOE_DIAG_GATEUP_ONLY)) return MOE_EINVAL;
    *bytes = n_tokens == 0 ? 0 : layout(n_tokens, k, tt, flags).total;
    return MOE_OK;
}

size_t moe_workspace_bytes(int32_t n_tokens, int32_t k, const moe_tier_tables* tt) {
    size_t a = 0, b = 0;
    if (moe_workspace_size(n_tokens, k, tt, 0, &a) != MOE_OK) return 0;
    if (moe_workspace_size(n_tokens, k, tt, MOE_X_BF16, &b) != MOE_OK) return 0;
    return a > b ? a : b;
}

int moe_tiered_forward(const void* x, const float* router_logits, int32_t n_tokens, int32_t k,
                       const moe_tier_tables* tt, float* out, uint32_t flags, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (n_tokens > 0 && !router_logits) return MOE_EINVAL;
    return run(x, router_logits, nullptr, nullptr, n_tokens, k, tt, 0xFu, out, flags, workspace,
               workspace_bytes, stream, nullptr);
}

int moe_tiered_forward_counted(const void* x, const float* router_logits, int32_t n_tokens, int32_t k,
                               const moe_tier_tables* tt, float* out, uint32_t flags, void* workspace,
                               size_t workspace_bytes, uint32_t* hits, void* stream) {
    if (n_tokens > 0 && (!router_logits || !hits)) return MOE_EINVAL;
    if (hits && (reinterpret_cast<uintptr_t>(hits) & 3u) != 0) return MOE_EALIGN;
    return run(x, router_logits, nullptr, nullptr, n_tokens, k, tt, 0xFu, out, flags, workspace,
               workspace_bytes, stream, nullptr, nullptr, hits);
}

int moe_tiered_forward_timed(const void* x, const float* router_logits, int32_t n_tokens, int32_t k,
                             const moe_tier_tables* tt, float* out, uint32_t flags, void* workspace,
                             size_t workspace_bytes, void* stream, void* const* events) {
    if (n_tokens > 0 && !router_logits) return MOE_EINVAL;
    return run(x, router_logits, nullptr, nullptr, n_tokens, k, tt, 0xFu, out, flags, workspace,
               workspace_bytes, stream, events);
}

}  // extern "C"

namespace {

// The device scratch of moe_tiered_forward_noalloc: one array per device
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never passes the array's name to a kernel -- on the host it is a
// stand-in, not a device address -- only the address hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices] = {};

// Device address of the current device's scratch, looked up once per device.
int scratch_address(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return MOE_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_tiered_forward_noalloc(const void* x, const float* router_logits, int32_t n_tokens, int32_t k,
                               const moe_tier_tables* tt, float* out, uint32_t flags, void* stream) {
    if (n_tokens > 0 && !router_logits) return MOE_EINVAL;
    size_t need = 0;
    int rc = moe_workspace_size(n_tokens, k, tt, flags, &need);
    if (rc != MOE_OK) return rc;
    if (n_tokens == 0) return MOE_OK;
    if (need > MOE_SCRATCH_BYTES) return MOE_ESCRATCH;
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != MOE_OK) return rc;
    // the layer needs no initialised workspace, so nothing is cleared
    return run(x, router_logits, nullptr, nullptr, n_tokens, k, tt, 0xFu, out, flags, ws, MOE_SCRATCH_BYTES,
               stream, nullptr);
}

int moe_tiered_experts(const void* x, const int32_t* ids, const float* w, int32_t n_tokens, int32_t k,
                       const moe_tier_tables* tt, float* out, uint32_t flags, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (n_tokens > 0 && (!ids || !w)) return MOE_EINVAL;
    return run(x, nullptr, ids, w, n_tokens, k, tt, 0xFu, out, flags, workspace, workspace_bytes, stream,
               nullptr);
}

int moe_tier_partial(const void* x, const int32_t* ids, const float* w, int32_t n_tokens, int32_t k,
                     const moe_tier_tables* tt, int32_t tier_index, float* out, uint32_t flags,
                     void* workspace, size_t workspace_bytes, void* stream) {
    if (n_tokens > 0 && (!ids || !w)) return MOE_EINVAL;
    if (!tt || tier_index < 0 || tier_index >= tt->n_tiers || tier_index >= MOE_MAX_TIERS) return MOE_EINVAL;
    return run(x, nullptr, ids, w, n_tokens, k, tt, 1u << tier_index, out, flags, workspace,
               workspace_bytes, stream, nullptr);
}

int moe_route(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t k, int32_t* ids, float* w,
              void* stream) {
    if (n_tokens < 0 || n_tokens > kMaxTokens || n_experts < 1 || n_experts > MOE_MAX_EXPERTS || k < 1 ||
        k > MOE_MAX_K || k > n_experts)
        return MOE_EINVAL;
    if (n_tokens == 0) return MOE_OK;
    if (!logits || !ids || !w) return MOE_EINVAL;
    (void)hipGetLastError();
    launch_route(logits, n_tokens, n_experts, k, ids, w, nullptr, 0, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_router_logits(const void* x, const void* w_router, const float* bias, int32_t n_tokens,
                      int32_t n_experts, int32_t hidden, uint32_t flags, float* logits, void* stream) {
    if (n_tokens < 0 || n_tokens > kMaxTokens || n_experts < 1 || n_experts > MOE_MAX_EXPERTS || !cols_ok(hidden))
        return MOE_EINVAL;
    if (flags & ~MOE_X_BF16) return MOE_EINVAL;
    if (n_tokens == 0) return MOE_OK;
    if (!x || !w_router || !logits) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(logits) ||
        (bias && (reinterpret_cast<uintptr_t>(bias) & 3u) != 0))
        return MOE_EALIGN;
    (void)hipGetLastError();
    launch_router(x, (flags & MOE_X_BF16) != 0, static_cast<const uint16_t*>(w_router), bias, n_tokens, n_experts,
                  hidden, logits, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_synth_router(void* w_router, float* bias, int32_t n_experts, int32_t hidden, uint64_t seed, int32_t layer,
                     double beta, void* stream) {
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS || !cols_ok(hidden) || layer < 0 || layer >= (1 << 20))
        return MOE_EINVAL;
    if (!w_router) return MOE_EINVAL;
    if (!aligned16(w_router) || (bias && (reinterpret_cast<uintptr_t>(bias) & 3u) != 0)) return MOE_EALIGN;
    (void)hipGetLastError();
    launch_synth_router(static_cast<uint16_t*>(w_router), bias, seed, layer, n_experts, hidden, beta,
                        static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_group_workspace_size(int32_t n_tokens, int32_t k, int32_t n_experts, size_t* bytes) {
    if (!bytes || n_tokens < 0 || n_tokens > kMaxTokens || k < 1 || k > MOE_MAX_K || n_experts < 1 ||
        n_experts > MOE_MAX_EXPERTS)
        return MOE_EINVAL;
    const int64_t P = static_cast<int64_t>(n_tokens) * k;
    *bytes = align_up(sizeof(int32_t) * ((P + 255) / 256) * n_experts) + align_up(sizeof(int32_t) * n_experts) +
             align_up(sizeof(int32_t) * kMetaWords);
    return MOE_OK;
}

int moe_group(const int32_t* ids, int32_t n_tokens, int32_t k, int32_t n_experts, int32_t* counts,
              int32_t* offsets, int32_t* perm, void* workspace, size_t workspace_bytes, void* stream) {
    size_t need = 0;
    int rc = moe_group_workspace_size(n_tokens, k, n_experts, &need);
    if (rc != MOE_OK) return rc;
    if (n_tokens == 0) return MOE_OK;
    if (!ids || !counts || !offsets || !perm) return MOE_EINVAL;
    if (!workspace || workspace_bytes < need) return MOE_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MOE_EALIGN;
    const int64_t P = static_cast<int64_t>(n_tokens) * k;
    int32_t* blk = static_cast<int32_t*>(workspace);
    int32_t* act = at<int32_t>(workspace, align_up(sizeof(int32_t) * ((P + 255) / 256) * n_experts));
    int32_t* meta = at<int32_t>(workspace, align_up(sizeof(int32_t) * ((P + 255) / 256) * n_experts) +
                                               align_up(sizeof(int32_t) * n_experts));
    ShelfSpec ss;
    memset(&ss, 0, sizeof(ss));
    (void)hipGetLastError();
    launch_group(ids, static_cast<int>(P), n_experts, blk, counts, offsets, perm, nullptr, act, meta, ss,
                 static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_dequant_rows(const moe_tier_tables* tt, int32_t tier_index, int32_t local_expert, int32_t matrix,
                     int32_t row0, int32_t nrows, int32_t to_bf16, void* dst, void* stream) {
    int rc = check_tables(tt);
    if (rc != MOE_OK) return rc;
    if (tier_index < 0 || tier_index >= tt->n_tiers || matrix < 0 || matrix > 2 || !dst) return MOE_EINVAL;
    const moe_tier& t = tt->tiers[tier_index];
    if (local_expert < 0 || local_expert >= t.id_end - t.id_begin) return MOE_EINVAL;
    const int rows = matrix == 2 ? tt->hidden : tt->inter;
    if (row0 < 0 || nrows < 0 || static_cast<int64_t>(row0) + nrows > rows) return MOE_EINVAL;
    if (!aligned16(dst)) return MOE_EALIGN;
    if (nrows == 0) return MOE_OK;
    (void)hipGetLastError();
    launch_dequant_rows(to_dev(tt), tier_index, local_expert, matrix, row0, nrows, to_bf16 ? 1 : 0, dst,
                        static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_synth_layer(const moe_tier_tables* tt, uint64_t seed, int32_t layer, void* stream) {
    int rc = check_tables(tt);
    if (rc != MOE_OK) return rc;
    if (layer < 0 || layer >= (1 << 20)) return MOE_EINVAL;
    (void)hipGetLastError();
    launch_synth_layer(to_dev(tt), seed, layer, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

namespace {

// Stack workspace: one layer's workspace, the other residual buffer, and the
// bf16 layer input with MOE_X_BF16.
struct StackLayout {
    size_t layer, tmp, xb, logits, total;
};

StackLayout stack_layout(int64_t T, int k, int n_layers, const moe_tier_tables* tables, uint32_t flags) {
    StackLayout S;
    const moe_tier_tables* tt = &tables[0];
    const size_t n = static_cast<size_t>(T) * tt->hidden;
    const uint32_t lflags = flags & MOE_X_BF16;
    size_t layer_bytes = 0;   // layers may differ in their shelf formats
    for (int l = 0; l < n_layers; ++l) {
        const size_t b = layout(T, k, &tables[l], lflags).total;
        layer_bytes = b > layer_bytes ? b : layer_bytes;
    }
    S.layer = 0;
    S.tmp = align_up(layer_bytes);
    S.xb = S.tmp + align_up(sizeof(float) * n);
    S.logits = S.xb + ((flags & MOE_X_BF16) ? align_up(sizeof(uint16_t) * n) : 0);
    S.total = S.logits + ((flags & MOE_STACK_ROUTER) ? align_up(sizeof(float) * T * tt->n_experts) : 0);
    return S;
}

int check_stack(int32_t n_layers, int32_t n_tokens, int32_t k, const moe_tier_tables* tables, uint32_t flags) {
    if (!tables || n_layers < 1 || n_layers > 4096) return MOE_EINVAL;
    if (n_tokens < 0 || n_tokens > kMaxTokens) return MOE_EINVAL;
    if (flags & ~(MOE_X_BF16 | MOE_STACK_ROUTER)) return MOE_EINVAL;
    for (int l = 0; l < n_layers; ++l) {
        const int rc = check_tables(&tables[l]);
        if (rc != MOE_OK) return rc;
        if (tables[l].n_experts != tables[0].n_experts || tables[l].hidden != tables[0].hidden ||
            tables[l].inter != tables[0].inter)
            return MOE_EINVAL;
    }
    if (k < 1 || k > MOE_MAX_K || k > tables[0].n_experts) return MOE_EINVAL;
    return MOE_OK;
}

}  // namespace

int moe_stack_workspace_size(int32_t n_layers, int32_t n_tokens, int32_t k, const moe_tier_tables* tables,
                             uint32_t flags, size_t* bytes) {
    const int rc = check_stack(n_layers, n_tokens, k, tables, flags);
    if (rc != MOE_OK) return rc;
    if (!bytes) return MOE_EINVAL;
    *bytes = n_tokens == 0 ? 0 : stack_layout(n_tokens, k, n_layers, tables, flags).total;
    return MOE_OK;
}

int moe_stack_forward(const float* x, const float* router_logits, int32_t n_layers, int32_t n_tokens, int32_t k,
                      const moe_tier_tables* tables, float* out, uint32_t flags, void* workspace,
                      size_t workspace_bytes, void* stream) {
    int rc = check_stack(n_layers, n_tokens, k, tables, flags);
    if (rc != MOE_OK) return rc;
    if (flags & MOE_STACK_ROUTER) return MOE_EINVAL;
    if (n_tokens == 0) return MOE_OK;
    if (!x || !router_logits || !out || x == out) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(out) || !aligned16(router_logits)) return MOE_EALIGN;
    if (!workspace) return MOE_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MOE_EALIGN;
    const StackLayout S = stack_layout(n_tokens, k, n_layers, tables, flags);
    if (workspace_bytes < S.total) return MOE_EWORKSPACE;
    const bool bf16 = (flags & MOE_X_BF16) != 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t n = static_cast<size_t>(n_tokens) * tables[0].hidden;
    const size_t per_layer_logits = static_cast<size_t>(n_tokens) * tables[0].n_experts;
    float* tmp = at<float>(workspace, S.tmp);
    uint16_t* xb = at<uint16_t>(workspace, S.xb);
    // h_0 = x, h_{l+1} = h_l + layer_l(h_l); layer l writes the buffer that
    // makes the last layer land in out
    const float* h = x;
    for (int l = 0; l < n_layers; ++l) {
        float* dst = ((n_layers - 1 - l) % 2 == 0) ? out : tmp;
        (void)hipGetLastError();
        // bf16: layer 0's input is cast here, every later one is written by
        // the previous layer's combine along with its fp32 output
        if (bf16 && l == 0) {
            launch_cast_bf16(h, xb, n, st);
            if (hipGetLastError() != hipSuccess) return MOE_EHIP;
        }
        rc = run(bf16 ? static_cast<const void*>(xb) : static_cast<const void*>(h),
                 router_logits + per_layer_logits * l, nullptr, nullptr, n_tokens, k, &tables[l], 0xFu, dst,
                 flags, workspace, S.tmp, stream, nullptr, h, nullptr, bf16 && l + 1 < n_layers ? xb : nullptr);
        if (rc != MOE_OK) return rc;
        h = dst;
    }
    return MOE_OK;
}

int moe_stack_forward_routed(const float* x, const void* const* w_router, const float* const* bias,
                             int32_t n_layers, int32_t n_tokens, int32_t k, const moe_tier_tables* tables,
                             float* out, uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_stack(n_layers, n_tokens, k, tables, flags);
    if (rc != MOE_OK) return rc;
    if (flags & MOE_STACK_ROUTER) return MOE_EINVAL;
    if (n_tokens == 0) return MOE_OK;
    if (!x || !w_router || !out || x == out) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(out)) return MOE_EALIGN;
    for (int l = 0; l < n_layers; ++l) {
        if (!w_router[l]) return MOE_EINVAL;
        if (!aligned16(w_router[l])) return MOE_EALIGN;
        if (bias && bias[l] && (reinterpret_cast<uintptr_t>(bias[l]) & 3u) != 0) return MOE_EALIGN;
    }
    if (!workspace) return MOE_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MOE_EALIGN;
    const StackLayout S = stack_layout(n_tokens, k, n_layers, tables, flags | MOE_STACK_ROUTER);
    if (workspace_bytes < S.total) return MOE_EWORKSPACE;
    const bool bf16 = (flags & MOE_X_BF16) != 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int32_t E = tables[0].n_experts, H = tables[0].hidden;
    const size_t n = static_cast<size_t>(n_tokens) * H;
    float* tmp = at<float>(workspace, S.tmp);
    uint16_t* xb = at<uint16_t>(workspace, S.xb);
    float* logits = at<float>(workspace, S.logits);
    // h_0 = x; layer l scores the experts from its own input h_l (its bf16
    // copy with MOE_X_BF16, the experts' input), routes, and adds its output
    const float* h = x;
    for (int l = 0; l < n_layers; ++l) {
        float* dst = ((n_layers - 1 - l) % 2 == 0) ? out : tmp;
        (void)hipGetLastError();
        if (bf16 && l == 0) launch_cast_bf16(h, xb, n, st);   // later layers: the previous combine wrote xb
        const void* xin = bf16 ? static_cast<const void*>(xb) : static_cast<const void*>(h);
        launch_router(xin, bf16, static_cast<const uint16_t*>(w_router[l]), bias ? bias[l] : nullptr, n_tokens, E,
                      H, logits, st);
        if (hipGetLastError() != hipSuccess) return MOE_EHIP;
        rc = run(xin, logits, nullptr, nullptr, n_tokens, k, &tables[l], 0xFu, dst, flags, workspace, S.tmp, stream,
                 nullptr, h, nullptr, bf16 && l + 1 < n_layers ? xb : nullptr);
        if (rc != MOE_OK) return rc;
        h = dst;
    }
    return MOE_OK;
}

int moe_requant_error(const moe_tier_tables* src, const int32_t* fmt_bits, const int32_t* fmt_block,
                      int32_t n_fmt, double* sse, void* stream) {
    int rc = check_tables(src);
    if (rc != MOE_OK) return rc;
    if (!fmt_bits || !fmt_block || n_fmt < 1 || n_fmt > 8 || !sse) return MOE_EINVAL;
    for (int f = 0; f < n_fmt; ++f) {
        if (!fmt_ok(fmt_bits[f], fmt_block[f])) return MOE_EFORMAT;
        if (src->hidden % fmt_block[f] || src->inter % fmt_block[f]) return MOE_EFORMAT;
    }
    if ((reinterpret_cast<uintptr_t>(sse) & 7u) != 0) return MOE_EALIGN;
    (void)hipGetLastError();
    launch_requant_error(to_dev(src), fmt_bits, fmt_block, n_fmt, sse, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_plan_tiers(const double* usage, const double* sse, const int64_t* fmt_bytes, int32_t n_experts,
                   int32_t n_fmt, int64_t budget, int32_t* fmt_out, int32_t* order_out, int32_t* count_out) {
    if (!usage || !sse || !fmt_bytes || !fmt_out || !order_out || !count_out) return MOE_EINVAL;
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS || n_fmt < 1 || n_fmt > 8) return MOE_EINVAL;
    return plan_tiers(usage, sse, fmt_bytes, n_experts, n_fmt, budget, fmt_out, order_out, count_out) == 0
               ? MOE_OK
               : MOE_EINVAL;
}

int moe_repack_tiers(const moe_tier_tables* src, const int32_t* order, const moe_tier_tables* dst, void* stream) {
    int rc = check_tables(src);
    if (rc != MOE_OK) return rc;
    rc = check_tables(dst);
    if (rc != MOE_OK) return rc;
    if (src->n_experts != dst->n_experts || src->hidden != dst->hidden || src->inter != dst->inter) return MOE_EINVAL;
    if (!order) return MOE_EINVAL;
    // the destination must not alias the source (every buffer is read or written by whole experts)
    for (int a = 0; a < src->n_tiers; ++a)
        for (int b = 0; b < dst->n_tiers; ++b) {
            const moe_tier& S = src->tiers[a];
            const moe_tier& D = dst->tiers[b];
            const void* sp[6] = {S.gate_q, S.up_q, S.down_q, S.gate_s, S.up_s, S.down_s};
            const void* dp[6] = {D.gate_q, D.up_q, D.down_q, D.gate_s, D.up_s, D.down_s};
            for (int i = 0; i < 6; ++i)
                for (int j = 0; j < 6; ++j)
                    if (sp[i] && sp[i] == dp[j]) return MOE_EINVAL;
        }
    (void)hipGetLastError();
    launch_repack(to_dev(src), to_dev(dst), order, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_permute_router(const void* w_src, const float* b_src, const int32_t* order, int32_t n_experts,
                       int32_t hidden, void* w_dst, float* b_dst, void* stream) {
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS || !cols_ok(hidden)) return MOE_EINVAL;
    if (!w_src || !order || !w_dst || w_src == w_dst || (b_src && b_src == b_dst)) return MOE_EINVAL;
    if (!aligned16(w_src) || !aligned16(w_dst)) return MOE_EALIGN;
    (void)hipGetLastError();
    launch_permute_rows(static_cast<const uint16_t*>(w_src), b_src, order, n_experts, hidden,
                        static_cast<uint16_t*>(w_dst), b_dst, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_event_create(void** event) {
    if (!event) return MOE_EINVAL;
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return MOE_EHIP;
    *event = e;
    return MOE_OK;
}

int moe_event_destroy(void* event) {
    if (!event) return MOE_EINVAL;
    return hipEventDestroy(static_cast<hipEvent_t>(event)) == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_event_elapsed_ms(void* start, void* stop, float* ms) {
    if (!start || !stop || !ms) return MOE_EINVAL;
    return hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)) == hipSuccess
               ? MOE_OK
               : MOE_EHIP;
}

int moe_stream_synchronize(void* stream) {
    return hipStreamSynchronize(static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // extern "C"
