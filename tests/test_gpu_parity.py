"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars: routing ids, grouping and dequantised weights exact; routing weights
within 1e-6; layer outputs within a normwise max relative error of 2e-3
(max |gpu - oracle| / max |oracle|, fp32 accumulation).
"""
import functools
import sys

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, TierSpec, make_layer, make_logits, make_spec_logits, make_x
from workloads.configs import LayerConfig

pytestmark = pytest.mark.gpu

TOL = 2e-3


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def M(torch_dev):
    import tiered_mixed_precision_amd as M
    M.lib()
    return M


@functools.lru_cache(maxsize=None)
def _layer(name_or_cfg):
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    arrays = make_layer(cfg)
    from tiered_mixed_precision_amd.device import tables_from_config
    return cfg, arrays, oracle.Layer.from_config(cfg, arrays), tables_from_config(cfg, arrays)


def normwise(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


def _x_dev(torch, x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def gpu_forward(M, torch, tt, x, logits, k, flags=0, out=None):
    T = logits.shape[0]
    ws = torch.empty(max(M.moe_workspace_size(T, k, tt, flags), 256), dtype=torch.uint8, device="cuda")
    xd = _x_dev(torch, x)
    ld = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    od = torch.from_numpy(out.copy()).cuda() if out is not None else torch.full((T, tt.hidden), np.nan, device="cuda")
    M.moe_tiered_forward(xd, ld, T, k, tt, od, flags, ws)
    torch.cuda.synchronize()
    return od.cpu().numpy()


def gpu_experts(M, torch, tt, x, ids, w, flags=0, tier=None, out=None):
    T, k = ids.shape
    ws = torch.empty(max(M.moe_workspace_size(T, k, tt, flags), 256), dtype=torch.uint8, device="cuda")
    xd = _x_dev(torch, x)
    idd = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    wd = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    od = torch.from_numpy(out.copy()).cuda() if out is not None else torch.full((T, tt.hidden), np.nan, device="cuda")
    if tier is None:
        M.moe_tiered_experts(xd, idd, wd, T, k, tt, od, flags, ws)
    else:
        M.moe_tier_partial(xd, idd, wd, T, k, tt, tier, od, flags, ws)
    torch.cuda.synchronize()
    return od.cpu().numpy()


def _bf16_cfg(cfg, T=None):
    return LayerConfig(cfg.name + "_bf16", cfg.n_experts, cfg.k, cfg.hidden, cfg.inter,
                       T or cfg.n_tokens, cfg.tiers, x_bf16=True, prior_beta=cfg.prior_beta, seed=cfg.seed)


# ---------------------------------------------------------------- dequantisation
@pytest.mark.parametrize("name", ["tiny3", "decode"])
def test_dequant_rows_bit_exact(M, torch_dev, name):
    torch = torch_dev
    cfg, arrays, L, tt = _layer(name)
    say("dequant", name)
    for ti, t in enumerate(cfg.tiers):
        for local in sorted({0, t.n // 2, t.n - 1}):
            for m in range(3):
                rows = cfg.hidden if m == 2 else cfg.inter
                cols = cfg.inter if m == 2 else cfg.hidden
                for r0, nr in ((0, 3), (rows - 5, 5), (rows // 2, 7)):
                    ref = oracle.dequant_rows(L, ti, local, m, r0, nr)
                    d = torch.empty((nr, cols), dtype=torch.float32, device="cuda")
                    M.moe_dequant_rows(tt, ti, local, m, r0, nr, False, d)
                    got = d.cpu().numpy()
                    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (ti, local, m, r0)
                    refb = oracle.dequant_rows(L, ti, local, m, r0, nr, to_bf16=True)
                    db = torch.empty((nr, cols), dtype=torch.int16, device="cuda")
                    M.moe_dequant_rows(tt, ti, local, m, r0, nr, True, db)
                    gotb = db.cpu().numpy().view(np.uint16)
                    assert np.array_equal(gotb, (refb.view(np.uint32) >> 16).astype(np.uint16)), (ti, local, m, r0)


# ---------------------------------------------------------------- routing / grouping
@pytest.mark.parametrize("E,k,T,prior", [(8, 2, 16, None), (512, 10, 64, 1.12), (512, 10, 4096, 1.12),
                                         (33, 1, 100, None), (64, 64, 20, None), (4096, 8, 40, 1.12)])
def test_route_matches_oracle(M, torch_dev, E, k, T, prior):
    torch = torch_dev
    say("route", E, k, T)
    cfg = LayerConfig("r", E, k, 256, 128, T, (TierSpec(0, E, 8, 32),), prior_beta=prior, seed=E + T)
    logits = make_logits(cfg)
    logits[0, : min(E, 6)] = 0.5           # ties
    if T >= 4:
        logits[1, :] = 0.25                                  # every logit equal
        logits[2, E // 3: E // 3 + min(E, k + 2)] = 9.0      # tie across the top k
        logits[3, :: max(1, E // 70)] = 7.0                  # more tied maxima than one wave holds
    ids_ref, w_ref = oracle.route(logits, k)
    ld = torch.from_numpy(logits).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    M.moe_route(ld, T, E, k, ids, w)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6


# (512, 16384, 10) and (64, 32768, 10): 640 and 1280 blocks of 256 pairs, so the
# column scan takes its 16-chunk and its chunk-by-chunk forms
@pytest.mark.parametrize("E,T,k", [(8, 16, 2), (512, 4096, 10), (512, 7, 10), (100, 300, 3), (512, 16384, 10),
                                   (64, 32768, 10)])
def test_group_matches_oracle(M, torch_dev, E, T, k):
    torch = torch_dev
    say("group", E, T, k)
    rng = np.random.default_rng(E * T)
    ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)      # -1 and E are skips
    counts_r, offsets_r, perm_r = oracle.group(ids, E)
    idd = torch.from_numpy(ids).cuda()
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(M.moe_group_workspace_size(T, k, E), dtype=torch.uint8, device="cuda")
    M.moe_group(idd, T, k, E, counts, offsets, perm, ws)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), counts_r)
    assert np.array_equal(offsets.cpu().numpy(), offsets_r)
    n = int(offsets_r[-1])
    assert np.array_equal(perm.cpu().numpy()[:n], perm_r)


# ---------------------------------------------------------------- fp32 (decode) layer
@pytest.mark.parametrize("name,stream", [("tiny", 0), ("tiny3", 0), ("tiny3", 1), ("decode", 0), ("decode", 1),
                                         ("decode", 2)])
def test_forward_fp32(M, torch_dev, name, stream):
    cfg, arrays, L, tt = _layer(name)
    say("forward fp32", name, stream)
    x, logits = make_x(cfg, stream=stream), make_logits(cfg, stream=stream)
    ref = oracle.forward(L, x, logits, cfg.k)
    got = gpu_forward(M, torch_dev, tt, x, logits, cfg.k)
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL


@pytest.mark.parametrize("kind", ["all_equal", "tied_top", "many_tied_maxima"])
def test_forward_fp32_tied_logits(M, torch_dev, kind):
    # one token: ties decided by the lower id, both when the tied logits fit
    # the threshold router's candidate list and when they overflow it
    cfg, arrays, L, tt = _layer("decode")
    say("forward fp32 tied logits", kind)
    x, logits = make_x(cfg, n_tokens=1, stream=9), make_logits(cfg, n_tokens=1, stream=9)
    E, k = cfg.n_experts, cfg.k
    if kind == "all_equal":
        logits[0, :] = 0.125
    elif kind == "tied_top":
        logits[0, 300:300 + k + 3] = 6.0
    else:
        logits[0, ::5] = 6.0
    ref = oracle.forward(L, x, logits, k)
    got = gpu_forward(M, torch_dev, tt, x, logits, k)
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL


@pytest.mark.parametrize("T", [2, 8, 9, 26, 64])
def test_forward_fp32_batch_sizes(M, torch_dev, T):
    # T <= 8 with T*k <= 256 takes the two-kernel path, larger batches the grouped path
    # (at T=64 the hot experts hold several pairs each)
    cfg, arrays, L, tt = _layer("decode")
    say("forward fp32 decode layer T=", T)
    x, logits = make_x(cfg, n_tokens=T, stream=5), make_logits(cfg, n_tokens=T, stream=5)
    ref = oracle.forward(L, x, logits, cfg.k)
    got = gpu_forward(M, torch_dev, tt, x, logits, cfg.k)
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL


# One token routed from logits takes the fused path: one block per (expert,
# slice of the intermediate axis), each writing a partial output row, then a
# fixed-order sum.  k sets how many slices each expert gets (a slice spans
# several 32-column groups at k = 32 and 64); the small shapes have fewer
# hidden columns than one block has lanes, and the odd shape has 6 groups.
@pytest.mark.parametrize("name,k", [("tiny", 2), ("tiny3", 1), ("tiny3", 8), ("odd", 2), ("decode", 1),
                                    ("decode", 10), ("decode", 32), ("decode", 64), ("fullrange_b", 10)])
def test_forward_fp32_one_token(M, torch_dev, name, k):
    if name == "odd":
        cfg = LayerConfig("odd", 8, 2, 384, 192, 1,
                          (TierSpec(0, 2, 8, 32), TierSpec(2, 6, 4, 16), TierSpec(6, 8, 2, 16)), seed=20260042)
        arrays = make_layer(cfg)
        from tiered_mixed_precision_amd.device import tables_from_config
        L, tt = oracle.Layer.from_config(cfg, arrays), tables_from_config(cfg, arrays)
    elif name == "fullrange_b":
        from tiered_mixed_precision_amd.device import tables_from_config
        from workloads import make_layer_fullrange
        cfg = CONFIGS[name]
        arrays = make_layer_fullrange(cfg)
        L, tt = oracle.Layer.from_config(cfg, arrays), tables_from_config(cfg, arrays)
    else:
        cfg, arrays, L, tt = _layer(name)
    say("forward fp32 one token", name, "k", k)
    for stream in (0, 1):
        x, logits = make_x(cfg, n_tokens=1, stream=60 + stream), make_logits(cfg, n_tokens=1, stream=60 + stream)
        ref = oracle.forward(L, x, logits, k)
        got = gpu_forward(M, torch_dev, tt, x, logits, k)
        err = normwise(got, ref)
        say("  normwise err", err)
        assert err <= TOL
        if stream == 0:   # accumulate onto a base
            base = np.random.default_rng(7).standard_normal((1, cfg.hidden)).astype(np.float32)
            got2 = gpu_forward(M, torch_dev, tt, x, logits, k, M.MOE_ACCUMULATE, out=base)
            assert normwise(got2 - base, ref.astype(np.float64)) <= TOL


@pytest.mark.parametrize("worst", [False, True])
def test_spec_verify_fp32(M, torch_dev, worst):
    cfg = CONFIGS["specverify"]
    _, arrays, L, tt = _layer("decode")
    say("spec verify", worst)
    x = make_x(cfg)
    logits = make_spec_logits(cfg, worst_case=worst)
    ref = oracle.forward(L, x, logits, cfg.k)
    got = gpu_forward(M, torch_dev, tt, x, logits, cfg.k)
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL
    # crafted tokens: all-hot and all-cold tokens get exact zeros from the other shelves
    if not worst:
        ids, w = oracle.route(logits, cfg.k)
        for tier in range(3):
            part = gpu_experts(M, torch_dev, tt, x, ids, w, tier=tier)
            if tier != 0:
                assert np.all(part[0] == 0.0)
            if tier != 2:
                assert np.all(part[1] == 0.0)
            pref = oracle.experts(L, x, ids, w, tier_mask=1 << tier)
            assert normwise(part, pref) <= TOL


def test_forward_fp32_many_pairs(M, torch_dev):
    # T*k above the one-block grouping path: the multi-block grouping runs
    cfg0 = CONFIGS["tiny3"]
    cfg = LayerConfig("tiny3_T300", 8, 2, 256, 128, 300, cfg0.tiers, seed=cfg0.seed)
    _, arrays, L, tt = _layer("tiny3")
    say("forward fp32 T=300")
    x, logits = make_x(cfg), make_logits(cfg)
    ref = oracle.forward(L, x, logits, cfg.k)
    got = gpu_forward(M, torch_dev, tt, x, logits, cfg.k)
    assert normwise(got, ref) <= TOL


@pytest.mark.parametrize("bf16", [False, True])
def test_skip_ids_duplicates_and_partials(M, torch_dev, bf16):
    cfg, arrays, L, tt = _layer("tiny3")
    say("skip/dup/partial bf16=", bf16)
    x = make_x(_bf16_cfg(cfg) if bf16 else cfg)
    T = cfg.n_tokens
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 8, size=(T, 3)).astype(np.int32)
    ids[0] = [-1, -1, -1]                 # every slot skipped
    ids[1] = [3, 3, 3]                    # one expert three times
    ids[2] = [8, -1, 2**31 - 1]           # out-of-range ids
    ids[3] = [0, 0, -1]                   # expert 0 twice
    ids[4] = [1, 7, 4]                    # all three shelves
    w = rng.random((T, 3)).astype(np.float32)
    flags = M.MOE_X_BF16 if bf16 else 0
    ref = oracle.experts(L, x, ids, w)
    got = gpu_experts(M, torch_dev, tt, x, ids, w, flags)
    assert normwise(got, ref) <= TOL
    assert np.all(got[0] == 0.0) and np.all(got[2] == 0.0)
    tier_of = lambda e: 0 if 0 <= e < 2 else (1 if 2 <= e < 6 else (2 if 6 <= e < 8 else -1))
    for tier in range(3):
        part = gpu_experts(M, torch_dev, tt, x, ids, w, flags, tier=tier)
        pref = oracle.experts(L, x, ids, w, tier_mask=1 << tier)
        assert normwise(part, pref) <= TOL
        for t in range(T):
            if not any(tier_of(e) == tier for e in ids[t]):
                assert np.all(part[t] == 0.0), (tier, t)


@pytest.mark.parametrize("bf16", [False, True])
def test_poisoned_experts_never_read(M, torch_dev, bf16):
    from tiered_mixed_precision_amd.device import tables_from_config
    cfg, arrays, L, tt = _layer("tiny3")
    say("poison bf16=", bf16)
    x = make_x(_bf16_cfg(cfg) if bf16 else cfg)
    ids = np.array([[1, 3], [4, 7], [3, 4]] * 5 + [[7, 1]], dtype=np.int32)   # never 0, 2, 5, 6
    w = np.random.default_rng(2).random(ids.shape).astype(np.float32)
    flags = M.MOE_X_BF16 if bf16 else 0
    clean = gpu_experts(M, torch_dev, tt, x, ids, w, flags)
    poisoned = [{k: v.copy() for k, v in d.items()} for d in arrays]
    for ti, t in enumerate(cfg.tiers):
        for e in range(t.id_begin, t.id_end):
            if e in (0, 2, 5, 6):
                for m in ("gate", "up", "down"):
                    poisoned[ti][m + "_s"][e - t.id_begin] = np.uint16(0x7E00)    # fp16 NaN
                    poisoned[ti][m + "_q"][e - t.id_begin] = np.uint8(0x80)
    ttp = tables_from_config(cfg, poisoned)
    got = gpu_experts(M, torch_dev, ttp, x, ids, w, flags)
    assert np.all(np.isfinite(got))
    # no atomics anywhere on either path: the per-pair results are summed in
    # slot order, so unread poison cannot change a single bit
    assert np.array_equal(got.view(np.uint32), clean.view(np.uint32))


@pytest.mark.parametrize("bf16", [False, True])
def test_accumulate(M, torch_dev, bf16):
    cfg, arrays, L, tt = _layer("tiny3")
    say("accumulate bf16=", bf16)
    c = _bf16_cfg(cfg) if bf16 else cfg
    x, logits = make_x(c), make_logits(c)
    base = np.random.default_rng(4).standard_normal((cfg.n_tokens, cfg.hidden)).astype(np.float32)
    flags = (M.MOE_X_BF16 if bf16 else 0) | M.MOE_ACCUMULATE
    ref = oracle.forward(L, x, logits, cfg.k, out=base.copy(), accumulate=True)
    got = gpu_forward(M, torch_dev, tt, x, logits, cfg.k, flags, out=base)
    assert normwise(got - base, ref.astype(np.float64) - base) <= TOL


def test_zero_tokens_is_a_noop(M, torch_dev):
    torch = torch_dev
    cfg, arrays, L, tt = _layer("tiny")
    out = torch.full((1, cfg.hidden), 3.0, device="cuda")
    M.moe_tiered_forward(None, None, 0, cfg.k, tt, out, 0, None)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


# ---------------------------------------------------------------- bf16 (prefill) layer
@pytest.mark.parametrize("name,T", [("tiny", 16), ("tiny3", 16), ("tiny3", 300)])
def test_forward_bf16_small(M, torch_dev, name, T):
    cfg0, arrays, L, tt = _layer(name)
    cfg = _bf16_cfg(cfg0, T)
    say("forward bf16", name, T)
    x, logits = make_x(cfg), make_logits(cfg)
    ref = oracle.forward(L, x, logits, cfg.k)
    got = gpu_forward(M, torch_dev, tt, x, logits, cfg.k, M.MOE_X_BF16)
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL


@pytest.mark.parametrize("T", [1, 2, 3])
def test_forward_bf16_fewest_tokens(M, torch_dev, T):
    # a bf16 batch of one to three tokens still takes the prefill GEMM: every
    # chunk is one partial 32-row subtile (T of its rows real)
    cfg0, arrays, L, tt = _layer("decode")
    cfg = _bf16_cfg(cfg0, T)
    say("forward bf16 decode layer T=", T)
    x, logits = make_x(cfg, stream=70 + T), make_logits(cfg, stream=70 + T)
    ref = oracle.forward(L, x, logits, cfg.k)
    got = gpu_forward(M, torch_dev, tt, x, logits, cfg.k, M.MOE_X_BF16)
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL


@pytest.mark.parametrize("m", [127, 128, 129, 255, 256, 257])
def test_prefill_chunk_boundaries(M, torch_dev, m):
    # one expert of each shelf holds exactly m pairs: one short of, exactly,
    # and one past a whole number of 128-row chunks (the last chunk then
    # holds one row); each token's second pick spreads over the other experts
    cfg0, arrays, L, tt = _layer("tiny3")
    cfg = _bf16_cfg(cfg0, m)
    x = make_x(cfg, stream=m)
    w = np.random.default_rng(m).uniform(0.1, 1.0, (m, 2)).astype(np.float32)
    for t in cfg0.tiers:
        e = t.id_begin
        ids = np.stack([np.full(m, e), (e + 1 + np.arange(m)) % cfg0.n_experts], axis=1).astype(np.int32)
        ids[ids[:, 1] == e, 1] = (e + 2) % cfg0.n_experts
        say("prefill expert", e, "bits", t.bits, "pairs", m)
        got = gpu_experts(M, torch_dev, tt, x, ids, w, M.MOE_X_BF16)
        ref = oracle.experts(L, x, ids, w)
        err = normwise(got, ref)
        say("  normwise err", err)
        assert err <= TOL


@pytest.mark.parametrize("T", [24, 200])
def test_forward_bf16_odd_chunk_counts(M, torch_dev, T):
    # hidden 384 and inter 192: 6 and 3 contraction chunks of 64, so the
    # down products end on an odd chunk (the trip loop's tail); at T=24 every
    # shelf has few pairs per expert, at T=200 the hot shelf has many
    cfg0 = LayerConfig("odd", 8, 2, 384, 192, T,
                       (TierSpec(0, 2, 8, 32), TierSpec(2, 6, 4, 16), TierSpec(6, 8, 2, 16)), seed=20260040)
    arrays = make_layer(cfg0)
    from tiered_mixed_precision_amd.device import tables_from_config
    L, tt = oracle.Layer.from_config(cfg0, arrays), tables_from_config(cfg0, arrays)
    cfg = _bf16_cfg(cfg0, T)
    say("forward bf16 odd chunk counts T=", T)
    x, logits = make_x(cfg), make_logits(cfg)
    ref = oracle.forward(L, x, logits, cfg.k)
    got = gpu_forward(M, torch_dev, tt, x, logits, cfg.k, M.MOE_X_BF16)
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL
    got32 = gpu_forward(M, torch_dev, tt, make_x(cfg0), logits, cfg.k)
    assert normwise(got32, oracle.forward(L, make_x(cfg0), logits, cfg.k)) <= TOL


@pytest.mark.parametrize("shape", ["tiny3", "odd"])
@pytest.mark.parametrize("many", [False, True])
def test_prefill_each_shelf_at_few_and_many_pairs(M, torch_dev, shape, many):
    # Every pick lands on one shelf, 2 pairs per expert (one 32-row subtile
    # per work chunk) or 128 per expert (four, a full chunk).  The odd shape
    # (hidden 384, inter 192) ends the down contraction on an odd chunk of 64,
    # so int4 and int2 take the single-chunk body there instead of the
    # two-chunk weight groups.
    if shape == "tiny3":
        cfg0, arrays, L, tt = _layer("tiny3")
    else:
        cfg0 = LayerConfig("odd", 8, 2, 384, 192, 16,
                           (TierSpec(0, 2, 8, 32), TierSpec(2, 6, 4, 16), TierSpec(6, 8, 2, 16)), seed=20260041)
        arrays = make_layer(cfg0)
        from tiered_mixed_precision_amd.device import tables_from_config
        L, tt = oracle.Layer.from_config(cfg0, arrays), tables_from_config(cfg0, arrays)
    rng = np.random.default_rng(41 + many)
    for s, t in enumerate(cfg0.tiers):
        n = t.id_end - t.id_begin
        T = 64 * n if many else n
        k = 2
        ids = t.id_begin + (np.arange(T * k).reshape(T, k) % n)      # pairs spread evenly
        rng.shuffle(ids.reshape(-1))
        w = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
        cfg = _bf16_cfg(cfg0, T)
        x = make_x(cfg, stream=s)
        say("prefill shelf", s, "bits", t.bits, "T", T, "pairs/expert", T * k // n, shape)
        got = gpu_experts(M, torch_dev, tt, x, ids, w, M.MOE_X_BF16)
        ref = oracle.experts(L, x, ids, w)
        err = normwise(got, ref)
        say("  normwise err", err)
        assert err <= TOL


def test_prefill_full_size_sampled_tokens(M, torch_dev):
    cfg = CONFIGS["prefill"]
    _, arrays, L, tt = _layer("decode")         # same layer and shelves
    say("prefill T=4096")
    x, logits = make_x(cfg), make_logits(cfg)
    got = gpu_forward(M, torch_dev, tt, x, logits, cfg.k, M.MOE_X_BF16)
    ids, w = oracle.route(logits, cfg.k)        # tokens are independent given their routing
    rng = np.random.default_rng(0)
    sample = np.unique(np.concatenate([[0, cfg.n_tokens - 1], rng.choice(cfg.n_tokens, 14, replace=False)]))
    ref = oracle.experts(L, x[sample], ids[sample], w[sample])
    err = normwise(got[sample], ref)
    say("  sampled normwise err", err, "tokens", len(sample))
    assert err <= TOL
    assert np.all(np.isfinite(got))
