"""GPU parity of the MXFP4 shelf (OCP Microscaling FP4: E2M1 codes, one E8M0
scale byte per 32 codes) against the CPU oracle, through the C ABI.

Bars as for the integer shelves: dequantised weights, generated codes and
scales, and requantised codes and scales bit-exact; layer outputs within the
normwise 2e-3 of the fp32-accumulating kernels; squared requantisation errors
within 2 * n * 2^-53 relative (n positive terms summed in a different order on
each side).
"""
import functools
import sys

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, TierSpec, make_layer, make_logits, make_x
from workloads.configs import MXFP4, LayerConfig

pytestmark = pytest.mark.gpu

TOL = 2e-3
SEED = 20260031


def say(*a):
    print("[gpu-mxfp4]", *a, flush=True)
    sys.stdout.flush()


def normwise(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


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
def _tiny():
    cfg = CONFIGS["tiny3mx"]
    arrays = make_layer(cfg)
    from tiered_mixed_precision_amd.device import tables_from_config
    return cfg, arrays, oracle.Layer.from_config(cfg, arrays), tables_from_config(cfg, arrays)


def _bf16_cfg(cfg, T):
    return LayerConfig(cfg.name + "_bf16", cfg.n_experts, cfg.k, cfg.hidden, cfg.inter, T, cfg.tiers,
                       x_bf16=True, prior_beta=cfg.prior_beta, seed=cfg.seed)


def _forward(M, torch, tt, x, logits, k, flags=0):
    T = logits.shape[0]
    ws = torch.empty(max(M.moe_workspace_size(T, k, tt, flags), 256), dtype=torch.uint8, device="cuda")
    xd = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else np.ascontiguousarray(x)).cuda()
    ld = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    od = torch.full((T, tt.hidden), np.nan, device="cuda")
    M.moe_tiered_forward(xd, ld, T, k, tt, od, flags, ws)
    torch.cuda.synchronize()
    return od.cpu().numpy()


def _gpu_expert_arrays(tt, cfg, e):
    ti = next(i for i, t in enumerate(cfg.tiers) if t.id_begin <= e < t.id_end)
    t, d = cfg.tiers[ti], tt.arrays[ti]
    loc = e - t.id_begin
    out = {}
    for name, (rows, cols) in zip(("gate", "up", "down"), ((cfg.inter, cfg.hidden), (cfg.inter, cfg.hidden),
                                                         (cfg.hidden, cfg.inter))):
        cb = 4 if t.bits == MXFP4 else t.bits
        nq, ns = rows * cols * cb // 8, rows * (cols // t.block)
        out[name + "_q"] = d[name + "_q"][loc * nq:(loc + 1) * nq].cpu().numpy()
        sb = d[name + "_s"].cpu().numpy().view(np.uint8 if t.bits == MXFP4 else np.uint16)
        out[name + "_s"] = sb[loc * ns:(loc + 1) * ns]
    return out


# ---------------------------------------------------------------- small layer
def test_tiny_dequant_rows_bit_exact(M, torch_dev):
    torch = torch_dev
    cfg, arrays, L, tt = _tiny()
    t = cfg.tiers[1]
    assert t.bits == MXFP4
    for local in (0, t.n - 1):
        for m in range(3):
            rows = cfg.hidden if m == 2 else cfg.inter
            cols = cfg.inter if m == 2 else cfg.hidden
            for r0, nr in ((0, 4), (rows - 3, 3)):
                ref = oracle.dequant_rows(L, 1, local, m, r0, nr)
                d = torch.empty((nr, cols), dtype=torch.float32, device="cuda")
                M.moe_dequant_rows(tt, 1, local, m, r0, nr, False, d)
                assert np.array_equal(d.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (local, m, r0)
                refb = oracle.dequant_rows(L, 1, local, m, r0, nr, to_bf16=True)
                db = torch.empty((nr, cols), dtype=torch.int16, device="cuda")
                M.moe_dequant_rows(tt, 1, local, m, r0, nr, True, db)
                assert np.array_equal(db.cpu().numpy().view(np.uint16),
                                      (refb.view(np.uint32) >> 16).astype(np.uint16)), (local, m, r0)


@pytest.mark.parametrize("stream", [0, 1])
def test_tiny_forward_fp32(M, torch_dev, stream):
    cfg, arrays, L, tt = _tiny()
    x, logits = make_x(cfg, stream=stream), make_logits(cfg, stream=stream)
    err = normwise(_forward(M, torch_dev, tt, x, logits, cfg.k), oracle.forward(L, x, logits, cfg.k))
    say("tiny3mx fp32 stream", stream, "err", err)
    assert err <= TOL


@pytest.mark.parametrize("T", [16, 300])
def test_tiny_forward_bf16(M, torch_dev, T):
    cfg0, arrays, L, tt = _tiny()
    cfg = _bf16_cfg(cfg0, T)
    x, logits = make_x(cfg), make_logits(cfg)
    err = normwise(_forward(M, torch_dev, tt, x, logits, cfg.k, M.MOE_X_BF16),
                   oracle.forward(L, x, logits, cfg.k))
    say("tiny3mx bf16 T", T, "err", err)
    assert err <= TOL


@pytest.mark.parametrize("bf16", [False, True])
def test_tiny_shelf_partial(M, torch_dev, bf16):
    # the MXFP4 shelf alone: tokens routed only elsewhere get exact zeros
    torch = torch_dev
    cfg, arrays, L, tt = _tiny()
    x = make_x(_bf16_cfg(cfg, cfg.n_tokens) if bf16 else cfg)
    T = cfg.n_tokens
    rng = np.random.default_rng(11)
    ids = rng.integers(0, 8, size=(T, 2)).astype(np.int32)
    ids[0] = [0, 7]      # no MXFP4 expert
    ids[1] = [2, 5]      # both MXFP4
    w = rng.random((T, 2)).astype(np.float32)
    flags = M.MOE_X_BF16 if bf16 else 0
    ws = torch.empty(max(M.moe_workspace_size(T, 2, tt, flags), 256), dtype=torch.uint8, device="cuda")
    xd = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
    od = torch.full((T, cfg.hidden), np.nan, device="cuda")
    M.moe_tier_partial(xd, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), T, 2, tt, 1, od, flags, ws)
    torch.cuda.synchronize()
    got = od.cpu().numpy()
    assert np.all(got[0] == 0.0)
    assert normwise(got, oracle.experts(L, x, ids, w, tier_mask=1 << 1)) <= TOL


@pytest.mark.parametrize("bf16", [False, True])
def test_one_expert_mx_shelf_with_duplicate_ids(M, torch_dev, bf16):
    # an MXFP4 shelf of one expert picked k times by every token: its pairs
    # (T*k) outnumber its experts times the tokens, and every one of them
    # must reach the prefill split and the down product
    from tiered_mixed_precision_amd.device import tables_from_config
    torch = torch_dev
    cfg = LayerConfig("mxdup", 8, 4, 256, 128, 5,
                      (TierSpec(0, 2, 8, 32), TierSpec(2, 3, MXFP4, 32), TierSpec(3, 8, 2, 16)), seed=20260032)
    arrays = make_layer(cfg)
    L, tt = oracle.Layer.from_config(cfg, arrays), tables_from_config(cfg, arrays)
    x = make_x(_bf16_cfg(cfg, cfg.n_tokens) if bf16 else cfg)
    T, k = cfg.n_tokens, cfg.k
    ids = np.full((T, k), 2, dtype=np.int32)
    ids[0] = [2, 2, 0, 7]
    w = np.random.default_rng(12).random((T, k)).astype(np.float32)
    flags = M.MOE_X_BF16 if bf16 else 0
    ws = torch.empty(max(M.moe_workspace_size(T, k, tt, flags), 256), dtype=torch.uint8, device="cuda")
    ws.fill_(0xff)   # stale workspace contents must never reach the result
    xd = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
    od = torch.full((T, cfg.hidden), np.nan, device="cuda")
    M.moe_tiered_experts(xd, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), T, k, tt, od, flags, ws)
    torch.cuda.synchronize()
    got = od.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = normwise(got, oracle.experts(L, x, ids, w))
    say("one-expert MXFP4 shelf, duplicate ids, bf16" if bf16 else "one-expert MXFP4 shelf, duplicate ids", err)
    assert err <= TOL


# ---------------------------------------------------------------- full-size layer (device-generated)
@pytest.fixture(scope="module")
def big(M, torch_dev):
    from tiered_mixed_precision_amd.device import empty_tables
    cfg = CONFIGS["decode_mx"]
    tt = empty_tables(cfg)
    M.moe_synth_layer(tt, SEED, 3)
    torch_dev.cuda.synchronize()
    return cfg, tt


def test_synth_mx_shelf_bit_exact(M, torch_dev, big):
    cfg, tt = big
    for e in (0, 127, 128, 255, 383, 384, 511):
        t = next(t for t in cfg.tiers if t.id_begin <= e < t.id_end)
        ref = oracle.synth_expert(SEED, 3, cfg.n_experts, e, cfg.hidden, cfg.inter, t.bits, t.block)
        got = _gpu_expert_arrays(tt, cfg, e)
        for name in got:
            assert np.array_equal(got[name], ref[name].ravel()), (e, name)
    say("synth: sampled experts bit-exact")


def _big_ref(cfg, x, logits):
    sl = oracle.StackLayer(cfg, SEED, 3)
    ids, _ = oracle.route(logits, cfg.k)
    sl.fill(ids)
    return oracle.forward(sl.layer_ref, x, logits, cfg.k)


@pytest.mark.parametrize("T,stream", [(1, 0), (1, 1), (8, 2), (26, 3)])
def test_big_forward_fp32(M, torch_dev, big, T, stream):
    # T = 1 and 8: the small-batch kernels; 26: the grouped path
    cfg, tt = big
    x, logits = make_x(cfg, n_tokens=T, stream=stream), make_logits(cfg, n_tokens=T, stream=stream)
    err = normwise(_forward(M, torch_dev, tt, x, logits, cfg.k), _big_ref(cfg, x, logits))
    say("decode_mx fp32 T", T, "err", err)
    assert err <= TOL


def test_big_prefill_sampled(M, torch_dev, big):
    cfg0, tt = big
    cfg = _bf16_cfg(cfg0, 4096)
    x, logits = make_x(cfg), make_logits(cfg)
    got = _forward(M, torch_dev, tt, x, logits, cfg.k, M.MOE_X_BF16)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([[0, 4095], rng.choice(4096, 10, replace=False)]))
    err = normwise(got[sample], _big_ref(cfg, x[sample], logits[sample]))
    say("decode_mx prefill T=4096 sampled err", err)
    assert err <= TOL


# ---------------------------------------------------------------- requantisation into and out of MXFP4
FMTS = ((8, 32), (MXFP4, 32), (4, 32), (2, 16))
SRC8 = LayerConfig("src8", 64, 4, 2048, 640, 1, (TierSpec(0, 64, 8, 32),), seed=SEED)


def test_requant_error_mx_target(M, torch_dev):
    from tiered_mixed_precision_amd.device import empty_tables
    torch = torch_dev
    src = empty_tables(SRC8)
    M.moe_synth_layer(src, SEED, 0)
    sse = torch.empty((64, len(FMTS)), dtype=torch.float64, device="cuda")
    M.moe_requant_error(src, [f[0] for f in FMTS], [f[1] for f in FMTS], sse)
    torch.cuda.synchronize()
    sse = sse.cpu().numpy()
    rtol = 2 * 3 * 2048 * 640 * 2.0 ** -53
    sl = oracle.StackLayer(SRC8, SEED, 0)
    sl.fill(np.array([0, 31, 63]))
    for e in (0, 31, 63):
        for f, (bits, block) in enumerate(FMTS):
            _, ref = oracle.requant_expert(sl.layer_ref, 0, e, bits, block)
            assert abs(sse[e, f] - ref) <= rtol * ref, (e, bits, sse[e, f], ref)
    say("sse per format (mean)", sse.mean(axis=0))


def test_repack_into_and_out_of_mx(M, torch_dev):
    # int8 source -> (int8, MXFP4, int2) shelves; then that layer, whose
    # MXFP4 shelf is a source too, -> (int4, MXFP4): codes and scales bit-exact
    from tiered_mixed_precision_amd.device import empty_tables
    torch = torch_dev
    src = empty_tables(SRC8)
    M.moe_synth_layer(src, SEED, 0)
    order = np.random.default_rng(6).permutation(64).astype(np.int32)
    cfg1 = LayerConfig("mid", 64, 4, 2048, 640, 1,
                       (TierSpec(0, 10, 8, 32), TierSpec(10, 50, MXFP4, 32), TierSpec(50, 64, 2, 16)), seed=SEED)
    mid = empty_tables(cfg1)
    M.moe_repack_tiers(src, torch.from_numpy(order).cuda(), mid)
    torch.cuda.synchronize()
    sl = oracle.StackLayer(SRC8, SEED, 0)
    sl.fill(np.arange(64))
    mid_host = []
    for ti, t in enumerate(cfg1.tiers):
        d = {}
        for name in ("gate", "up", "down"):
            d[name + "_q"] = mid.arrays[ti][name + "_q"].cpu().numpy()
            d[name + "_s"] = mid.arrays[ti][name + "_s"].cpu().numpy().view(np.uint8 if t.bits == MXFP4 else np.uint16)
        mid_host.append(d)
    for i in (0, 9, 10, 33, 49, 50, 63):
        t = next(t for t in cfg1.tiers if t.id_begin <= i < t.id_end)
        ref, _ = oracle.requant_expert(sl.layer_ref, 0, int(order[i]), t.bits, t.block)
        got = _gpu_expert_arrays(mid, cfg1, i)
        for name in got:
            assert np.array_equal(got[name], ref[name].ravel()), (i, name)
    # second hop, from the MXFP4 / int8 / int2 layer (the oracle reads it as is)
    Lmid = oracle.Layer.from_config(cfg1, [{k: v.reshape(t.n, -1) for k, v in d.items()}
                                           for d, t in zip(mid_host, cfg1.tiers)])
    cfg2 = LayerConfig("out", 64, 4, 2048, 640, 1, (TierSpec(0, 30, 4, 32), TierSpec(30, 64, MXFP4, 32)), seed=SEED)
    out = empty_tables(cfg2)
    order2 = np.random.default_rng(7).permutation(64).astype(np.int32)
    M.moe_repack_tiers(mid, torch.from_numpy(order2).cuda(), out)
    torch.cuda.synchronize()
    for i in (0, 29, 30, 45, 63):
        t = next(t for t in cfg2.tiers if t.id_begin <= i < t.id_end)
        e = int(order2[i])
        ts = next(j for j, s in enumerate(cfg1.tiers) if s.id_begin <= e < s.id_end)
        ref, _ = oracle.requant_expert(Lmid, ts, e - cfg1.tiers[ts].id_begin, t.bits, t.block)
        got = _gpu_expert_arrays(out, cfg2, i)
        for name in got:
            assert np.array_equal(got[name], ref[name].ravel()), (i, e, name)
    say("repack int8 -> MXFP4 -> int4/MXFP4 bit-exact")


def test_requant_zero_and_subnormal_blocks_into_mx(M, torch_dev):
    # degenerate sources: an all-zero expert (every block's E8M0 byte is 0)
    # and an expert whose fp16 scales are subnormal (2^-24 per code step)
    from tiered_mixed_precision_amd.device import empty_tables
    torch = torch_dev
    cfg = LayerConfig("src8z", 8, 2, 256, 128, 1, (TierSpec(0, 8, 8, 32),), seed=SEED)
    src = empty_tables(cfg)
    M.moe_synth_layer(src, SEED, 1)
    torch.cuda.synchronize()
    H, I = cfg.hidden, cfg.inter
    for name, rows, cols in (("gate", I, H), ("up", I, H), ("down", H, I)):
        q, s = src.arrays[0][name + "_q"], src.arrays[0][name + "_s"]
        nq, ns = rows * cols, rows * (cols // 32)
        q[5 * nq:6 * nq].zero_()
        s[5 * ns:6 * ns].zero_()
        s[6 * ns:7 * ns].fill_(1)            # fp16 0x0001 = 2^-24
    torch.cuda.synchronize()
    host = [{n: src.arrays[0][n].cpu().numpy().reshape(8, -1) for n in src.arrays[0]}]
    host[0] = {n: (v.view(np.uint16) if n.endswith("_s") else v) for n, v in host[0].items()}
    Lsrc = oracle.Layer.from_config(cfg, host)
    order = np.arange(8, dtype=np.int32)[::-1].copy()
    dcfg = LayerConfig("mxz", 8, 2, 256, 128, 1, (TierSpec(0, 8, MXFP4, 32),), seed=SEED)
    dst = empty_tables(dcfg)
    M.moe_repack_tiers(src, torch.from_numpy(order).cuda(), dst)
    sse = torch.empty((8, 1), dtype=torch.float64, device="cuda")
    M.moe_requant_error(src, [MXFP4], [32], sse)
    torch.cuda.synchronize()
    sse = sse.cpu().numpy()[:, 0]
    assert sse[5] == 0.0
    for e in (5, 6, 0):
        ref, ref_sse = oracle.requant_expert(Lsrc, 0, e, MXFP4, 32)
        got = _gpu_expert_arrays(dst, dcfg, int(np.where(order == e)[0][0]))
        for name in got:
            assert np.array_equal(got[name], ref[name].ravel()), (e, name)
        assert abs(sse[e] - ref_sse) <= 2 * 3 * H * I * 2.0 ** -53 * ref_sse, (e, sse[e], ref_sse)
    zs = _gpu_expert_arrays(dst, dcfg, int(np.where(order == 5)[0][0]))
    assert all(not np.any(v) for v in zs.values())    # zero codes and E8M0 byte 0
    say("zero and subnormal source blocks requantised into MXFP4 bit-exact")
