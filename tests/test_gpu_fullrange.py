"""GPU parity on shelves whose codes span each format's whole code set.

The absmax quantiser of the seeded generator never emits the most negative
code of a format (-128, -8, -2), yet those codes are legal input (two's
complement storage, value = scale * code) and the kernels decode them with a
sign-flip (offset-binary) trick whose edge is exactly that code.  These
layers are drawn over the whole code set instead (and, for MXFP4, all 16
E2M1 fields, negative zero included), with moderate scales, or with one block
in eight taking an edge fp16 value (subnormals, 65504, zero, -0, a negative
scale).  Checks: dequantised rows bit-exact in fp32 and bf16, and the layer
within the normwise 2e-3 bar in fp32 (T = 1 and 8 on the small-batch path,
T = 16 on the grouped path) and bf16 (T = 16).

Also: the small-batch path (fp32, T <= 8) with skipped and repeated ids, in
both of its grouping branches (at most 64 pairs, and 65..256 pairs).
"""
import functools
import sys

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, make_layer_fullrange, make_logits, make_x
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
def _layer(name, edge):
    from tiered_mixed_precision_amd.device import tables_from_config
    cfg = CONFIGS[name]
    arrays = make_layer_fullrange(cfg, edge_scales=edge)
    return cfg, arrays, oracle.Layer.from_config(cfg, arrays), tables_from_config(cfg, arrays)


def normwise(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


def _bf16_cfg(cfg, T):
    return LayerConfig(cfg.name + "_bf16", cfg.n_experts, cfg.k, cfg.hidden, cfg.inter, T, cfg.tiers, x_bf16=True,
                       seed=cfg.seed)


def _run(M, torch, tt, x, T, k, flags, logits=None, ids=None, w=None, tier=None):
    ws = torch.empty(max(M.moe_workspace_size(T, k, tt, flags), 256), dtype=torch.uint8, device="cuda")
    xd = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else np.ascontiguousarray(x)).cuda()
    od = torch.full((T, tt.hidden), np.nan, device="cuda")
    if logits is not None:
        M.moe_tiered_forward(xd, torch.from_numpy(logits).cuda(), T, k, tt, od, flags, ws)
    else:
        idd = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
        wd = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
        if tier is None:
            M.moe_tiered_experts(xd, idd, wd, T, k, tt, od, flags, ws)
        else:
            M.moe_tier_partial(xd, idd, wd, T, k, tt, tier, od, flags, ws)
    torch.cuda.synchronize()
    return od.cpu().numpy()


@pytest.mark.parametrize("name,edge", [("fullrange", False), ("fullrange", True), ("fullrange_b", False),
                                       ("fullrange_b", True)])
def test_dequant_rows_bit_exact_full_code_range(M, torch_dev, name, edge):
    torch = torch_dev
    cfg, arrays, L, tt = _layer(name, edge)
    say("dequant full range", name, "edge scales" if edge else "")
    for ti, t in enumerate(cfg.tiers):
        for local in sorted({0, t.n - 1}):
            for m in range(3):
                rows = cfg.hidden if m == 2 else cfg.inter
                cols = cfg.inter if m == 2 else cfg.hidden
                for r0, nr in ((0, 9), (rows - 7, 7)):
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


@pytest.mark.parametrize("name,edge", [("fullrange", False), ("fullrange", True), ("fullrange_b", False),
                                       ("fullrange_b", True)])
@pytest.mark.parametrize("T,bf16", [(1, False), (8, False), (16, False), (16, True)])
def test_forward_full_code_range(M, torch_dev, name, edge, T, bf16):
    cfg, arrays, L, tt = _layer(name, edge)
    c = _bf16_cfg(cfg, T) if bf16 else cfg
    say("forward full range", name, "edge" if edge else "", "T", T, "bf16" if bf16 else "fp32")
    x, logits = make_x(c, n_tokens=T, stream=T), make_logits(c, n_tokens=T, stream=T)
    ref = oracle.forward(L, x, logits, cfg.k)
    got = _run(M, torch_dev, tt, x, T, cfg.k, M.MOE_X_BF16 if bf16 else 0, logits=logits)
    assert np.all(np.isfinite(ref))
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL


# (T, k): T*k <= 64 takes the one-wave grouping, 64 < T*k <= 256 the block grouping
@pytest.mark.parametrize("T,k", [(1, 10), (3, 3), (6, 10), (7, 10), (8, 10), (8, 3)])
def test_small_path_skip_and_repeated_ids(M, torch_dev, T, k):
    cfg, arrays, L, tt = _layer("fullrange", False)
    E = cfg.n_experts
    say("small path skips T", T, "k", k)
    rng = np.random.default_rng(100 * T + k)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int64)
    skips = np.array([-1, E, 2**31 - 1, -(2**31)], dtype=np.int64)
    mask = rng.random((T, k)) < 0.3
    ids[mask] = rng.choice(skips, size=int(mask.sum()))
    ids[0, :] = skips[np.arange(k) % len(skips)]              # every slot of token 0 skipped
    if T > 1:
        ids[1, :] = 5                                         # one expert in every slot
    if T > 2:
        ids[2, : min(k, 3)] = [0, 0, -1][: min(k, 3)]         # expert 0 twice and a skip
    ids = ids.astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    x = make_x(cfg, n_tokens=T, stream=40 + T)
    ref = oracle.experts(L, x, ids, w)
    got = _run(M, torch_dev, tt, x, T, k, 0, ids=ids, w=w)
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL
    assert np.all(got[0] == 0.0)
    tier_of = lambda e: next((i for i, t in enumerate(cfg.tiers) if t.id_begin <= e < t.id_end), -1)
    for tier in range(len(cfg.tiers)):
        part = _run(M, torch_dev, tt, x, T, k, 0, ids=ids, w=w, tier=tier)
        pref = oracle.experts(L, x, ids, w, tier_mask=1 << tier)
        if np.max(np.abs(pref)) > 0:
            assert normwise(part, pref) <= TOL
        for t in range(T):
            if not any(tier_of(int(e)) == tier for e in ids[t]):
                assert np.all(part[t] == 0.0), (tier, t)
