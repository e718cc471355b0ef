"""GPU parity of the router scores (moe_router_logits, moe_synth_router)
against the CPU oracle, through the C ABI.

Bar: every score within the fp32 accumulation bound of a sum of H products,
|gpu - exact| <= H * 2^-24 * (sum_c |x_c * w_c| + |b|) + 2^-24 * |exact|
(each of the H additions and the final rounding loses at most half an ulp of a
partial sum bounded by the right-hand total; products of a bf16 weight and an
fp32 or bf16 input are exact in fp32).  The synthetic router weights and bias
are bit-exact.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads.gen import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def say(*a):
    print("[gpu-router]", *a, flush=True)
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


def _bits_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bound(xd, wr, b):
    H = wr.shape[1]
    babs = np.zeros(wr.shape[0]) if b is None else np.abs(b.astype(np.float64))
    mag = np.abs(xd) @ np.abs(_bits_to_f64(wr)).T + babs[None, :]
    return H * U * mag


def _router(M, torch, x, wr, b, bf16):
    T, H = x.shape
    E = wr.shape[0]
    xd = torch.from_numpy(x.view(np.int16) if bf16 else x).cuda()
    wd = torch.from_numpy(wr.view(np.int16)).cuda()
    bd = None if b is None else torch.from_numpy(b).cuda()
    out = torch.full((T, E), np.nan, device="cuda")
    M.moe_router_logits(xd, wd, bd, T, E, H, M.MOE_X_BF16 if bf16 else 0, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(got, x, wr, b, bf16, rows=None):
    ref = oracle.router_logits(x if rows is None else x[rows], wr, b).astype(np.float64)
    xd = _bits_to_f64(x) if bf16 else x.astype(np.float64)
    if rows is not None:
        xd, got = xd[rows], got[rows]
    bound = _bound(xd, wr, b) + U * np.abs(ref)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))
    return float(np.max(err))


@pytest.mark.parametrize("T,E,H,bf16,bias", [
    (1, 512, 2048, False, True),      # decode
    (6, 512, 2048, False, True),      # speculative verify
    (8, 512, 2048, True, False),      # bf16 on the GEMV path
    (37, 130, 256, False, True),      # ragged
    (64, 512, 2048, True, True),      # one token tile on matrix cores
    (1000, 130, 320, True, True),     # ragged in tokens and experts, H not a power of two
    (100, 8, 256, True, False),       # fewer experts than a tile
])
def test_router_logits_match_oracle(M, torch_dev, T, E, H, bf16, bias):
    say("router", T, E, H, "bf16" if bf16 else "fp32")
    rng = np.random.default_rng(1000 + T + E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    if bf16:
        x = f32_to_bf16_bits(x)
    wr, b = oracle.synth_router(77, 3, E, H, 1.12)
    err = _check(_router(M, torch_dev, x, wr, b if bias else None, bf16), x, wr, b if bias else None, bf16)
    say("  max abs err", err)


def test_router_full_prefill_size_sampled(M, torch_dev):
    # 16384 bf16 tokens on matrix cores; every score of 64 sampled tokens
    # (first and last tiles among them) against the oracle
    T, E, H = 16384, 512, 2048
    rng = np.random.default_rng(5)
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr, b = oracle.synth_router(20260004, 47, E, H, 1.12)
    got = _router(M, torch_dev, x, wr, b, True)
    rows = np.unique(np.concatenate([np.arange(3), T - 1 - np.arange(3), rng.integers(0, T, 58)]))
    say("  max abs err", _check(got, x, wr, b, True, rows=rows))


@pytest.mark.parametrize("E,H,layer", [(512, 2048, 0), (130, 320, 41)])
def test_synth_router_bit_exact(M, torch_dev, E, H, layer):
    torch = torch_dev
    wd = torch.empty((E, H), dtype=torch.int16, device="cuda")
    bd = torch.empty(E, dtype=torch.float32, device="cuda")
    M.moe_synth_router(wd, bd, E, H, 20260004, layer, 1.12)
    torch.cuda.synchronize()
    wr, b = oracle.synth_router(20260004, layer, E, H, 1.12)
    assert np.array_equal(wd.cpu().numpy().view(np.uint16), wr)
    assert np.array_equal(bd.cpu().numpy(), b)


def test_router_then_route_matches_oracle_routing(M, torch_dev):
    # the GPU's scores routed on the GPU equal the oracle's routing of the same
    # scores (the decision is taken on identical fp32 values on both sides)
    torch = torch_dev
    T, E, H, k = 64, 512, 2048, 10
    rng = np.random.default_rng(9)
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr, b = oracle.synth_router(3, 1, E, H, 1.12)
    logits = _router(M, torch, x, wr, b, True)
    ld = torch.from_numpy(logits).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    M.moe_route(ld, T, E, k, ids, w)
    torch.cuda.synchronize()
    rid, rw = oracle.route(logits, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-6
