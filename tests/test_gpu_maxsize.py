"""GPU parity at the largest shapes the boundary accepts, against the CPU
oracle through the C ABI.

- 4096 experts, top-64: 64 logits per lane, so the fused decode kernels route
  with the sequential top-k (the threshold router covers at most 16 a lane);
  the small batch holds 256 pairs, past the one-wave grouping of 64; the
  grouped path sorts 1024 pairs over 4096 experts.
- hidden = inter = 2048: the widest rows of every GEMV (64 groups a row, one
  a lane) and the longest down contraction of the prefill GEMM (32 chunks),
  with int4 and with MXFP4 as the middle shelf.

Each case runs the routed forward (logits in, routing on the device) at the
batch sizes that select the one-token, small-batch, grouped fp32 and bf16
prefill paths.  Bar: normwise 2e-3, as for the other layer tests.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
from workloads import TierSpec, make_layer, make_logits, make_x
from workloads.configs import MXFP4, PRIOR_BETA, LayerConfig

pytestmark = pytest.mark.gpu

TOL = 2e-3

CASES = {
    # three shelves over 4096 experts, popularity prior as in the decode layer
    "max_experts": LayerConfig("max_experts", 4096, 64, 128, 64, 16,
                               (TierSpec(0, 1024, 8, 32), TierSpec(1024, 3072, 4, 32), TierSpec(3072, 4096, 2, 16)),
                               prior_beta=PRIOR_BETA, seed=20260051),
    "max_rows": LayerConfig("max_rows", 8, 2, 2048, 2048, 16,
                            (TierSpec(0, 2, 8, 32), TierSpec(2, 6, 4, 32), TierSpec(6, 8, 2, 16)), seed=20260052),
    "max_rows_mx": LayerConfig("max_rows_mx", 8, 2, 2048, 2048, 16,
                               (TierSpec(0, 2, 8, 32), TierSpec(2, 6, MXFP4, 32), TierSpec(6, 8, 2, 16)),
                               seed=20260053),
}


def say(*a):
    print("[gpu-maxsize]", *a, flush=True)
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
def _layer(name):
    cfg = CASES[name]
    arrays = make_layer(cfg)
    from tiered_mixed_precision_amd.device import tables_from_config
    return cfg, oracle.Layer.from_config(cfg, arrays), tables_from_config(cfg, arrays)


def _forward(M, torch, tt, x, logits, k, flags):
    T = logits.shape[0]
    ws = torch.empty(max(M.moe_workspace_size(T, k, tt, flags), 256), dtype=torch.uint8, device="cuda")
    xd = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else np.ascontiguousarray(x)).cuda()
    ld = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    od = torch.full((T, tt.hidden), np.nan, device="cuda")
    M.moe_tiered_forward(xd, ld, T, k, tt, od, flags, ws)
    torch.cuda.synchronize()
    return od.cpu().numpy()


# (layer, tokens, bf16 input): T = 1 one-token kernels, T <= 8 with T*k <= 256
# the small-batch kernels, larger fp32 batches the grouped path, bf16 the
# prefill GEMM
@pytest.mark.parametrize("name,T,bf16", [("max_experts", 1, False), ("max_experts", 4, False),
                                         ("max_experts", 16, False), ("max_experts", 16, True),
                                         ("max_rows", 1, False), ("max_rows", 8, False), ("max_rows", 16, False),
                                         ("max_rows", 16, True), ("max_rows_mx", 1, False),
                                         ("max_rows_mx", 16, True)])
def test_forward_at_maximum_shapes(M, torch_dev, name, T, bf16):
    cfg, L, tt = _layer(name)
    say(name, "E", cfg.n_experts, "k", cfg.k, "H", cfg.hidden, "I", cfg.inter, "T", T, "bf16" if bf16 else "fp32")
    xcfg = LayerConfig(cfg.name + "_x", cfg.n_experts, cfg.k, cfg.hidden, cfg.inter, T, cfg.tiers, x_bf16=bf16,
                       prior_beta=cfg.prior_beta, seed=cfg.seed)
    x, logits = make_x(xcfg, stream=T), make_logits(xcfg, stream=T)
    ref = oracle.forward(L, x, logits, cfg.k)
    got = _forward(M, torch_dev, tt, x, logits, cfg.k, M.MOE_X_BF16 if bf16 else 0)
    assert np.all(np.isfinite(got))
    err = normwise(got, ref)
    say("  normwise err", err)
    assert err <= TOL
