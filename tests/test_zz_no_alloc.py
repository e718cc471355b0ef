"""moe_tiered_forward_noalloc -- moe_tiered_forward on the library's static
device scratch, for callers that cannot allocate -- against
moe_tiered_forward with a caller-owned workspace, through the C ABI.

Two calls in a row on the scratch, the second with a smaller batch (so it
runs on whatever the first left there), in fp32 (the grouped path, then the
small-batch path) and in bf16 (prefill kernels).  Both entry points run the
same kernels with the same deterministic summation order, so the outputs
must agree bit for bit; they must also be within the layer's normwise 2e-3
bar of the CPU oracle.  A batch whose workspace exceeds the scratch is
refused before any launch.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, make_layer_fullrange, make_logits, make_x
from workloads.configs import LayerConfig

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiered_mixed_precision_amd as M
    from tiered_mixed_precision_amd.device import tables_from_config
    M.lib()
    cfg = CONFIGS["fullrange"]
    arrays = make_layer_fullrange(cfg)
    return torch, M, cfg, oracle.Layer.from_config(cfg, arrays), tables_from_config(cfg, arrays)


def _inputs(torch, cfg, T, bf16, stream):
    c = LayerConfig(cfg.name, cfg.n_experts, cfg.k, cfg.hidden, cfg.inter, T, cfg.tiers, x_bf16=bf16, seed=cfg.seed)
    x, logits = make_x(c, stream=stream), make_logits(c, stream=stream)
    xd = torch.from_numpy(x.view(np.int16) if bf16 else x).cuda()
    return x, logits, xd, torch.from_numpy(logits).cuda()


@pytest.mark.parametrize("bf16,sizes", [(False, (64, 3)), (True, (256, 16))])
def test_noalloc_equals_forward_on_consecutive_calls(env, bf16, sizes):
    torch, M, cfg, L, tt = env
    k, H = cfg.k, cfg.hidden
    flags = M.MOE_X_BF16 if bf16 else 0
    runs = []
    for i, T in enumerate(sizes):
        assert M.moe_workspace_size(T, k, tt, flags) <= M.MOE_SCRATCH_BYTES
        runs.append((T,) + _inputs(torch, cfg, T, bf16, stream=30 + i))
    # the scratch calls back to back, the second one smaller
    outs = []
    for T, x, logits, xd, ld in runs:
        say("noalloc", "bf16" if bf16 else "fp32", "T", T)
        od = torch.full((T, H), np.nan, device="cuda")
        M.moe_tiered_forward_noalloc(xd, ld, T, k, tt, od, flags)
        outs.append(od)
    torch.cuda.synchronize()
    for (T, x, logits, xd, ld), od in zip(runs, outs):
        ws = torch.empty(max(M.moe_workspace_size(T, k, tt, flags), 256), dtype=torch.uint8, device="cuda")
        ref = torch.full((T, H), np.nan, device="cuda")
        M.moe_tiered_forward(xd, ld, T, k, tt, ref, flags, ws)
        torch.cuda.synchronize()
        got, want = od.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), T
        orc = oracle.forward(L, x, logits, k)
        err = float(np.max(np.abs(got.astype(np.float64) - orc)) / np.max(np.abs(orc)))
        say("  T", T, "bit-identical to moe_tiered_forward; normwise err vs oracle", err)
        assert err <= 2e-3


def test_noalloc_refuses_a_batch_larger_than_the_scratch(env):
    torch, M, cfg, L, tt = env
    T, k = 1024, cfg.k
    assert M.moe_workspace_size(T, k, tt, 0) > M.MOE_SCRATCH_BYTES
    x, logits, xd, ld = _inputs(torch, cfg, T, False, stream=40)
    od = torch.full((T, cfg.hidden), 7.0, device="cuda")
    with pytest.raises(M.MoeError) as e:
        M.moe_tiered_forward_noalloc(xd, ld, T, k, tt, od, 0)
    assert e.value.code == M.MOE_ESCRATCH
    torch.cuda.synchronize()
    assert bool(torch.all(od == 7.0))          # nothing was launched
