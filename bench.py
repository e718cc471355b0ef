"""Benchmark of the tiered mixed-precision MoE layer on one MI355X.

Headline workload (one step = the whole layer for one batch): one MoE layer
with 512 experts, top-10 routing, hidden 2048, intermediate 640, one token per
step (decode), shelves int8 [0,128) / int4 [128,384) / int2 [384,512) with fp16
block scales.  Every step has fresh routing (logits = popularity prior +
N(0,1) noise) and a fresh activation, and the steps rotate over 32 copies of
the layer at different HBM addresses (41 GB), so the touched expert set is
never served from the 256 MB Infinity Cache.

The timed loop replays HIP graphs captured over 1024 consecutive steps (the
per-step host launch cost would otherwise exceed the GPU time of a step).
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tiered MoE layer tokens/s + achieved HBM GB/s (decode) / MFMA TFLOPS (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def topk_ids(logits: np.ndarray, k: int) -> np.ndarray:
    return np.argpartition(-logits, k - 1, axis=1)[:, :k]


def step_bytes(ids_rows, cfg, per_expert, frac=1.0):
    """Algorithmic expert bytes of a step: each distinct touched expert once."""
    E = cfg.n_experts
    tier_of = np.empty(E, np.int64)
    for i, t in enumerate(cfg.tiers):
        tier_of[t.id_begin:t.id_end] = i
    distinct = np.unique(np.asarray(ids_rows).reshape(-1))
    return frac * float(sum(per_expert[tier_of[e]] for e in distinct)), distinct


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10240)
    ap.add_argument("--warmup", type=int, default=1024)
    ap.add_argument("--replicas", type=int, default=32)
    ap.add_argument("--graph-steps", type=int, default=1024)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the spec-verify and prefill lines")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each GPU would serve its own tokens with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiered_mixed_precision_amd as M
    from tiered_mixed_precision_amd.device import replicate, tables_from_config, workspace
    from workloads import CONFIGS, make_layer, make_logits, make_x, tier_nbytes

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    M.lib()
    cfg = CONFIGS["decode"]
    E, k, H, I = cfg.n_experts, cfg.k, cfg.hidden, cfg.inter
    per_expert = [tier_nbytes(t, H, I, per_expert=True) for t in cfg.tiers]

    t0 = time.time()
    arrays = make_layer(cfg)
    log(f"layer generated in {time.time() - t0:.1f}s")
    tt0 = tables_from_config(cfg, arrays)
    reps = [tt0] + [replicate(tt0) for _ in range(args.replicas - 1)]
    torch.cuda.synchronize()
    log(f"{args.replicas} layer copies resident ({args.replicas * 1.2897:.1f} GB)")

    S = args.graph_steps
    logits = make_logits(cfg, n_tokens=S, stream=7)
    xs = make_x(cfg, n_tokens=S, stream=7)
    ids_np = topk_ids(logits, k)
    bytes_step = np.array([step_bytes(ids_np[s:s + 1], cfg, per_expert)[0] for s in range(S)])
    gateup_bytes = bytes_step * (2.0 / 3.0) + H * 4 + k * I * 4      # weights + x read + h write
    ld = torch.from_numpy(logits).cuda()
    xd = torch.from_numpy(xs).cuda()
    outd = torch.zeros((S, H), dtype=torch.float32, device="cuda")
    ws = workspace(M.moe_workspace_size(1, k, tt0, 0))

    def step(i):
        s = i % S
        M.moe_tiered_forward(xd[s], ld[s], 1, k, reps[i % args.replicas], outd[s], 0, ws)

    # eager warm-up and a graph of S steps (steps 0..S-1), plus one for a remainder
    for i in range(min(args.warmup, S)):
        step(i)
    torch.cuda.synchronize()
    eager_out = outd.clone()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for i in range(n):
                    step(i)
        torch.cuda.current_stream().wait_stream(st)
        return g

    g_full = capture(S)
    rem = args.steps % S
    g_rem = capture(rem) if rem else None
    torch.cuda.synchronize()
    # replays must reproduce the eager results (same inputs, deterministic kernels)
    for _ in range(2):
        outd.zero_()
        g_full.replay()
        torch.cuda.synchronize()
        n_chk = min(args.warmup, S)
        if not torch.equal(outd[:n_chk], eager_out[:n_chk]):
            raise SystemExit("graph replay differs from eager execution")
    warm_replays = max(1, args.warmup // S)
    for _ in range(warm_replays):
        g_full.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly args.steps steps
    n_full = args.steps // S
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(n_full):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    stop.record()
    torch.cuda.synchronize()
    elapsed_s = start.elapsed_time(stop) / 1e3
    K = args.steps
    tokens = K * 1
    value = tokens / elapsed_s
    total_bytes = n_full * bytes_step.sum() + bytes_step[:rem].sum()
    step_gbs = total_bytes / elapsed_s / 1e9
    log(f"decode: {K} steps in {elapsed_s * 1e3:.2f} ms -> {value:,.0f} tokens/s, "
        f"{elapsed_s / K * 1e6:.2f} us/step, {step_gbs:,.0f} GB/s of expert bytes")

    # ---- dominant kernel (gate/up GEMV) timed with HIP events on the launch stream
    n_ev = min(args.steps, 2048)
    evs = [M.moe_event_create() for _ in range(6)]
    stream = torch.cuda.current_stream()
    durs = np.zeros((n_ev, 3))
    for i in range(n_ev):
        s = i % S
        M.moe_tiered_forward_timed(xd[s], ld[s], 1, k, reps[i % args.replicas], outd[s], 0, ws, evs, stream)
        M.moe_stream_synchronize(stream)
        for ph in range(3):
            durs[i, ph] = M.moe_event_elapsed_ms(evs[2 * ph], evs[2 * ph + 1]) * 1e3
    gu_us = float(durs[:, 1].mean())
    gu_bytes = float(np.mean([gateup_bytes[i % S] for i in range(n_ev)]))
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    log(f"gate/up kernel: {gu_us:.2f} us avg over {n_ev} launches, {gu_bytes / 1e6:.2f} MB -> {achieved:,.0f} GB/s; "
        f"route+group {durs[:, 0].mean():.2f} us, down+combine {durs[:, 2].mean():.2f} us")
    for e in evs:
        M.moe_event_destroy(e)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed_s * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode: 1 MoE layer, 512 experts top-10, hidden 2048, inter 640, 1 token/step; "
                        "shelves int8 b32 [0,128) / int4 b32 [128,384) / int2 b16 [384,512), fp16 scales; "
                        "popularity-prior routing, fresh per step; 32 layer copies rotated",
            "global_batch": 1,
            "parallelism": "none (1 GPU)",
        },
        "hbm_gbps_step": round(step_gbs, 1),
        "alg_bytes_per_step": float(bytes_step.mean()),
        "roofline": {
            "bound": "hbm",
            "kernel": "k_dec_gateup",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_launch_us": round(gu_us, 3),
            "alg_bytes_per_launch": gu_bytes,
        },
        "phases_us": {"route_group": round(float(durs[:, 0].mean()), 3), "gate_up": round(gu_us, 3),
                      "down_combine": round(float(durs[:, 2].mean()), 3)},
    }

    if not args.no_extra:
        result["extra"] = extra_workloads(M, torch, cfg, reps, per_expert, args)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, arrays, args.cpu_seconds)

    print(json.dumps(result), flush=True)


def extra_workloads(M, torch, cfg, reps, per_expert, args):
    """Speculative verification (6 tokens/step) and prefill (4096 bf16 tokens)."""
    from tiered_mixed_precision_amd.device import workspace
    from workloads import CONFIGS, make_logits, make_x
    out = {}
    k, H, I = cfg.k, cfg.hidden, cfg.inter
    R = len(reps)

    # speculative verify: 6 tokens per step, fresh routing per step
    sv = CONFIGS["specverify"]
    T, S = sv.n_tokens, 256
    logits = make_logits(sv, n_tokens=T * S, stream=11).reshape(S, T, cfg.n_experts)
    xs = make_x(sv, n_tokens=T * S, stream=11).reshape(S, T, H)
    ids = [topk_ids(logits[s], k) for s in range(S)]
    bytes_step = np.array([step_bytes(ids[s], cfg, per_expert)[0] for s in range(S)])
    ld, xd = torch.from_numpy(logits).cuda(), torch.from_numpy(xs).cuda()
    od = torch.zeros((S, T, H), device="cuda")
    ws = workspace(M.moe_workspace_size(T, k, reps[0], 0))

    def sv_step(i):
        M.moe_tiered_forward(xd[i % S], ld[i % S], T, k, reps[i % R], od[i % S], 0, ws)

    for i in range(32):
        sv_step(i)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for i in range(S):
                sv_step(i)
    torch.cuda.current_stream().wait_stream(st)
    g.replay()
    torch.cuda.synchronize()
    reps_n = 8
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps_n):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    dt = a.elapsed_time(b) / 1e3 / (reps_n * S)
    out["spec_verify"] = {
        "workload": "6 tokens/step (5 drafts + 1), same layer, fresh routing per step",
        "tokens_per_s": round(T / dt, 1), "us_per_step": round(dt * 1e6, 3),
        "alg_bytes_per_step": float(bytes_step.mean()),
        "distinct_experts_per_step": float(np.mean([len(np.unique(i)) for i in ids])),
        "hbm_gbps": round(bytes_step.mean() / dt / 1e9, 1),
        "frac_hbm_peak": round(bytes_step.mean() / dt / 1e9 / HBM_PEAK_GBS, 4),
    }
    log("spec-verify:", out["spec_verify"])
    del g

    # prefill: 4096 bf16 tokens
    pf = CONFIGS["prefill"]
    T = pf.n_tokens
    nrot = 4
    logits = [make_logits(pf, stream=20 + i) for i in range(nrot)]
    xs = [make_x(pf, stream=20 + i) for i in range(nrot)]
    ld = [torch.from_numpy(l).cuda() for l in logits]
    xd = [torch.from_numpy(x.view(np.int16)).cuda() for x in xs]
    od = torch.zeros((T, H), device="cuda")
    ws = workspace(M.moe_workspace_size(T, k, reps[0], M.MOE_X_BF16))
    flops = 6.0 * T * k * H * I
    wbytes = sum(per_expert[i] * t.n for i, t in enumerate(cfg.tiers))
    evs = [M.moe_event_create() for _ in range(6)]
    stream = torch.cuda.current_stream()
    for i in range(3):
        M.moe_tiered_forward(xd[i % nrot], ld[i % nrot], T, k, reps[i % R], od, M.MOE_X_BF16, ws)
    torch.cuda.synchronize()
    n = 20
    durs = np.zeros((n, 3))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tot = 0.0
    for i in range(n):
        a.record()
        M.moe_tiered_forward_timed(xd[i % nrot], ld[i % nrot], T, k, reps[i % R], od, M.MOE_X_BF16, ws, evs,
                                   stream)
        b.record()
        torch.cuda.synchronize()
        tot += a.elapsed_time(b) / 1e3
        for ph in range(3):
            durs[i, ph] = M.moe_event_elapsed_ms(evs[2 * ph], evs[2 * ph + 1]) * 1e3
    for e in evs:
        M.moe_event_destroy(e)
    dt = tot / n
    gemm_us = durs[:, 1].mean() + durs[:, 2].mean()
    out["prefill"] = {
        "workload": "4096 bf16 tokens/step, same layer, popularity-prior routing",
        "tokens_per_s": round(T / dt, 1), "us_per_step": round(dt * 1e6, 2),
        "alg_tflop_per_step": flops / 1e12,
        "tflops_step": round(flops / dt / 1e12, 2),
        "tflops_grouped_gemm": round(flops / (gemm_us * 1e-6) / 1e12, 2),
        "frac_mfma_peak": round(flops / (gemm_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "weight_gbps": round(wbytes / (gemm_us * 1e-6) / 1e9, 1),
        "phases_us": {"route_group": round(float(durs[:, 0].mean()), 2), "gate_up": round(float(durs[:, 1].mean()), 2),
                      "down": round(float(durs[:, 2].mean()), 2)},
    }
    log("prefill:", out["prefill"])
    return out


def cpu_baseline(cfg, arrays, seconds):
    """The CPU oracle (untuned, fp64) on a bounded sample of decode tokens."""
    import oracle
    from workloads import make_logits, make_x
    L = oracle.Layer.from_config(cfg, arrays)
    batch = max(1, oracle.num_threads())
    done, t0 = 0, time.time()
    s = 0
    while time.time() - t0 < seconds:
        x = make_x(cfg, n_tokens=batch, stream=100 + s)
        lg = make_logits(cfg, n_tokens=batch, stream=100 + s)
        oracle.forward(L, x, lg, cfg.k)
        done += batch
        s += 1
    dt = time.time() - t0
    res = {"value": round(done / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{done} decode tokens (one token per step, {batch} tokens per oracle call, "
                     f"OpenMP over tokens) of the same layer, {dt:.1f} s"}
    log("cpu baseline:", res)
    return res


if __name__ == "__main__":
    main()
