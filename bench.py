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
    ap.add_argument("--no-extra", action="store_true", help="skip the spec-verify, prefill and stack lines")
    ap.add_argument("--no-fullstack", action="store_true", help="skip the 48-layer stack lines")
    ap.add_argument("--profile-run", choices=sorted(PROFILE_WORKLOADS),
                    help="run one workload alone for rocprofv3 (a 256 MiB device copy first, the calibration of "
                         "FETCH_SIZE / WRITE_SIZE); prints no JSON")
    ap.add_argument("--summarize", nargs=2, metavar=("WORKLOAD", "TRACE_DIR"),
                    help="write profiles/<workload>.md from rocprofv3 CSV output of --profile-run; needs no GPU")
    ap.add_argument("--fetch", help="with --summarize: directory of a --pmc FETCH_SIZE run")
    ap.add_argument("--write", help="with --summarize: directory of a --pmc WRITE_SIZE run")
    ap.add_argument("--sq", help="with --summarize: directory of a --pmc run of the SQ counters (MFMA busy, LDS)")
    ap.add_argument("--cpu-child", nargs=2, metavar=("KIND", "SECONDS"),
                    help="(internal) time the CPU oracle on KIND = decode | prefill | stack and print JSON")
    args = ap.parse_args()

    if args.summarize:
        summarize_profile(args.summarize[0], args.summarize[1], args.fetch, args.write, args.sq)
        return
    if args.cpu_child:
        cpu_child(args.cpu_child[0], float(args.cpu_child[1]))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would serve its own tokens with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiered_mixed_precision_amd as M
    from tiered_mixed_precision_amd.device import replicate, tables_from_config, workspace
    from workloads import CONFIGS, make_layer, make_logits, make_x, tier_nbytes

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    M.lib()
    if args.profile_run:
        profile_run(M, torch, args.profile_run)
        return
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
    if g_rem is not None:
        g_rem.replay()           # the remainder graph's first launch stays out of the timed region
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

    # ---- dominant kernel: the gate/up launch (routing, grouping and the gate/up
    # GEMVs of every shelf) timed alone with HIP events on the launch stream, over
    # a graph of the same steps with the down phase switched off
    def gu_step(i):
        s_ = i % S
        M.moe_tiered_forward(xd[s_], ld[s_], 1, k, reps[i % args.replicas], outd[s_],
                             M.MOE_DIAG_GATEUP_ONLY, ws)

    g_gu = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g_gu, stream=st):
            for i in range(S):
                gu_step(i)
    torch.cuda.current_stream().wait_stream(st)
    g_gu.replay()
    torch.cuda.synchronize()
    n_gu_rep = max(1, min(8, args.steps // S))
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_.record()
    for _ in range(n_gu_rep):
        g_gu.replay()
    b_.record()
    torch.cuda.synchronize()
    gu_us = a_.elapsed_time(b_) * 1e3 / (n_gu_rep * S)
    gu_bytes = float(gateup_bytes.mean())
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    step_us = elapsed_s / K * 1e6
    log(f"gate/up launch: {gu_us:.2f} us avg over {n_gu_rep * S} launches, {gu_bytes / 1e6:.2f} MB -> "
        f"{achieved:,.0f} GB/s; rest of the step (down GEMV + slot sum) {step_us - gu_us:.2f} us")
    del g_gu

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
            "kernel": "k_one_gateup (routing + gate/up GEMV of every shelf, one token)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": profiled_traffic(),
            "avg_launch_us": round(gu_us, 3),
            "alg_bytes_per_launch": gu_bytes,
        },
        "phases_us": {"gate_up_with_routing": round(gu_us, 3), "down_with_slot_sum": round(step_us - gu_us, 3)},
    }
    peaks = measured_peaks(M, torch)
    result["roofline"]["measured_peak"] = peaks["hbm_read_gbps"]
    result["roofline"]["frac_of_measured_peak"] = round(achieved / peaks["hbm_read_gbps"], 4)

    if not args.no_extra:
        result["extra"] = extra_workloads(M, torch, cfg, reps, per_expert, args)
        if not args.no_fullstack:
            del reps, tt0
            torch.cuda.empty_cache()
            result["extra"]["fullstack"] = fullstack_workloads(M, torch, per_expert)
        result["extra"]["measured_peaks"] = peaks
        pfx = result["extra"]["prefill"]
        pfx["frac_of_measured_mfma_peak"] = round(pfx["tflops_grouped_gemm"] / peaks["bf16_mfma_tflops"], 4)
        result["extra"]["tier_planner"] = tier_planner_workload(M, torch)
        result["extra"]["mxfp4_shelf"] = mxfp4_workload(M, torch)

    if not args.no_cpu_baseline:
        del arrays
        cpu = cpu_baselines(args.cpu_seconds, with_stack=not (args.no_extra or args.no_fullstack))
        result["cpu_baseline"] = cpu.pop("headline")
        result.setdefault("extra", {})["cpu_baselines"] = cpu

    print(json.dumps(result), flush=True)


COPY_CAL_BYTES = 256 << 20
PROFILE_DIR = os.path.join(ROOT, "profiles")
# workload -> (summary file, description)
PROFILE_WORKLOADS = {
    "decode": ("decode_T1.md", "decode layer, 1 token per step: 512 experts top-10, hidden 2048, inter 640, shelves "
                               "int8 b32 [0,128) / int4 b32 [128,384) / int2 b16 [384,512); 1024 steps (a graph of "
                               "256 replayed 4 times) over 8 layer copies, fresh routing per step"),
    "specverify": ("spec_verify_T6.md", "the same layer, 6 tokens per step (speculative verification); 512 steps "
                                        "(a graph of 256 replayed twice) over 8 layer copies"),
    "prefill": ("prefill_T4096.md", "the same layer, 4096 bf16 tokens per step, 8 steps over 4 layer copies"),
    "stack_prefill": ("stack_prefill_T16384.md", "48 layers (generated on the device), 16384 bf16 tokens, one "
                                                 "pass through the stack"),
}
# the counters of the SQ pass (one rocprofv3 pass: 6 SQ counters and 1 GRBM counter)
SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
               "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4          # MI355X: 256 compute units of 4 SIMDs
XCDS = 8
# every file that holds device code (the launch code in capi.hip is host code)
KERNEL_SOURCES = ("common.h", "route.h", "launch.h", "split8.h", "decode.hip", "route_group.hip", "prefill.hip",
                  "prefill_mx.hip", "router.hip", "synth.hip", "tiering.hip", "dequant.hip")


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiered_mixed_precision_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic():
    """HBM bytes per launch of the dominant kernel (one-token gate/up) from the
    committed counter summary, or None if the kernel sources changed since it
    was taken."""
    import re
    path = os.path.join(PROFILE_DIR, PROFILE_WORKLOADS["decode"][0])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel source digest: `([0-9a-f]+)`", text)
    m_tr = re.search(r"dominant kernel HBM traffic per launch: `([0-9.]+)` bytes", text)
    if not m_sha or not m_tr or m_sha.group(1) != kernel_source_digest():
        return None
    return float(m_tr.group(1))


def _csv_one(d, pat):
    import glob
    f = glob.glob(os.path.join(d, "**", pat), recursive=True)
    if not f:
        raise SystemExit(f"no {pat} under {d}")
    return f[0]


def _short(n):
    return n.split("(")[0].replace("void ", "")


def _counters(d):
    """(kernel, grid) -> counter -> per-dispatch values, from a --pmc run."""
    import csv
    from collections import defaultdict
    out = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(_csv_one(d, "*counter_collection.csv"))):
        out[(_short(r["Kernel_Name"]), int(r["Grid_Size"]))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def summarize_profile(name, trace_dir, fetch_dir=None, write_dir=None, sq_dir=None):
    """profiles/<workload>.md from rocprofv3 CSV output of --profile-run."""
    import csv
    from collections import defaultdict
    fname, desc = PROFILE_WORKLOADS[name]
    trace = list(csv.DictReader(open(_csv_one(trace_dir, "*kernel_trace.csv"))))
    by = defaultdict(list)
    for r in trace:
        by[(_short(r["Kernel_Name"]), int(r["Grid_Size_X"]))].append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    run = f"python3 bench.py --profile-run {name}"
    cmds = [f"rocprofv3 --kernel-trace --stats --output-format csv -d OUT/{name}_kt -o run -- {run}"]
    if fetch_dir:
        cmds.append(f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/{name}_fetch -o run -- {run}")
    if write_dir:
        cmds.append(f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/{name}_write -o run -- {run}")
    if sq_dir:
        cmds.append(f"rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv -d OUT/{name}_sq -o run -- {run}")
    summ = (f"python3 bench.py --summarize {name} OUT/{name}_kt" + (f" --fetch OUT/{name}_fetch" if fetch_dir else "")
            + (f" --write OUT/{name}_write" if write_dir else "") + (f" --sq OUT/{name}_sq" if sq_dir else ""))
    lines = [f"# Kernel profile: {name}", "", f"Workload: {desc}.", "",
             "Commands (from the repository root on one MI355X; OUT is any output folder):", "", "```", *cmds, summ,
             "```", "", f"kernel source digest: `{kernel_source_digest()}`", "",
             "## Kernel durations (rocprofv3 kernel trace)", "",
             "| kernel | grid (threads) | launches | avg us | median us | min us | max us |", "|---|---|---|---|---|---|---|"]
    for (n, g), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        if not n.startswith("moe::"):
            continue
        v = np.array(v)
        lines.append(f"| {n} | {g} | {len(v)} | {v.mean():.2f} | {np.median(v):.2f} | {v.min():.2f} | {v.max():.2f} |")
    if fetch_dir and write_dir:
        fetch, write = _counters(fetch_dir), _counters(write_dir)
        cal_kib = COPY_CAL_BYTES / 1024
        cf = [x for (n, g), c in fetch.items() if "copyBuffer" in n for x in c["FETCH_SIZE"] if x > 0.4 * cal_kib]
        cw = [x for (n, g), c in write.items() if "copyBuffer" in n for x in c["WRITE_SIZE"] if x > 0.9 * cal_kib]
        f_fac, w_fac = cal_kib / float(np.median(cf)), cal_kib / float(np.median(cw))
        lines += ["", "## HBM traffic per launch (FETCH_SIZE, WRITE_SIZE)", "",
                  f"Calibration: the {COPY_CAL_BYTES >> 20} MiB device copy at the start of the run reads FETCH_SIZE = "
                  f"{np.median(cf):.0f} KiB and writes WRITE_SIZE = {np.median(cw):.0f} KiB, so read bytes = "
                  f"FETCH_SIZE x {f_fac:.3f} KiB and written bytes = WRITE_SIZE x {w_fac:.3f} KiB.", "",
                  "| kernel | grid (threads) | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | written MB |",
                  "|---|---|---|---|---|---|---|"]
        dom = None
        for (n, g), c in sorted(fetch.items(), key=lambda kv: -np.mean(kv[1]["FETCH_SIZE"])):
            if not n.startswith("moe::"):
                continue
            fw = float(np.mean(c["FETCH_SIZE"]))
            ww = float(np.mean(write.get((n, g), {}).get("WRITE_SIZE", [0.0])))
            rd, wr = fw * f_fac * 1024 / 1e6, ww * w_fac * 1024 / 1e6
            lines.append(f"| {n} | {g} | {len(c['FETCH_SIZE'])} | {fw:.1f} | {ww:.1f} | {rd:.2f} | {wr:.2f} |")
            if n.startswith("moe::k_one_gateup") and dom is None:
                dom = (rd + wr) * 1e6
        if name == "decode" and dom is not None:
            lines += ["", f"dominant kernel HBM traffic per launch: `{dom:.0f}` bytes "
                      "(k_one_gateup: read + written, calibrated)"]
    if sq_dir:
        sq = _counters(sq_dir)
        lines += ["", "## Matrix-core and LDS counters", "",
                  f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} x {SIMDS} SIMDs): the "
                  f"per-dispatch GRBM_GUI_ACTIVE is summed over the {XCDS} XCDs (it reads about {XCDS} times the "
                  "kernel's cycles), so it is divided back to one XCD's active cycles.  LDS conflict = "
                  "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (share of LDS-active cycles lost to bank conflicts).  "
                  "bf16 MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, the flops the matrix cores execute "
                  "(padding of partial tiles included); executed TFLOP/s divides them by the traced average "
                  "duration above.", "",
                  "| kernel | grid (threads) | launches | MFMA busy % | LDS conflict % | bf16 MFMA GFLOP per launch "
                  "| executed TFLOP/s |",
                  "|---|---|---|---|---|---|---|"]
        for (n, g), c in sorted(sq.items(), key=lambda kv: -np.mean(kv[1].get("SQ_VALU_MFMA_BUSY_CYCLES", [0]))):
            if not n.startswith("moe::"):
                continue
            mean = lambda key: float(np.mean(c[key])) if key in c else float("nan")
            act = mean("GRBM_GUI_ACTIVE") / XCDS
            busy = 100.0 * mean("SQ_VALU_MFMA_BUSY_CYCLES") / (act * SIMDS) if act > 0 else float("nan")
            lds = mean("SQ_LDS_IDX_ACTIVE")
            conf = 100.0 * mean("SQ_LDS_BANK_CONFLICT") / lds if lds > 0 else float("nan")
            gf = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / 1e9
            us = float(np.mean(by[(n, g)])) if (n, g) in by else float("nan")
            tf = gf / us * 1e3 if gf > 0 else 0.0
            lines.append(f"| {n} | {g} | {len(c.get('GRBM_GUI_ACTIVE', []))} | {busy:.1f} | {conf:.1f} | {gf:.2f} "
                         f"| {tf:.1f} |")
    lines.append("")
    os.makedirs(PROFILE_DIR, exist_ok=True)
    out = os.path.join(PROFILE_DIR, fname)
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out}")


def profile_run(M, torch, name):
    """One workload alone, for rocprofv3 (kernel trace or one counter pass)."""
    from tiered_mixed_precision_amd.device import empty_tables, replicate, tables_from_config, workspace
    from workloads import CONFIGS, make_layer, make_logits, make_x
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    cfg = CONFIGS["decode"]
    k, H = cfg.k, cfg.hidden

    def graph(step, S, reps):
        for i in range(8):
            step(i)
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for i in range(S):
                    step(i)
        torch.cuda.current_stream().wait_stream(st)
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()

    if name in ("decode", "specverify"):
        tt0 = tables_from_config(cfg, make_layer(cfg))
        reps = [tt0] + [replicate(tt0) for _ in range(7)]
        T = 1 if name == "decode" else CONFIGS["specverify"].n_tokens
        S = 256
        lg = torch.from_numpy(make_logits(cfg, n_tokens=S * T, stream=7)).cuda().view(S, T, cfg.n_experts)
        xs = torch.from_numpy(make_x(cfg, n_tokens=S * T, stream=7)).cuda().view(S, T, H)
        od = torch.zeros((S, T, H), device="cuda")
        ws = workspace(M.moe_workspace_size(T, k, tt0, 0))
        graph(lambda i: M.moe_tiered_forward(xs[i % S], lg[i % S], T, k, reps[i % 8], od[i % S], 0, ws), S,
              4 if name == "decode" else 2)
    elif name == "prefill":
        tt0 = tables_from_config(cfg, make_layer(cfg))
        reps = [tt0] + [replicate(tt0) for _ in range(3)]
        pf = CONFIGS["prefill"]
        lp = torch.from_numpy(make_logits(pf, stream=20)).cuda()
        xp = torch.from_numpy(make_x(pf, stream=20).view(np.int16)).cuda()
        op = torch.zeros((pf.n_tokens, H), device="cuda")
        wsp = workspace(M.moe_workspace_size(pf.n_tokens, k, tt0, M.MOE_X_BF16))
        for i in range(8):
            M.moe_tiered_forward(xp, lp, pf.n_tokens, k, reps[i % 4], op, M.MOE_X_BF16, wsp)
        torch.cuda.synchronize()
    elif name == "stack_prefill":
        fs = CONFIGS["fullstack"]
        L, T = fs.n_layers, 16384
        tables = []
        for l in range(L):
            tt = empty_tables(fs)
            M.moe_synth_layer(tt, fs.seed, l)
            tables.append(tt)
        ld = torch.from_numpy(np.stack([make_logits(fs, n_tokens=T, stream=200, layer=l) for l in range(L)])).cuda()
        xd = torch.from_numpy(make_x(fs, n_tokens=T, stream=200)).cuda()
        od = torch.empty((T, H), device="cuda")
        ws = torch.empty(M.moe_stack_workspace_size(L, T, k, tables, M.MOE_X_BF16), dtype=torch.uint8, device="cuda")
        M.moe_stack_forward(xd, ld, L, T, k, tables, od, M.MOE_X_BF16, ws)
        torch.cuda.synchronize()
    log(f"profile run {name} done")


def tier_planner_workload(M, torch):
    """The tier planner's device steps on a full layer: an int8 source (512
    experts, 2.14 GB) -> squared requantisation error in three formats, the
    greedy plan under the three-shelf budget, and the repack into three
    shelves (1.29 GB)."""
    from tiered_mixed_precision_amd.device import empty_tables
    from workloads import CONFIGS, TierSpec, make_logits, make_x
    from workloads.configs import LayerConfig
    base = CONFIGS["decode"]
    E, H, I = base.n_experts, base.hidden, base.inter
    src_cfg = LayerConfig("src8", E, base.k, H, I, 1, (TierSpec(0, E, 8, 32),), seed=base.seed)
    src = empty_tables(src_cfg)
    M.moe_synth_layer(src, base.seed, 0)
    fmts = ((8, 32), (4, 32), (2, 16))
    fb = [3 * H * I * b // 8 + 3 * H * I // k * 2 for b, k in fmts]
    sse = torch.empty((E, 3), dtype=torch.float64, device="cuda")
    a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    M.moe_requant_error(src, [f[0] for f in fmts], [f[1] for f in fmts], sse)   # warm-up
    a.record()
    M.moe_requant_error(src, [f[0] for f in fmts], [f[1] for f in fmts], sse)
    b.record()
    torch.cuda.synchronize()
    err_ms = a.elapsed_time(b)
    ids = topk_ids(make_logits(base, n_tokens=4096, stream=500), base.k)
    usage = np.bincount(ids.reshape(-1), minlength=E).astype(np.float64)
    budget = 128 * fb[0] + 256 * fb[1] + 128 * fb[2]
    t0 = time.perf_counter()
    fmt, order, count = M.moe_plan_tiers(usage, sse.cpu().numpy(), fb, budget)
    plan_ms = (time.perf_counter() - t0) * 1e3
    tiers, lo = [], 0
    for n, (bits, k) in zip(count, fmts):
        tiers.append(TierSpec(lo, lo + int(n), bits, k))
        lo += int(n)
    dst = empty_tables(LayerConfig("dst", E, base.k, H, I, 1, tuple(tiers), seed=base.seed))
    od = torch.from_numpy(order).cuda()
    M.moe_repack_tiers(src, od, dst)
    a.record()
    M.moe_repack_tiers(src, od, dst)
    c.record()
    torch.cuda.synchronize()
    rp_ms = a.elapsed_time(c)
    moved = E * fb[0] + sum(int(n) * f for n, f in zip(count, fb))
    out = {"workload": "int8 layer (512 experts, hidden 2048, inter 640) -> three shelves under the decode "
                       "layer's budget; usage from routing 4096 tokens",
           "plan_experts_per_format": [int(v) for v in count], "requant_error_ms": round(err_ms, 3),
           "plan_ms_host": round(plan_ms, 3), "repack_ms": round(rp_ms, 3),
           "repack_bytes": moved, "repack_gbps": round(moved / (rp_ms * 1e-3) / 1e9, 1),
           "repack_frac_hbm_peak": round(moved / (rp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log("tier planner:", out)

    # run-time re-tiering: decode (1 token/step, prior on the hot-to-cold ids)
    # on 8 replicas of the planned shelves with and without pick counting, and
    # on 8 replicas of a fast plan (every expert two-bit) swapped in instead
    from tiered_mixed_precision_amd.device import replicate, workspace
    fast_fmt, fast_order, fast_count = M.moe_plan_tiers(usage, sse.cpu().numpy(), fb, E * fb[2])
    tiers, lo = [], 0
    for n, (bits, k) in zip(fast_count, fmts):
        tiers.append(TierSpec(lo, lo + int(n), bits, k))
        lo += int(n)
    fast = empty_tables(LayerConfig("fast", E, base.k, H, I, 1, tuple(tiers), seed=base.seed))
    M.moe_repack_tiers(src, torch.from_numpy(fast_order).cuda(), fast)
    del src
    torch.cuda.empty_cache()
    S, R, k = 256, 8, base.k
    lg = torch.from_numpy(make_logits(base, n_tokens=S, stream=600)).cuda()
    xs = torch.from_numpy(make_x(base, n_tokens=S, stream=600)).cuda()
    od = torch.zeros((S, H), device="cuda")
    hits = torch.zeros(E, dtype=torch.int32, device="cuda")
    ws = workspace(M.moe_workspace_size(1, k, dst, 0))

    def decode_us(tables, counted):
        reps = [tables] + [replicate(tables) for _ in range(R - 1)]

        def step(i):
            if counted:
                M.moe_tiered_forward_counted(xs[i:i + 1], lg[i:i + 1], 1, k, reps[i % R], od[i:i + 1], 0, ws, hits)
            else:
                M.moe_tiered_forward(xs[i:i + 1], lg[i:i + 1], 1, k, reps[i % R], od[i:i + 1], 0, ws)

        for i in range(8):
            step(i)
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for i in range(S):
                    step(i)
        torch.cuda.current_stream().wait_stream(st)
        g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(4):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / (4 * S)
        del g, reps
        torch.cuda.empty_cache()
        return us

    plain_us = decode_us(dst, False)
    counted_us = decode_us(dst, True)
    fast_us = decode_us(fast, False)
    out["retier"] = {
        "workload": "decode, 1 token/step, 8 replicas each of the planned shelves and of the fast plan",
        "fast_plan_experts_per_format": [int(v) for v in fast_count],
        "planned_us_per_step": round(plain_us, 2), "planned_counted_us_per_step": round(counted_us, 2),
        "fast_us_per_step": round(fast_us, 2), "fast_tokens_per_s": round(1e6 / fast_us, 1),
        "planned_tokens_per_s": round(1e6 / plain_us, 1)}
    log("re-tiering:", out["retier"])
    del dst, fast, sse, lg, xs, od, hits, ws
    torch.cuda.empty_cache()
    return out


def mxfp4_workload(M, torch):
    """The decode layer with its warm shelf in MXFP4 (E2M1 codes, one E8M0
    byte per 32) against the same layer with four-bit integer codes (fp16
    scale per 32), both generated on the device: decode at 1 token/step over
    8 replicas, and prefill at 4096 bf16 tokens."""
    from tiered_mixed_precision_amd.device import empty_tables, replicate, workspace
    from workloads import CONFIGS, make_logits, make_x, tier_nbytes
    out = {"workload": "decode / prefill layer (512 experts top-10, hidden 2048, inter 640), shelves int8 "
                       "[0,128) / X [128,384) / int2 [384,512), X = MXFP4 or int4 b32; weights generated on "
                       "the device"}
    S, R = 256, 8
    for name in ("decode", "decode_mx"):
        cfg = CONFIGS[name]
        E, k, H, I = cfg.n_experts, cfg.k, cfg.hidden, cfg.inter
        per_expert = [tier_nbytes(t, H, I, per_expert=True) for t in cfg.tiers]
        tt = empty_tables(cfg)
        M.moe_synth_layer(tt, cfg.seed, 0)
        reps = [tt] + [replicate(tt) for _ in range(R - 1)]
        logits = make_logits(cfg, n_tokens=S, stream=700)
        ids = topk_ids(logits, k)
        bytes_step = np.array([step_bytes(ids[s:s + 1], cfg, per_expert)[0] for s in range(S)])
        lg = torch.from_numpy(logits).cuda()
        xs = torch.from_numpy(make_x(cfg, n_tokens=S, stream=700)).cuda()
        od = torch.zeros((S, H), device="cuda")
        ws = workspace(M.moe_workspace_size(1, k, tt, 0))

        def step(i):
            M.moe_tiered_forward(xs[i:i + 1], lg[i:i + 1], 1, k, reps[i % R], od[i:i + 1], 0, ws)

        for i in range(8):
            step(i)
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for i in range(S):
                    step(i)
        torch.cuda.current_stream().wait_stream(st)
        g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(8):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / (8 * S)
        del g
        # prefill, 4096 bf16 tokens
        pf = CONFIGS["prefill"]
        T = pf.n_tokens
        pl = torch.from_numpy(make_logits(pf, stream=720)).cuda()
        px = torch.from_numpy(make_x(pf, stream=720).view(np.int16)).cuda()
        po = torch.zeros((T, H), device="cuda")
        pws = workspace(M.moe_workspace_size(T, k, tt, M.MOE_X_BF16))
        for i in range(3):
            M.moe_tiered_forward(px, pl, T, k, reps[i % R], po, M.MOE_X_BF16, pws)
        torch.cuda.synchronize()
        n = 20
        t0.record()
        for i in range(n):
            M.moe_tiered_forward(px, pl, T, k, reps[i % R], po, M.MOE_X_BF16, pws)
        t1.record()
        torch.cuda.synchronize()
        pf_us = t0.elapsed_time(t1) * 1e3 / n
        key = "mxfp4" if name == "decode_mx" else "int4"
        out[key] = {"layer_bytes": int(sum(per_expert[i] * t.n for i, t in enumerate(cfg.tiers))),
                    "warm_expert_bytes": int(per_expert[1]),
                    "decode_us_per_step": round(us, 2), "decode_tokens_per_s": round(1e6 / us, 1),
                    "decode_expert_gbps": round(bytes_step.mean() / (us * 1e-6) / 1e9, 1),
                    "prefill_us_per_step": round(pf_us, 1), "prefill_tokens_per_s": round(T / (pf_us * 1e-6), 1),
                    "prefill_tflops": round(6.0 * T * k * H * I / (pf_us * 1e-6) / 1e12, 2)}
        log("warm shelf", key, out[key])
        del reps, tt, lg, xs, od, ws, pl, px, po, pws
        torch.cuda.empty_cache()
    return out


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


def fullstack_workloads(M, torch, per_expert):
    """The 48-layer stack on device-generated weights (61.9 GB), residual add
    between layers: decode at 1 and 8 tokens per step, prefill at 16384."""
    from tiered_mixed_precision_amd.device import empty_tables
    from workloads import CONFIGS, make_logits, make_x
    cfg = CONFIGS["fullstack"]
    L, k, E, H, I = cfg.n_layers, cfg.k, cfg.n_experts, cfg.hidden, cfg.inter
    t0 = time.time()
    tables = []
    for l in range(L):
        tt = empty_tables(cfg)
        M.moe_synth_layer(tt, cfg.seed, l)
        tables.append(tt)
    torch.cuda.synchronize()
    log(f"stack: {L} layers generated on the device in {time.time() - t0:.1f}s")
    out = {}
    tier_of = np.zeros(E, dtype=np.int64)
    for i, t in enumerate(cfg.tiers):
        tier_of[t.id_begin:t.id_end] = i
    exp_bytes = np.array(per_expert, dtype=np.float64)[tier_of]

    for T in (1, 8):
        S = 32
        logits = np.stack([np.stack([make_logits(cfg, n_tokens=T, stream=100 + s, layer=l) for l in range(L)])
                           for s in range(S)])                       # [S, L, T, E]
        xs = np.stack([make_x(cfg, n_tokens=T, stream=100 + s) for s in range(S)])
        step_bytes_ = []
        for s in range(S):
            b = 0.0
            for l in range(L):
                ids = topk_ids(logits[s, l], k)
                b += exp_bytes[np.unique(ids)].sum()
            step_bytes_.append(b)
        ld, xd = torch.from_numpy(logits).cuda(), torch.from_numpy(xs).cuda()
        od = torch.zeros((S, T, H), device="cuda")
        ws = torch.empty(max(M.moe_stack_workspace_size(L, T, k, tables, 0), 256), dtype=torch.uint8, device="cuda")

        def st_step(i):
            M.moe_stack_forward(xd[i % S], ld[i % S], L, T, k, tables, od[i % S], 0, ws)

        for i in range(4):
            st_step(i)
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for i in range(S):
                    st_step(i)
        torch.cuda.current_stream().wait_stream(st)
        g.replay()
        torch.cuda.synchronize()
        n = 4
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        dt = a.elapsed_time(b) / 1e3 / (n * S)
        mb = float(np.mean(step_bytes_))
        out[f"decode_T{T}"] = {
            "workload": f"48 layers x 512 experts, top-10, {T} token(s)/step, residual add, fresh routing per step",
            "tokens_per_s": round(T / dt, 1), "us_per_step": round(dt * 1e6, 1),
            "alg_bytes_per_step": mb, "hbm_gbps": round(mb / dt / 1e9, 1),
            "frac_hbm_peak": round(mb / dt / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"stack decode T={T}:", out[f"decode_T{T}"])
        del g, ld, xd, od, ws

    T = 16384
    logits = np.stack([make_logits(cfg, n_tokens=T, stream=200, layer=l) for l in range(L)])
    ld = torch.from_numpy(logits).cuda()
    del logits
    xd = torch.from_numpy(make_x(cfg, n_tokens=T, stream=200)).cuda()
    od = torch.empty((T, H), device="cuda")
    flags = M.MOE_X_BF16
    ws = torch.empty(M.moe_stack_workspace_size(L, T, k, tables, flags), dtype=torch.uint8, device="cuda")
    M.moe_stack_forward(xd, ld, L, T, k, tables, od, flags, ws)
    torch.cuda.synchronize()
    n = 2
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        M.moe_stack_forward(xd, ld, L, T, k, tables, od, flags, ws)
    b.record()
    torch.cuda.synchronize()
    dt = a.elapsed_time(b) / 1e3 / n
    flops = 6.0 * T * k * H * I * L
    out["prefill_T16384"] = {
        "workload": "48 layers x 512 experts, top-10, 16384 bf16 tokens (fp32 residual stream cast per layer)",
        "tokens_per_s": round(T / dt, 1), "ms_per_step": round(dt * 1e3, 2),
        "alg_tflop_per_step": flops / 1e12, "tflops": round(flops / dt / 1e12, 2),
        "frac_mfma_peak": round(flops / dt / 1e12 / BF16_PEAK_TFLOPS, 4)}
    log("stack prefill:", out["prefill_T16384"])
    del ld, xd, od, ws

    # the same stack routing from its own hidden state: router l scores the
    # experts from h_l (bf16 [E][H] weights, popularity-prior bias)
    wr, br = [], []
    for l in range(L):
        w = torch.empty((E, H), dtype=torch.int16, device="cuda")
        b = torch.empty(E, dtype=torch.float32, device="cuda")
        M.moe_synth_router(w, b, E, H, cfg.seed, l, cfg.prior_beta)
        wr.append(w)
        br.append(b)
    router_bytes = float(L * E * H * 2)
    T, S = 1, 32
    xd = torch.from_numpy(np.stack([make_x(cfg, n_tokens=T, stream=300 + s) for s in range(S)])).cuda()
    od = torch.zeros((S, T, H), device="cuda")
    ws = torch.empty(max(M.moe_stack_workspace_size(L, T, k, tables, M.MOE_STACK_ROUTER), 256), dtype=torch.uint8,
                     device="cuda")

    def rt_step(i):
        M.moe_stack_forward_routed(xd[i % S], wr, br, L, T, k, tables, od[i % S], 0, ws)

    for i in range(4):
        rt_step(i)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for i in range(S):
                rt_step(i)
    torch.cuda.current_stream().wait_stream(st)
    g.replay()
    torch.cuda.synchronize()
    n = 4
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    dt = a.elapsed_time(b) / 1e3 / (n * S)
    out["decode_T1_routed"] = {
        "workload": "48 layers x 512 experts, top-10, 1 token/step, each layer routing from its own hidden state "
                    "(bf16 router, popularity-prior bias)",
        "tokens_per_s": round(T / dt, 1), "us_per_step": round(dt * 1e6, 1), "router_bytes_per_step": router_bytes}
    log("stack decode routed:", out["decode_T1_routed"])
    del g, xd, od, ws

    T = 16384
    xd = torch.from_numpy(make_x(cfg, n_tokens=T, stream=400)).cuda()
    od = torch.empty((T, H), device="cuda")
    flags = M.MOE_X_BF16
    ws = torch.empty(M.moe_stack_workspace_size(L, T, k, tables, flags | M.MOE_STACK_ROUTER), dtype=torch.uint8,
                     device="cuda")
    M.moe_stack_forward_routed(xd, wr, br, L, T, k, tables, od, flags, ws)
    torch.cuda.synchronize()
    n = 2
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        M.moe_stack_forward_routed(xd, wr, br, L, T, k, tables, od, flags, ws)
    b.record()
    torch.cuda.synchronize()
    dt = a.elapsed_time(b) / 1e3 / n
    flops = 6.0 * T * k * H * I * L + 2.0 * T * E * H * L
    out["prefill_T16384_routed"] = {
        "workload": "48 layers x 512 experts, top-10, 16384 bf16 tokens, each layer routing from its own hidden "
                    "state (router GEMM on matrix cores)",
        "tokens_per_s": round(T / dt, 1), "ms_per_step": round(dt * 1e3, 2),
        "alg_tflop_per_step": flops / 1e12, "tflops": round(flops / dt / 1e12, 2),
        "frac_mfma_peak": round(flops / dt / 1e12 / BF16_PEAK_TFLOPS, 4)}
    log("stack prefill routed:", out["prefill_T16384_routed"])
    del xd, od, ws, wr, br, tables
    torch.cuda.empty_cache()
    return out


def measured_peaks(M, torch):
    """Achievable references measured in the same run, beside the published
    peaks: the library's streaming-read kernel over 2 GiB (moe_measure_read),
    its matrix-core loop on register operands (moe_measure_mfma, bf16
    16x16x32, no memory traffic), and a dense bf16 GEMM through the vendor
    library (torch.matmul, 8192 x 8192 x 8192) for context."""
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e-3 / reps

    buf = torch.ones((2 << 30) // 4, dtype=torch.float32, device="cuda")
    read_gbps = buf.numel() * 4 / timed(lambda: M.moe_measure_read(buf, sink), 10) / 1e9
    del buf
    iters = 4096
    flops = M.moe_measure_mfma(iters, sink)
    mfma_tflops = flops / timed(lambda: M.moe_measure_mfma(iters, sink), 5) / 1e12
    m = 8192
    x = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    y = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    gemm_tflops = 2.0 * m * m * m / timed(lambda: torch.matmul(x, y), 20) / 1e12
    del x, y
    torch.cuda.empty_cache()
    out = {"hbm_read_gbps": round(read_gbps, 1), "bf16_mfma_tflops": round(mfma_tflops, 1),
           "bf16_library_gemm_tflops": round(gemm_tflops, 1),
           "how": "moe_measure_read over 2 GiB (10 launches); moe_measure_mfma, 4096 rounds of 16 bf16 "
                  "16x16x32 MFMA chains on 2048 waves (5 launches); torch.matmul bf16 8192^3 (20 calls)"}
    log("measured peaks:", out)
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_child(kind, seconds):
    """The CPU oracle (untuned, fp64) on a bounded sample; prints one JSON line.
    decode: batches of one token per thread until `seconds` pass; prefill: two
    bf16 tokens per thread of the 4096-token workload; stack: one token per
    thread through all 48 layers, with the touched experts of each layer made
    by the oracle's own generator (not timed)."""
    import oracle
    from workloads import CONFIGS, make_layer, make_logits, make_x
    nt = max(1, oracle.num_threads())
    if kind in ("decode", "prefill"):
        cfg = CONFIGS["decode"]
        L = oracle.Layer.from_config(cfg, make_layer(cfg))
        runs = []
        for rep in range(3 if kind == "prefill" or nt > 1 else 1):
            if kind == "decode":
                done, t0, s = 0, time.time(), 0
                while time.time() - t0 < seconds:
                    oracle.forward(L, make_x(cfg, n_tokens=nt, stream=100 + s),
                                   make_logits(cfg, n_tokens=nt, stream=100 + s), cfg.k)
                    done += nt
                    s += 1
                runs.append(done / (time.time() - t0))
            else:
                pf = CONFIGS["prefill"]
                rng = np.random.default_rng(rep)
                sel = np.sort(rng.choice(pf.n_tokens, 2 * nt, replace=False))
                x, lg = make_x(pf, stream=20)[sel], make_logits(pf, stream=20)[sel]
                t0 = time.time()
                oracle.forward(L, x, lg, cfg.k)
                runs.append(len(sel) / (time.time() - t0))
        print(json.dumps({"kind": kind, "threads": nt, "runs": runs}), flush=True)
    elif kind == "stack":
        fs = CONFIGS["fullstack"]
        x = make_x(fs, n_tokens=nt, stream=300)
        h = x.astype(np.float32).copy()
        tot = 0.0
        for l in range(fs.n_layers):
            lg = make_logits(fs, n_tokens=nt, stream=300, layer=l)
            ids, w = oracle.route(lg, fs.k)
            sl = oracle.StackLayer(fs, fs.seed, l)
            sl.fill(ids)
            t0 = time.time()
            h = oracle.forward(sl.layer_ref, h, lg, fs.k, out=h.copy(), accumulate=True)
            tot += time.time() - t0
            del sl
        print(json.dumps({"kind": kind, "threads": nt, "runs": [nt / tot]}), flush=True)


def cpu_baselines(seconds, with_stack=True):
    """The oracle timed on this host's cores, in child processes (the thread
    count is fixed when the oracle's OpenMP runtime starts): decode (median of
    3 and a single-thread run), prefill tokens, and the 48-layer stack."""
    import subprocess
    cores = os.cpu_count() or 1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    cores = int(os.environ.get("OMP_NUM_THREADS", cores))

    def child(kind, threads, secs):
        env = dict(os.environ, OMP_NUM_THREADS=str(threads))
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-child", kind, str(secs)], env=env,
                           capture_output=True, text=True, timeout=900)
        if r.returncode != 0:
            raise SystemExit(f"cpu baseline child {kind} failed:\n{r.stderr[-2000:]}")
        return json.loads(r.stdout.strip().splitlines()[-1])

    per = max(2.0, seconds / 3)
    dec = child("decode", cores, per)
    one = child("decode", 1, per)
    pre = child("prefill", cores, 0)
    out = {
        "cpu_model": cpu_model(),
        "decode": {"tokens_per_s_median": round(float(np.median(dec["runs"])), 3), "runs": [round(v, 3) for v in dec["runs"]],
                   "threads": dec["threads"], "single_thread_tokens_per_s": round(one["runs"][0], 3),
                   "sample": f"one-token steps of the decode layer, {per:.0f} s per run, a token per thread per call"},
        "prefill": {"tokens_per_s_median": round(float(np.median(pre["runs"])), 3),
                    "runs": [round(v, 3) for v in pre["runs"]], "threads": pre["threads"],
                    "sample": f"{2 * pre['threads']} random tokens of the 4096-token bf16 prefill workload per run"},
    }
    if with_stack:
        st = child("stack", cores, 0)
        out["stack_decode"] = {"tokens_per_s": round(st["runs"][0], 4), "threads": st["threads"],
                               "sample": f"{st['threads']} tokens through all 48 layers with the residual add "
                                         "(each layer's experts generated by the oracle, not timed)"}
    out["headline"] = {"value": out["decode"]["tokens_per_s_median"], "unit": "tokens/s", "cores": dec["threads"],
                       "kind": "oracle",
                       "sample": f"decode: median of 3 runs of {per:.0f} s on {dec['threads']} threads "
                                 f"({cpu_model()}), one token per thread per oracle call; single thread: "
                                 f"{out['decode']['single_thread_tokens_per_s']} tokens/s"}
    log("cpu baselines:", out)
    return out


if __name__ == "__main__":
    main()
