#!/usr/bin/env python3
"""Benchmark of the SSD chunked-scan forward (and backward) on one MI355X.

One step = one full ``ssd_fwd`` (all stages) over the "layer" workload:
batch 2 x 2048 tokens, 24 heads x headdim 64, d_state 128, bf16 inputs
(the shape of the Mamba3 example on the page "长序列 Mamba 多卡训练，算力和
显存怎么同时省", §三).  Inputs are resident in HBM before timing starts.
Prints one JSON line:

* value / ms_per_step   -- W warm-up steps, then exactly K timed steps
  between two stream synchronizations (wall clock; caches warm).
* cold                  -- the same step with 512 MiB of scratch written
  before each one (more than L2 and the 256 MiB MALL together), timed with
  HIP events on the launch stream; median over the steps.
* roofline              -- the dominant kernel's algorithmic bytes per launch
  divided by its average duration (HIP events around K back-to-back
  launches of that stage alone on the launch stream); peak 8 TB/s HBM.
  ``traffic`` is the per-launch HBM bytes from the committed rocprofv3
  FETCH_SIZE / WRITE_SIZE summary, or null if the kernel sources changed
  since the counters were taken.
* stages                -- per stage: average µs (the same isolated timing),
  algorithmic flops and bytes, arithmetic intensity, and the fraction of the
  bf16 MFMA peak (2.5 PFLOP/s; fp32 157.3 TFLOP/s) and of HBM (8 TB/s).
* cpu_baseline          -- the C fp64 oracle (test infrastructure) timed on
  this host on the same workload, repeated for ~10 s.
* bwd                   -- outside the timed region: the backward pass
  (``ssd_bwd``, gradients of every input for a seeded dL/dy and dL/d
  final_state) on the same workload; null where it is not built.
* workloads             -- the other workloads of the pages' shapes (tiny,
  wide, packed varlen, 1M-token bidirectional), each timed the same way in
  this run: forward and backward ms per step, Mtokens/s, and the dominant
  forward kernel's HBM fraction.
* context               -- the pages' only throughput figure (about 950
  tokens/s whole-model training at 8K on one unstated A100-class GPU); not
  a kernel result and not comparable, so vs_baseline stays null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD chunked-scan fwd Mtokens/s at 1 GPU; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
# sources the span kernels are compiled from (their traffic counters go
# stale when either changes)
KERNEL_SRCS = [os.path.join(ROOT, "mamba_ssd_chunked_02_amd", "csrc", f)
               for f in ("ssd_kernels.hip", "ssd_device.h")]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic_layer.json")
STAGE_KERNEL = {"state": "span_kernel<{T}, {N}, 1, kModeState>", "pass": "state_pass_kernel<{T}>",
                "scan": "span_kernel<{T}, {N}, 1, kModeScan>",
                "fused": "span_kernel<{T}, {N}, 1, kModeFused>", "table": "span_table_kernel"}
DTYPE_LABEL = {"bf16": "bf16 in, bf16 span states, fp32 accumulation and final state",
               "f32": "fp32 in, fp32 span states and accumulation"}
CONTEXT = {"pages_tokens_per_s": 950,
           "what": "whole-model Mamba training at sequence 8K on one GPU, unstated "
                   "A100-class hardware (page 长序列 Mamba 多卡训练，算力和显存怎么同时省, §四)",
           "comparable": False}


def kernel_label(stage: str, plan, w) -> str:
    """Name of the kernel that runs a stage under this plan."""
    if plan.head_wave and stage in ("state", "scan"):
        mode = 1 if stage == "scan" else 0
        heads = plan.heads_per_wg if stage == "scan" else plan.heads_per_state_wg
        return (f"hw_span_kernel<{w.d_state}, {heads}, "
                f"{plan.cols_per_wave // 16}, {mode}>")
    return STAGE_KERNEL[stage].format(T="bf16" if w.dtype == "bf16" else "float", N=w.d_state)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stage_bytes(w, plan, spans_used: int) -> dict:
    """Algorithmic HBM bytes per launch of each stage: every operand read
    once and every result written once at the stage boundaries.

    Per token-head unit (T*H units): x (P*e), d_raw (e), B and C (N*e each,
    shared by the H/G heads of a group), y (P*e).  Per span-head: one N x P
    state stored in the input type (plus a 4-byte fp32 decay); init and
    final states are fp32.  e = element size of the inputs.
    fused_pass 1: the state launch forms only the first sps - 1 spans of
    each sequence (no scan reads the last one's state) and is charged their
    tokens' inputs and their states; span_scan is charged those span states
    and decays once, plus init and final states, and there is no pass.
    fused_pass 2: the one
    launch is charged its inputs and outputs plus each span state it hands
    on (all but the last span of a sequence) written once; the reads of
    those states by later spans are not counted."""
    e = 2 if w.dtype == "bf16" else 4
    T, H, P, N, G = w.tokens, w.nheads, w.headdim, w.d_state, w.ngroups
    S = w.nstates
    x = T * H * P * e
    draw = T * H * e
    bc = T * G * N * e
    y = T * H * P * e
    st = spans_used * H * N * P * e
    dec = spans_used * H * 4
    fin = S * H * N * P * 4
    init = fin if w.init != "zeros" else 0
    if plan.fused_pass == 2:
        handed = (spans_used - S) * H
        return {"fused": x + draw + 2 * bc + y + init + fin + handed * (N * P * e + 4)}
    if plan.fused_pass == 1:
        formed = spans_used - S                    # batch mode: all but each last span
        frac = formed * 64 * plan.chunks_per_span / T if T else 0.0
        stf, decf = formed * H * N * P * e, formed * H * 4
        return {"state": round((x + draw + bc) * frac) + stf + decf,
                "scan": x + draw + 2 * bc + stf + decf + init + fin + y}
    return {
        "state": x + draw + bc + st + dec,
        "pass": 2 * st + dec + fin + init,
        "scan": x + draw + 2 * bc + st + y,
    }


def stage_flops(w, plan, spans_used: int) -> dict:
    """Algorithmic flops per launch of each stage (multiply-adds count 2):
    the work the chunked method must do, not what a kernel recomputes.

    Per token-head: the chunk-state contraction B^T (w X), 2NP; the
    inter-chunk term C Hprev, 2NP; the causal intra-chunk product, (Q+1)P on
    average over a chunk's 64 positions.  Per token and B/C group: the
    causal C B^T, (Q+1)N.  Per span-head: the pair combine, 2NP.  Recomputing
    a state inside span_scan is not counted.  fused_pass 1: the state launch
    forms the first sps - 1 spans of each sequence (their tokens' chunk
    states and one combine per span); the scan carries the last span's
    chunk states on to the final state."""
    T, H, P, N, G, Q = w.tokens, w.nheads, w.headdim, w.d_state, w.ngroups, 64
    state = 2 * N * P * T * H
    scan = (2 * N * P + (Q + 1) * P) * T * H + (Q + 1) * N * T * G
    combine = 2 * N * P * spans_used * H
    if plan.fused_pass == 2:
        return {"fused": state + scan + combine}
    if plan.fused_pass == 1:
        formed = spans_used - w.nstates
        fstate = 2 * N * P * formed * 64 * plan.chunks_per_span * H
        return {"state": fstate, "scan": scan + (state - fstate) + 2 * N * P * formed * H}
    return {"state": state, "pass": combine, "scan": scan}


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def spans_used(w, plan, cu=None) -> int:
    """Spans the launch actually processes (one per K chunks per sequence)."""
    K = plan.chunks_per_span
    if w.nseq:
        import numpy as np
        lens = np.diff(cu.cpu().numpy().astype(np.int64))
        return int(sum(ceil_div(ceil_div(int(n), 64), K) for n in lens))
    return w.batch * ceil_div(ceil_div(w.seqlen, 64), K)


def read_traffic(kernel_hash: str, stage: str):
    try:
        with open(PMC_SUMMARY) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_hash:
        return None
    return d.get("stages", {}).get(stage, {}).get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, inputs, budget_s: float = 10.0) -> dict:
    from oracle import cref
    reps = 0
    t0 = time.perf_counter()
    while True:
        cref.ssd_ref_seq_c(inputs["x"], inputs["d_raw"], inputs["d_init"], inputs["B"],
                           inputs["C"], inputs["init_state"], inputs["cu_seqlens"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    return {"value": round(w.tokens * reps / el / 1e6, 4), "unit": "Mtokens/s",
            "cores": cref.threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"whole {w.name} workload ({w.batch}x{w.seqlen} tokens, {w.nheads} heads), "
                      f"fp64 sequential recurrence, {reps} repetitions in {el:.1f} s"}


def load_workload(w, dev):
    """(host inputs or None, device inputs)."""
    import torch
    from ssd_inputs import make_inputs, make_inputs_device
    host = make_inputs(w) if w.tokens <= (1 << 18) else None
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in host.items()} \
        if host is not None else make_inputs_device(w, dev)
    torch.cuda.synchronize()
    return host, d


def forward_calls(m, w, d, dev):
    """The prepared ssd_fwd calls of one step (two for the bidirectional
    workload, writing the halves of one [b, L, H, 2P] output) and that
    output."""
    import torch
    calls = [m.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                       init_state=d["init_state"], cu_seqlens=d["cu_seqlens"])]
    ycat = None
    if w.bidir:
        b, L, H, P = d["x"].shape
        ycat = torch.empty((b, L, H, 2 * P), dtype=d["x"].dtype, device=dev)
        ws = calls[0].workspace
        calls = [m.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], reverse=bool(rev),
                           y=ycat[..., P * rev:P * (rev + 1)], workspace=ws)
                 for rev in (0, 1)]
    return calls, ycat


def step_calls(m, w, d, calls, ycat):
    """What one timed forward step launches: the prepared calls, or for the
    bidirectional workload one ssd_fwd_bidir call into the same [b, L, H, 2P]
    output (both directions' span states from one pass where the spans
    allow).  ``calls`` stay the per-direction calls that single stages are
    timed with."""
    if not w.bidir:
        return calls
    return [m.prepare_bidir(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], y=ycat)]


def backward_calls(m, w, d, dev, calls, ycat):
    """The prepared ssd_bwd calls of one step, for a seeded dL/dy (and dL/d
    final_state); [] where the backward is not built for these sizes."""
    import torch
    if m.ssd_bwd_workspace_bytes(calls[0].dims) == 0:
        return []
    g = torch.Generator(device=dev).manual_seed(7)
    out = []
    for c in calls:
        c.run()
    if w.bidir:
        dycat = torch.randn(ycat.shape, generator=g, device=dev).to(ycat.dtype)
        P = d["x"].shape[3]
        ws = None
        for rev in (0, 1):
            bc = m.prepare_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                               ycat[..., P * rev:P * (rev + 1)], dycat[..., P * rev:P * (rev + 1)],
                               reverse=bool(rev), workspace=ws)
            ws = bc.workspace
            out.append(bc)
    else:
        y, fin = calls[0].y, calls[0].final_state
        dy = torch.randn(y.shape, generator=g, device=dev).to(y.dtype)
        dfin = torch.randn(fin.shape, generator=g, device=dev)
        out.append(m.prepare_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], y, dy,
                                 init_state=d["init_state"], cu_seqlens=d["cu_seqlens"],
                                 d_final=dfin))
    return out


def warm_for(fn, seconds: float) -> None:
    """Call fn until `seconds` of wall time have passed."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()


def wall_ms(fn, steps: int, warmup: int) -> float:
    """Wall-clock ms per call of fn: warmup calls, then steps calls between
    two synchronizations."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def stage_times_us(m, calls, stages, reps: int) -> dict:
    """Average µs of each stage, launched alone reps times between one HIP
    event pair on the launch stream (no event between launches)."""
    import torch
    stream = torch.cuda.current_stream()
    out = {}
    for name, mask in stages:
        for c in calls:
            c.run(mask)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            for c in calls:
                c.run(mask)
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) / (reps * len(calls)) * 1e3
    return out


def plan_stages(m, w, plan):
    stages = [("state", m.STAGE_STATE), ("pass", m.STAGE_PASS), ("scan", m.STAGE_SCAN)]
    if plan.fused_pass == 1:
        stages = [st for st in stages if st[0] != "pass"]
    if plan.fused_pass == 2:
        stages = [("fused", m.STAGE_SCAN)]
    return stages


def stage_report(w, plan, us: dict, fl: dict, by: dict) -> dict:
    peak = MFMA_PEAK_TFLOPS["bf16" if w.dtype == "bf16" else "f32"]
    rep = {}
    for k, t in us.items():
        if k not in by:
            continue
        s = t * 1e-6
        rep[k] = {"us": round(t, 3), "flops": fl[k], "bytes": by[k],
                  "ai_flop_per_byte": round(fl[k] / by[k], 2),
                  "mfma_frac": round(fl[k] / s / (peak * 1e12), 4),
                  "hbm_frac": round(by[k] / s / (HBM_PEAK_GBS * 1e9), 4)}
    return rep


def workload_line(m, name: str, dev, with_bwd: bool) -> dict:
    """Forward (and backward) timing of one more workload in this run."""
    import torch
    from ssd_inputs import by_name
    w = by_name(name)
    _, d = load_workload(w, dev)
    calls, ycat = forward_calls(m, w, d, dev)
    scalls = step_calls(m, w, d, calls, ycat)
    plan = m.ssd_fwd_plan(calls[0].dims)
    big = w.tokens >= (1 << 20)
    # enough warm-up and steps that first-call costs do not show (a step of
    # the largest workload takes ~5 ms); the warm-up also lasts at least
    # 0.2 s, so a GPU that sat idle (the CPU baseline runs before these
    # lines) is back at its working clock
    steps, warm = (20, 5) if big else (200, 20)
    warm_for(lambda: [c.run() for c in scalls], 0.2)
    fwd = wall_ms(lambda: [c.run() for c in scalls], steps, warm)
    stages = plan_stages(m, w, plan)
    us = stage_times_us(m, calls, stages, 5 if big else 50)
    used = spans_used(w, plan, d["cu_seqlens"])
    by = stage_bytes(w, plan, used)
    dom = max((n for n in us if n in by), key=lambda n: us[n])
    line = {"workload": f"{w.name}: {w.batch}x{w.seqlen} tokens, {w.nheads} heads x headdim "
                        f"{w.headdim}, d_state {w.d_state}, {w.dtype}"
                        + (f", {w.nseq} packed sequences" if w.nseq else "")
                        + (", fwd+rev" if w.bidir else ""),
            "fwd_ms_per_step": round(fwd, 5), "fwd_us_per_step": round(fwd * 1e3, 2),
            "fwd_mtokens_per_s": round(w.tokens / (fwd * 1e-3) / 1e6, 3),
            "kernel_family": "head-wave" if plan.head_wave else "span",
            "chunks_per_span": plan.chunks_per_span,
            "dominant": {"stage": dom, "kernel": kernel_label(dom, plan, w),
                         "us": round(us[dom], 3), "algorithmic_bytes": by[dom],
                         "hbm_frac": round(by[dom] / (us[dom] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)},
            "bwd_ms_per_step": None}
    if with_bwd:
        bcalls = backward_calls(m, w, d, dev, calls, ycat)
        if bcalls:
            bsteps, bwarm = (5, 2) if big else (50, 5)
            bwd = wall_ms(lambda: [bc.run() for bc in bcalls], bsteps, bwarm)
            line["bwd_ms_per_step"] = round(bwd, 5)
            line["bwd_mtokens_per_s"] = round(w.tokens / (bwd * 1e-3) / 1e6, 3)
        del bcalls
    del calls, scalls, ycat, d
    torch.cuda.empty_cache()
    return line


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the backward legs (profiles of the forward kernels alone)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads' lines")
    ap.add_argument("--cold-mib", type=int, default=512,
                    help="MiB of scratch written before each cold step (0: no cold timing)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before warm-up, run 3 plain device copies of this many MiB "
                         "(reference kernel for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the SSD scan here is built and timed on a "
              "single MI355X; run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import mamba_ssd_chunked_02_amd as m
    from ssd_inputs import by_name

    w = by_name(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    host, d = load_workload(w, dev)
    calls, ycat = forward_calls(m, w, d, dev)
    scalls = step_calls(m, w, d, calls, ycat)
    plan = m.ssd_fwd_plan(calls[0].dims)
    stream = torch.cuda.current_stream(dev)
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        for c in scalls:
            c.run()

    # timed region: exactly K steps, caches warm
    K = args.steps
    ms_per_step = wall_ms(step, K, args.warmup)

    # per-stage isolated timing, algorithmic work and the roofline
    stages = plan_stages(m, w, plan)
    us = stage_times_us(m, calls, stages, K)
    used = spans_used(w, plan, d["cu_seqlens"])
    sb = stage_bytes(w, plan, used)
    sf = stage_flops(w, plan, used)
    dom = max((n for n in us if n in sb), key=lambda n: us[n])
    achieved = sb[dom] / (us[dom] * 1e-6) / 1e9
    khash = kernel_source_hash()
    traffic = read_traffic(khash, dom)

    # cold steps: every cache overwritten before each one
    cold = None
    if args.cold_mib > 0:
        scratch = torch.empty(args.cold_mib << 20, dtype=torch.uint8, device=dev)
        times = []
        for i in range(min(K, 50)):
            scratch.fill_(i & 0xFF)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        cms = statistics.median(times)
        cold = {"ms_per_step": round(cms, 5), "value": round(w.tokens / (cms * 1e-3) / 1e6, 3),
                "unit": "Mtokens/s", "steps": len(times),
                "flush": f"{args.cold_mib} MiB written before each step (L2 and the 256 MiB "
                         f"MALL hold none of the inputs), HIP events around the step"}
        del scratch

    value = w.tokens / (ms_per_step * 1e-3) / 1e6
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Mtokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.batch}x{w.seqlen} tokens, {w.nheads} heads x "
                               f"headdim {w.headdim}, d_state {w.d_state}, chunk 64, "
                               + DTYPE_LABEL[w.dtype] + (", fwd+rev" if w.bidir else ""),
                   "global_batch": w.batch, "seq_len": w.seqlen, "parallelism": "single-gpu",
                   "chunks_per_span": plan.chunks_per_span,
                   "kernel_family": "head-wave" if plan.head_wave else "span",
                   "state_pass": ["separate launch", "folded into the scan",
                                  "one fused launch"][plan.fused_pass]},
        "roofline": {"bound": "hbm", "kernel": kernel_label(dom, plan, w),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": sb[dom],
                     "avg_us": round(us[dom], 3)},
        "stages": stage_report(w, plan, us, sf, sb),
        "cold": cold,
        "cpu_baseline": None,
        "bwd": None,
        "workloads": None,
        "context": CONTEXT,
    }
    if not args.no_bwd:
        bcalls = backward_calls(m, w, d, dev, calls, ycat)
        if bcalls:
            bwd_ms = wall_ms(lambda: [bc.run() for bc in bcalls], K, args.warmup)
            out["bwd"] = {"ms_per_step": round(bwd_ms, 5),
                          "value": round(w.tokens / (bwd_ms * 1e-3) / 1e6, 3), "unit": "Mtokens/s",
                          "steps": K, "warmup": args.warmup}
        del bcalls
    if not args.no_cpu_baseline and host is not None:
        out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_budget)
    if not args.no_workloads:
        del calls, ycat, d
        torch.cuda.empty_cache()
        out["workloads"] = {n: workload_line(m, n, dev, not args.no_bwd)
                            for n in ("tiny", "wide", "varlen", "bidir") if n != w.name}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
