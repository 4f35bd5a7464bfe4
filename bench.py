#!/usr/bin/env python3
"""Benchmark of the SSD chunked-scan forward (and backward) on one MI355X.

One step = one full ``ssd_fwd`` (all stages) over the "layer" workload:
batch 2 x 2048 tokens, 24 heads x headdim 64, d_state 128, bf16 inputs,
fp32 state (the shape of the Mamba3 example on the page
"长序列 Mamba 多卡训练，算力和显存怎么同时省", §三).  Inputs are resident in
HBM before timing starts.  Prints one JSON line:

* value / ms_per_step   -- W warm-up steps, then exactly K timed steps
  between two stream synchronizations (wall clock).
* roofline              -- the dominant kernel's algorithmic bytes per launch
  divided by its average duration; peak 8 TB/s HBM.  The dominant kernel is
  the slowest stage in K further steps with HIP events recorded around each
  stage on the launch stream; its average duration is then taken from one
  event pair around K back-to-back launches of that stage alone (no event
  overhead per launch).
  ``traffic`` is the per-launch HBM bytes from the committed rocprofv3
  FETCH_SIZE / WRITE_SIZE summary, or null if the kernel source changed
  since the counters were taken.
* cpu_baseline          -- the C fp64 oracle (test infrastructure) timed on
  this host on the same workload, repeated for ~10 s.
* bwd                   -- outside the timed region: the backward pass
  (``ssd_bwd``, gradients of every input for a seeded dL/dy and dL/d
  final_state; one call per direction for the bidirectional workload) on
  the same workload, W warm-up steps then K steps between two stream
  synchronizations; null where the backward is not built for the sizes.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD chunked-scan fwd Mtokens/s at 1 GPU; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
# sources the span kernels are compiled from (their traffic counters go
# stale when either changes)
KERNEL_SRCS = [os.path.join(ROOT, "mamba_ssd_chunked_02_amd", "csrc", f)
               for f in ("ssd_kernels.hip", "ssd_device.h")]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic_layer.json")
STAGE_KERNEL = {"state": "span_kernel<bf16, N, 1, kModeState>", "pass": "state_pass_kernel",
                "scan": "span_kernel<bf16, N, 1, kModeScan>",
                "fused": "span_kernel<bf16, N, 1, kModeFused>", "table": "span_table_kernel"}


def kernel_label(stage: str, plan, w) -> str:
    """Name of the kernel that runs a stage under this plan."""
    if plan.head_wave and stage in ("state", "scan"):
        mode = 1 if stage == "scan" else 0
        # the state kernel groups at most two heads
        heads = plan.heads_per_wg if stage == "scan" else min(plan.heads_per_wg, 2)
        return (f"hw_span_kernel<{w.d_state}, {heads}, "
                f"{plan.cols_per_wave // 16}, {mode}>")
    return STAGE_KERNEL[stage]


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
    fused_pass 1: span_scan is charged each span state and decay once, plus
    init and final states, and there is no pass.  fused_pass 2: the one
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
        return {"state": x + draw + bc + st + dec,
                "scan": x + draw + 2 * bc + st + dec + init + fin + y}
    return {
        "state": x + draw + bc + st + dec,
        "pass": 2 * st + dec + fin + init,
        "scan": x + draw + 2 * bc + st + y,
    }


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
            "cores": cref.threads(), "kind": "oracle",
            "sample": f"whole {w.name} workload ({w.batch}x{w.seqlen} tokens, {w.nheads} heads), "
                      f"fp64 sequential recurrence, {reps} repetitions in {el:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the backward leg (profiles of the forward kernels alone)")
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
    from ssd_inputs import by_name, make_inputs, make_inputs_device

    w = by_name(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    host = make_inputs(w) if w.tokens <= (1 << 18) else None
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in host.items()} \
        if host is not None else make_inputs_device(w, dev)
    torch.cuda.synchronize()

    calls = [m.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                       init_state=d["init_state"], cu_seqlens=d["cu_seqlens"])]
    if w.bidir:
        b, L, H, P = d["x"].shape
        ycat = torch.empty((b, L, H, 2 * P), dtype=d["x"].dtype, device=dev)
        ws = calls[0].workspace
        calls = [m.prepare(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], reverse=rev,
                           y=ycat[..., P * rev:P * (rev + 1)], workspace=ws)
                 for rev in (0, 1)]
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
        for c in calls:
            c.run()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / K * 1e3

    # per-kernel durations: HIP events around every stage on the launch stream
    stages = [("state", m.STAGE_STATE), ("pass", m.STAGE_PASS), ("scan", m.STAGE_SCAN)]
    if plan.fused_pass == 1:
        stages = [st for st in stages if st[0] != "pass"]
    if plan.fused_pass == 2:
        stages = [("fused", m.STAGE_SCAN)]
    if w.nseq:
        stages = [("table", m.STAGE_TABLE)] + stages
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(K * len(calls))]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        for j, c in enumerate(calls):
            e = ev[i * len(calls) + j]
            e[0].record(stream)
            for s, (_, mask) in enumerate(stages):
                c.run(mask)
                e[s + 1].record(stream)
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    avg_ms = {name: sum(e[s].elapsed_time(e[s + 1]) for e in ev) / len(ev)
              for s, (name, _) in enumerate(stages)}

    used = spans_used(w, plan, d["cu_seqlens"])
    sb = stage_bytes(w, plan, used)
    dom = max((n for n in avg_ms if n in sb), key=lambda n: avg_ms[n])
    dom_mask = dict(stages)[dom]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(K):
        for c in calls:
            c.run(dom_mask)
    e1.record(stream)
    torch.cuda.synchronize()
    dom_ms = e0.elapsed_time(e1) / (K * len(calls))
    achieved = sb[dom] / (dom_ms * 1e-3) / 1e9
    khash = kernel_source_hash()
    traffic = read_traffic(khash, dom)

    tokens = w.tokens
    value = tokens / (ms_per_step * 1e-3) / 1e6
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
                               f"{w.dtype} in / fp32 state" + (", fwd+rev" if w.bidir else ""),
                   "global_batch": w.batch, "seq_len": w.seqlen, "parallelism": "single-gpu",
                   "chunks_per_span": plan.chunks_per_span},
        "roofline": {"bound": "hbm", "kernel": kernel_label(dom, plan, w),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": sb[dom],
                     "avg_us": round(dom_ms * 1e3, 3)},
        "stages_us": {k: round(v * 1e3, 3) for k, v in avg_ms.items()},
        "stage_algorithmic_bytes": sb,
        "ms_per_step_with_stage_events": round(wall_ev / K * 1e3, 5),
        "cpu_baseline": None,
    }
    out["bwd"] = None
    if not args.no_bwd and m.ssd_bwd_workspace_bytes(calls[0].dims) > 0:
        g = torch.Generator(device=dev).manual_seed(7)
        bcalls = []
        if w.bidir:
            # one backward per direction, y and dy as halves of [b, L, H, 2P]
            step()
            dycat = torch.randn(ycat.shape, generator=g, device=dev).to(ycat.dtype)
            P = d["x"].shape[3]
            bws = None
            for rev in (0, 1):
                bc = m.prepare_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"],
                                   ycat[..., P * rev:P * (rev + 1)],
                                   dycat[..., P * rev:P * (rev + 1)], reverse=bool(rev),
                                   workspace=bws)
                bws = bc.workspace
                bcalls.append(bc)
        else:
            y, fin = calls[0].run()
            dy = torch.randn(y.shape, generator=g, device=dev).to(y.dtype)
            dfin = torch.randn(fin.shape, generator=g, device=dev)
            bcalls.append(m.prepare_bwd(d["x"], d["d_raw"], d["d_init"], d["B"], d["C"], y, dy,
                                        init_state=d["init_state"], cu_seqlens=d["cu_seqlens"],
                                        d_final=dfin))
        for _ in range(args.warmup):
            for bc in bcalls:
                bc.run()
        torch.cuda.synchronize()
        tb = time.perf_counter()
        for _ in range(K):
            for bc in bcalls:
                bc.run()
        torch.cuda.synchronize()
        bwd_ms = (time.perf_counter() - tb) / K * 1e3
        out["bwd"] = {"ms_per_step": round(bwd_ms, 5),
                      "value": round(tokens / (bwd_ms * 1e-3) / 1e6, 3), "unit": "Mtokens/s",
                      "steps": K, "warmup": args.warmup}
    if not args.no_cpu_baseline and host is not None:
        out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
