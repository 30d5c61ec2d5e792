"""Benchmark: ragged top-7 token log-probabilities on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole device path over one synthetic batch of the
workload: the row kernel (and, for split-vocab plans, the merge kernel)
reading every selected logits row once.  The logits and the row descriptors
are resident in HBM when the timed region starts (the descriptors are
uploaded once beforehand); a second, separately reported loop also runs the
host plan and the PCIe descriptor upload every step.

Small workloads fit in the 256 MB Infinity Cache, so the timed loop cycles
through copies of the logits totalling at least 1 GiB.

Prints one JSON line (rank 0, N = 1).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "logit rows/s and achieved HBM GB/s (% of peak), ragged top-7 logprobs, 1 GPU"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 1 << 30
DEFAULT_STEPS = {"no_echo_next_token": 200, "ragged_echo_mix": 200, "decode_peaked": 200,
                 "prefill_echo_large": 20, "tie_edge_stress": 30}


def algorithmic_bytes(plan_info, vocab):
    """Bytes a perfect implementation moves per launch: each read row once
    (4 V), 64 B of output and a 16 B descriptor per output row."""
    return int(plan_info["read_rows"]) * 4 * vocab + int(plan_info["out_rows"]) * (64 + 16)


def cpu_baseline(case, logits_dev, ntl_dev, budget_s=15.0):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import oracle.logprob_oracle as LO

    tasks = LO.row_tasks(case.offsets, case.echo, case.top_n, case.tokens, case.sampled,
                         case.has_logits)
    live = [o for o, t in enumerate(tasks) if t.top_n > 0]
    # rows of the same workload, in output order, until the budget is spent
    src = logits_dev if case.has_logits else ntl_dev
    cache = {}
    done, t_total = 0, 0.0
    for o in live:
        t = tasks[o]
        if t.src_row not in cache:
            cache.clear()
            cache[t.src_row] = src[t.src_row].cpu().numpy()
        row = cache[t.src_row]
        t0 = time.perf_counter()
        LO.compute_row(row, t.chosen, t.top_n, 8)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    return {"value": done / t_total, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {len(live)} read rows of {case.name} "
                      f"(float64 log-softmax + stable sort per row, one thread), "
                      f"{t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ragged_echo_mix")
    ap.add_argument("--split", type=int, default=None, help="force the plan's split")
    ap.add_argument("--waves", type=int, default=None, help="force waves per workgroup (4|8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-e2e", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import gen
    import ragged_token_log_amd as R

    R.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = gen.WORKLOADS[args.workload]()
    steps = args.steps or DEFAULT_STEPS.get(args.workload, 50)
    stream = torch.cuda.current_stream(dev)

    base = gen.device_logits(case, dev, torch)
    last = torch.from_numpy(case.offsets[1:].astype(np.int64) - 1).to(dev)
    ntl = base.index_select(0, last) if case.has_logits else base
    copy_bytes = base.numel() * 4
    n_copies = max(1, math.ceil(ROTATE_BYTES / copy_bytes))
    copies = [base] + [base.clone() for _ in range(n_copies - 1)]
    torch.cuda.synchronize()

    plan = R.Plan(case.offsets, case.echo, case.top_n, case.vocab, case.has_logits)
    if args.split:
        plan.set_split(args.split)
    if args.waves:
        plan.set_waves(args.waves)
    info = plan.info()
    lp, ids, ws = R.alloc_outputs(plan, dev, torch)
    plan.stage(case.tokens, case.sampled, ws, stream)   # descriptors resident in HBM

    def step(i):
        src = copies[i % n_copies]
        if case.has_logits:
            plan.launch(src, None, lp, ids, ws, stream)
        else:
            plan.launch(None, src, lp, ids, ws, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = total_ms / steps
    avg_launch_ms = float(np.mean(launch_ms))

    read_rows = int(info["read_rows"])
    rows_per_s = read_rows / (ms_per_step * 1e-3)
    alg_bytes = algorithmic_bytes(info, case.vocab)
    achieved_gbs = alg_bytes / (avg_launch_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded draws with the workload's shapes and distributions)",
        "config": {"workload": case.name, "batch": case.batch, "vocab": case.vocab,
                   "out_rows": int(info["out_rows"]), "read_rows": read_rows,
                   "split": int(info["split"]), "waves": int(info["waves"]),
                   "logits_copies_cycled": n_copies},
        "hbm_gbs": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "row_kernel",
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "avg_launch_us": avg_launch_ms * 1e3,
                     "p10_launch_us": float(np.percentile(launch_ms, 10)) * 1e3,
                     "p90_launch_us": float(np.percentile(launch_ms, 90)) * 1e3},
    }

    if not args.no_e2e:
        # host plan + descriptor upload over PCIe + launch, every step
        e2e_steps = min(steps, 50)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(e2e_steps):
            p2 = R.Plan(case.offsets, case.echo, case.top_n, case.vocab, case.has_logits)
            if args.split:
                p2.set_split(args.split)
            if args.waves:
                p2.set_waves(args.waves)
            src = copies[i % n_copies]
            p2.compute(src if case.has_logits else None, None if case.has_logits else src,
                       case.tokens, case.sampled, lp, ids, ws, stream)
            p2.close()
        torch.cuda.synchronize()
        e2e_ms = (time.perf_counter() - t0) * 1e3 / e2e_steps
        result["e2e_host_inputs"] = {"ms_per_step": e2e_ms, "rows_per_s": read_rows / (e2e_ms * 1e-3),
                                     "note": "plan + descriptor upload from host + launch per step"}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, base, ntl)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
