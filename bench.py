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
    (4 V), C columns of fp32 + uint32 output (64 B at C = 8) and a 16 B
    descriptor per output row."""
    cols = int(plan_info["columns"])
    return int(plan_info["read_rows"]) * 4 * vocab + int(plan_info["out_rows"]) * (8 * cols + 16)


def cpu_baseline(case, logits_dev, ntl_dev, cols=8, budget_s=10.0, max_rows=2000):
    """The oracle as it stands, on a bounded sample of the same workload: the
    first read rows in output order (at most max_rows), in repeated passes
    until about budget_s of oracle time has been spent."""
    import oracle.logprob_oracle as LO

    tasks = LO.row_tasks(case.offsets, case.echo, case.top_n, case.tokens, case.sampled,
                         case.has_logits)
    live = [o for o, t in enumerate(tasks) if t.top_n > 0][:max_rows]
    src = logits_dev if case.has_logits else ntl_dev
    rows = {}
    for o in live:
        r = tasks[o].src_row
        if r not in rows:
            rows[r] = src[r].cpu().numpy()
    done, t_total, passes = 0, 0.0, 0
    while t_total < budget_s:
        passes += 1
        for o in live:
            t = tasks[o]
            t0 = time.perf_counter()
            LO.compute_row(rows[t.src_row], t.chosen, t.top_n, cols)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= budget_s and passes > 1:
                break
    return {"value": done / t_total, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {len(live)} read rows of {case.name}, {passes} passes, "
                      f"{done} rows in {t_total:.1f} s (float64 log-softmax + full stable sort "
                      f"per row, one thread)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ragged_echo_mix")
    ap.add_argument("--split", type=int, default=None, help="force the plan's split")
    ap.add_argument("--waves", type=int, default=None, help="force waves per workgroup (4|8|16)")
    ap.add_argument("--levels", type=int, default=3,
                    help="heap depth: 2**levels output columns, top_n up to 2**levels - 1")
    ap.add_argument("--top-n", type=int, default=None,
                    help="replace every nonzero top_n of the workload with this value")
    ap.add_argument("--shards", type=int, default=0,
                    help="also time the vocabulary-sharded path: this many equal shards, "
                         "each reduced to records, then merged (all on this GPU)")
    ap.add_argument("--temperature", type=float, default=None,
                    help="log_softmax(logits / T) for every request")
    ap.add_argument("--top-k", type=int, default=0,
                    help="top-k front end (TopK on logits, then Softmax) for every request")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the plain-read probe over the same rows (the practical ceiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-e2e", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run 3 plain device copies of this many MiB "
                         "(a known-size kernel for calibrating FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="print the rows of rocprofv3 csv output directories")
    ap.add_argument("--write-profile", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/row_kernel_<workload>_{trace,counters}.txt from a "
                         "kernel-trace run and FETCH_SIZE / WRITE_SIZE runs of this workload")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.write_profile:
        write_profile(args.workload, *args.write_profile, split=args.split, waves=args.waves)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the log-probability kernels run on one GPU per process here; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import gen
    import ragged_token_log_amd as R

    R.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = gen.WORKLOADS[args.workload]()
    if args.top_n is not None:
        case.top_n = np.where(np.asarray(case.top_n) > 0, args.top_n, 0)
    steps = args.steps or DEFAULT_STEPS.get(args.workload, 50)
    stream = torch.cuda.current_stream(dev)

    base = gen.device_logits(case, dev, torch)
    last = torch.from_numpy(case.offsets[1:].astype(np.int64) - 1).to(dev)
    ntl = base.index_select(0, last) if case.has_logits else base
    copy_bytes = base.numel() * 4
    n_copies = max(1, math.ceil(ROTATE_BYTES / copy_bytes))
    copies = [base] + [base.clone() for _ in range(n_copies - 1)]
    torch.cuda.synchronize()

    plan = R.Plan(case.offsets, case.echo, case.top_n, case.vocab, case.has_logits,
                  levels=args.levels)
    if args.split:
        plan.set_split(args.split)
    if args.waves:
        plan.set_waves(args.waves)
    if args.temperature is not None:
        plan.set_temperature(args.temperature)
    if args.top_k:
        plan.set_top_k(args.top_k)
    info = plan.info()
    lp, ids, ws = R.alloc_outputs(plan, dev, torch)
    plan.stage(case.tokens, case.sampled, ws, stream)   # descriptors resident in HBM

    launchers = [plan.launcher(src if case.has_logits else None,
                               None if case.has_logits else src, lp, ids, ws, stream)
                 for src in copies]

    def step(i):
        launchers[i % n_copies]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed region runs the K steps back to back on the launch stream.
    # Events sit only between groups of steps (about ten groups), so that
    # recording them adds almost nothing to a step; the per-group averages
    # give the spread.
    group = max(1, steps // 10)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps // group + 2)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    bounds = [0]
    for i in range(steps):
        step(i)
        if (i + 1) % group == 0 or i + 1 == steps:
            marks[len(bounds)].record(stream)
            bounds.append(i + 1)
    torch.cuda.synchronize()
    total_ms = marks[0].elapsed_time(marks[len(bounds) - 1])
    group_ms = [marks[j - 1].elapsed_time(marks[j]) / (bounds[j] - bounds[j - 1])
                for j in range(1, len(bounds))]
    ms_per_step = total_ms / steps
    # one row-kernel launch per step when split == 1 (the plans of every
    # workload here); with split > 1 a step also holds the merge kernel, so
    # this is the duration of both
    avg_launch_ms = ms_per_step

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
                   "levels": args.levels, "max_top_n": int(np.max(case.top_n)),
                   "temperature": args.temperature if args.temperature is not None else 1.0,
                   "top_k": args.top_k,
                   "out_rows": int(info["out_rows"]), "read_rows": read_rows,
                   "split": int(info["split"]), "waves": int(info["waves"]),
                   "logits_copies_cycled": n_copies},
        "hbm_gbs": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "row_kernel",
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "avg_launch_us": avg_launch_ms * 1e3,
                     "p10_group_us": float(np.percentile(group_ms, 10)) * 1e3,
                     "p90_group_us": float(np.percentile(group_ms, 90)) * 1e3},
    }

    if not args.no_e2e:
        # host plan + descriptor upload over PCIe + launch, every step
        e2e_steps = min(steps, 50)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(e2e_steps):
            p2 = R.Plan(case.offsets, case.echo, case.top_n, case.vocab, case.has_logits,
                        levels=args.levels)
            if args.split:
                p2.set_split(args.split)
            if args.waves:
                p2.set_waves(args.waves)
            if args.temperature is not None:
                p2.set_temperature(args.temperature)
            if args.top_k:
                p2.set_top_k(args.top_k)
            src = copies[i % n_copies]
            p2.compute(src if case.has_logits else None, None if case.has_logits else src,
                       case.tokens, case.sampled, lp, ids, ws, stream)
            p2.close()
        torch.cuda.synchronize()
        e2e_ms = (time.perf_counter() - t0) * 1e3 / e2e_steps
        result["e2e_host_inputs"] = {"ms_per_step": e2e_ms, "rows_per_s": read_rows / (e2e_ms * 1e-3),
                                     "note": "plan + descriptor upload from host + launch per step"}

    # host result assembly (lp_assemble_ragged) on this step's outputs, after
    # their copy back: the per-request dicts of the page's compute_top
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    lp_h, ids_h = lp.cpu().numpy(), ids.cpu().numpy()
    t1 = time.perf_counter()
    reps = 0
    while True:
        plan.assemble(lp_h, ids_h)
        reps += 1
        if time.perf_counter() - t1 > 0.2:
            break
    asm_ms = (time.perf_counter() - t1) * 1e3 / reps
    result["host_assembly"] = {"ms": asm_ms, "rows_per_s": int(info["out_rows"]) / (asm_ms * 1e-3),
                               "copy_back_ms": (t1 - t0) * 1e3,
                               "note": "lp_assemble_ragged on the host, one thread; copy back "
                                       "of the (R, C) outputs timed separately"}

    if not args.no_probe and case.vocab % 4 == 0:
        result["probe"] = bench_probe(copies, n_copies, read_rows, case.vocab, steps, stream, torch,
                                      dev, R, alg_bytes, avg_launch_ms)

    if args.shards:
        result["shards"] = bench_shards(args, case, plan, info, copies, n_copies, torch, dev,
                                        stream, ws)

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        a = torch.ones(n, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    traffic = stored_traffic(case.name, info)
    if traffic is not None:
        result["roofline"]["traffic"] = traffic

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, base, ntl, cols=int(info["columns"]))

    print(json.dumps(result), flush=True)


def bench_probe(copies, n_copies, rows, vocab, steps, stream, torch, dev, R, alg_bytes, kernel_ms):
    """The plain streaming read (lp_bench_stream_read: one workgroup per row,
    nontemporal 16-byte loads, a sum per row) over as many rows of the same
    width, cycling through the same copies: what the memory system gives a
    kernel that only reads these bytes."""
    partial = torch.empty(max(rows, 1), dtype=torch.float32, device=dev)
    launch = [R.binding.stream_read_launcher(c, rows, vocab, partial, stream) for c in copies]
    for i in range(3):
        launch[i % n_copies]()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        launch[i % n_copies]()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    gbs = rows * vocab * 4 / (us * 1e-6) / 1e9
    return {"us": us, "gbs": gbs, "frac": gbs / HBM_PEAK_GBS,
            "kernel_time_over_probe": kernel_ms * 1e3 / us,
            "note": "plain read of the same number of rows and row width, same copies cycled"}


def bench_shards(args, case, plan, info, copies, n_copies, torch, dev, stream, ws):
    """The vocabulary-sharded path on one GPU: each of S equal column ranges
    of the logits as its own contiguous tensor (what one tensor-parallel rank
    holds), reduced to records; then the merge.  Times one shard's record
    kernel (what each rank runs) and the merge, each over the timed steps."""
    S = args.shards
    V = case.vocab
    bounds = [(k * V // S, (k + 1) * V // S) for k in range(S)]
    src_copies = copies[: max(1, min(n_copies, 4))]
    shards = [[c[:, b:e].contiguous() for (b, e) in bounds] for c in src_copies]
    words = int(info["record_words"])
    rec = torch.empty((S, int(info["out_rows"]), words), dtype=torch.int64, device=dev)
    lp = torch.empty((int(info["out_rows"]), int(info["columns"])), dtype=torch.float32, device=dev)
    ids = torch.empty(lp.shape, dtype=torch.uint32, device=dev)
    torch.cuda.synchronize()

    def records(i, k):
        t = shards[i % len(shards)][k]
        plan.shard_records(bounds[k][0], t if case.has_logits else None,
                           None if case.has_logits else t, rec[k], ws, stream)

    steps = 50
    for i in range(3):
        records(i, 0)
    plan.merge_shards(S, rec, lp, ids, ws, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for i in range(steps):
        records(i, i % S)
    ev[1].record(stream)
    for i in range(steps):
        plan.merge_shards(S, rec, lp, ids, ws, stream)
    ev[2].record(stream)
    torch.cuda.synchronize()
    rec_us = ev[0].elapsed_time(ev[1]) * 1e3 / steps
    merge_us = ev[1].elapsed_time(ev[2]) * 1e3 / steps
    shard_bytes = int(info["read_rows"]) * 4 * (V // S) + int(info["out_rows"]) * (16 + 8 * words)
    return {"n_shards": S, "record_kernel_us": rec_us, "merge_us": merge_us,
            "record_kernel_gbs": shard_bytes / (rec_us * 1e-6) / 1e9,
            "record_bytes_per_row": 8 * words,
            "note": "one shard's record kernel (what each tensor-parallel rank runs on its "
                    "columns) and the merge over all shards' records, each averaged over "
                    f"{steps} back-to-back launches; shard copies rotated"}


KERNEL_SOURCE = os.path.join(ROOT, "ragged_token_log_amd", "csrc", "logprob_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    """Hash of the device code (the kernels' namespace in the HIP source,
    comments and blank lines left out): host-side and comment edits leave
    recorded counters valid; the launch shape is checked separately."""
    import hashlib

    import re

    with open(KERNEL_SOURCE, "rb") as f:
        text = f.read()
    begin, end = text.index(b"namespace dev {"), text.index(b"}  // namespace dev")
    code = re.sub(rb"//[^\n]*", b"", text[begin:end])             # comments do not count
    code = b"\n".join(line.rstrip() for line in code.splitlines() if line.strip())
    return hashlib.sha256(code).hexdigest()[:16]


def shape_text(info):
    return (f"split={info['split']} waves={info['waves']} depth={info['depth']} "
            f"direct_rows={info['direct_rows']}")


def stored_traffic(workload, info):
    """HBM bytes per launch of the row kernel from the committed counter
    summary for this workload, if it was taken on the current kernel source
    and the same kernel shape; else None."""
    path = os.path.join(PROFILES, f"row_kernel_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    if vals.get("shape") != shape_text(info):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _read_csv(path):
    import csv

    with open(path, newline="", encoding="utf-8") as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    return None


COPY_PROBE_BYTES = 256 << 20


def _kernel_rows(d, suffix):
    path = _find(d, suffix)
    if path is None:
        raise SystemExit(f"no *{suffix} under {d}")
    return _read_csv(path)


def _counter_means(d):
    acc = {}
    for r in _kernel_rows(d, "counter_collection.csv"):
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def write_profile(workload, trace_dir, fetch_dir, write_dir, split=None, waves=None):
    """Writes the two committed summaries for `workload` from rocprofv3 csv
    output: kernel-trace statistics, and HBM traffic from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) scaled by what the same counters read for
    the 256 MiB device copy that --copy-probe-mb 256 runs."""
    import gen
    import ragged_token_log_amd as R

    case = gen.WORKLOADS[workload]()
    plan = R.Plan(case.offsets, case.echo, case.top_n, case.vocab, case.has_logits)
    if split:
        plan.set_split(split)
    if waves:
        plan.set_waves(waves)
    info = plan.info()
    alg = algorithmic_bytes(info, case.vocab)
    flags = (f" --split {split}" if split else "") + (f" --waves {waves}" if waves else "")
    stats = _kernel_rows(trace_dir, "kernel_stats.csv")
    ours = [r for r in stats if "row_kernel" in r["Name"] or "merge_kernel" in r["Name"]]
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"row_kernel_{workload}_trace.txt"), "w") as f:
        f.write(f"rocprofv3 kernel trace: {workload}\n")
        f.write(f"command: rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o trace "
                f"-- python bench.py --workload {workload} --no-cpu-baseline --no-e2e{flags}\n")
        f.write(f"shape: {shape_text(info)}\n")
        f.write(f"kernel_source_sha256: {kernel_source_hash()}\n")
        f.write(f"algorithmic_bytes_per_launch: {alg}\n")
        for r in ours:
            avg = float(r["AverageNs"])
            f.write(f"kernel: {r['Name']}\n  calls={r['Calls']} avg_ns={avg:.0f} "
                    f"min_ns={r['MinNs']} max_ns={r['MaxNs']} share_pct={float(r['Percentage']):.2f}\n"
                    f"  algorithmic GB/s at avg = {alg / avg:.1f}\n")
    fetch = _counter_means(fetch_dir)
    write = _counter_means(write_dir)
    copy_f = max(fetch.get("__amd_rocclr_copyBuffer", [0.0]))
    copy_w = max(write.get("__amd_rocclr_copyBuffer", [0.0]))
    kname = next(k for k in fetch if "row_kernel" in k)
    kf = sum(fetch[kname]) / len(fetch[kname])
    kw = sum(write[kname]) / len(write[kname])
    f_fetch = COPY_PROBE_BYTES / (copy_f * 1024.0)
    f_write = COPY_PROBE_BYTES / (copy_w * 1024.0)
    traffic = kf * 1024.0 * f_fetch + kw * 1024.0 * f_write
    with open(os.path.join(PROFILES, f"row_kernel_{workload}_counters.txt"), "w") as f:
        f.write(f"rocprofv3 counters: {workload}\n")
        for c, d in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            f.write(f"command_{d}: rocprofv3 --pmc {c} --output-format csv -d <dir> -o {d} -- python "
                    f"bench.py --workload {workload} --steps 5 --warmup 1 --no-cpu-baseline "
                    f"--no-e2e --copy-probe-mb 256{flags}\n")
        f.write(f"shape: {shape_text(info)}\n")
        f.write(f"kernel_source_sha256: {kernel_source_hash()}\n")
        f.write(f"kernel: {kname}\n")
        f.write(f"fetch_kib_per_dispatch: {kf:.1f}\n")
        f.write(f"write_kib_per_dispatch: {kw:.1f}\n")
        f.write(f"copy_probe: 256 MiB device copy (__amd_rocclr_copyBuffer) reads FETCH_SIZE "
                f"{copy_f:.1f} KiB and WRITE_SIZE {copy_w:.1f} KiB\n")
        f.write(f"fetch_scale: {f_fetch:.4f}\n")
        f.write(f"write_scale: {f_write:.4f}\n")
        f.write(f"traffic_bytes_per_launch: {traffic:.0f}\n")
        f.write(f"algorithmic_bytes_per_launch: {alg}\n")
        f.write(f"traffic_over_algorithmic: {traffic / alg:.4f}\n")
    print(f"wrote profiles for {workload}: traffic/algorithmic = {traffic / alg:.4f}")


def summarize(dirs):
    """Prints the rows of rocprofv3 csv output that the profile summaries use:
    kernel stats (name, calls, average / min / max ns) and, for counter runs,
    the per-dispatch average of each counter by kernel."""
    for d in dirs:
        print(f"== {d}")
        st = _find(d, "kernel_stats.csv")
        if st:
            for r in _read_csv(st):
                name = r.get("Name", "")[:60]
                print(f"  {name:60s} calls={r.get('Calls')} avg_ns={r.get('AverageNs')} "
                      f"min_ns={r.get('MinNs')} max_ns={r.get('MaxNs')} pct={r.get('Percentage')}")
        cc = _find(d, "counter_collection.csv")
        if cc:
            acc = {}
            for r in _read_csv(cc):
                key = (r.get("Kernel_Name", "")[:60], r.get("Counter_Name"))
                acc.setdefault(key, []).append(float(r.get("Counter_Value", "nan")))
            for (k, c), v in sorted(acc.items()):
                print(f"  {k:60s} {c}: dispatches={len(v)} mean={sum(v) / len(v):.1f} "
                      f"min={min(v):.1f} max={max(v):.1f}")


if __name__ == "__main__":
    main()
