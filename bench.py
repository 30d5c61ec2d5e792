"""Benchmark: ragged top-7 token log-probabilities on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default workload is the large prefill echo batch: 16 requests whose
prompt lengths are geometric with mean 2048 (clipped to [1, 4096]), 34637
echo rows in all, a vocabulary of 151936, top_n 5.  That is 21.05 GB of fp32
logits read per step, the largest configuration that fits one GPU.

A step is one pass of the whole device path over that batch, with the logits
and the row descriptors resident in HBM: lp_launch_ragged (the row kernel,
plus the merge kernel when rows are split).  The timed region is K steps back
to back on the launch stream between two HIP events on that stream;
`value` is rows read per second over it, and the roofline's `achieved` is the
algorithmic bytes of one launch over the mean step.  A second pass of K
steps with an event pair around each launch gives the spread (median, p10,
p90); those pairs add about 2 us to each interval, which matters only for
the short decode launches.

Beside it, each on the same run:
  compute_ragged  lp_compute_ragged per step: the descriptors built on the
                  host, uploaded over PCIe (or, up to 262144 rows, read by the
                  kernels from pinned host memory), then the launch.  Median,
                  p10 and p90 of the event intervals on the stream.  This is
                  the PCIe-inclusive rate; it is never `value`.
  compute_noalloc lp_compute_ragged_noalloc per step, the same way (plans
                  whose workspace fits its fixed 4 MiB).
  decode          the decode batch (256 rows of 128256, one boosted token per
                  row, top_n 7), measured the same way with its own roofline
                  fraction.
  probe           a plain streaming read of as many rows of the same width on
                  the same copies: the practical ceiling for these bytes;
                  beside it the fastest shape of the committed 36-shape
                  sweep (`--probe-sweep`, profiles/probe_sweep_<workload>.txt),
                  as recorded there and timed again in this run.
  cpu_baseline    the CPU oracle on the host, run before the GPU is touched:
                  one process, then one process per available core (at most
                  16), each on rows of the same workload drawn on the host.
                  After the GPU legs, the oracle also recomputes a few of the
                  timed output rows from their logits copied back, and the
                  line reports how many were checked and how many differ.

The headline takes exactly W untimed warmup steps (without --warmup, about
100 ms of launches: 4000 for decode, 5 for the prefill batch).  Every other
leg (the decode record, lp_compute_ragged, the probe) keeps launching untimed
for at least 100 ms first: after an idle spell the first milliseconds of
short launches run slower than the steady state.

Workloads that fit the 256 MB Infinity Cache are timed while cycling through
copies of the logits whose read rows total at least 1 GiB.

Prints one JSON line (N = 1: the benchmark drives one GPU).

    python bench.py --cpu-full
times the oracle on every workload in full on the host (all cores) and
prints one JSON line per workload.

    python bench.py --workload W --write-profile TRACE_DIR FETCH_DIR WRITE_DIR
    python bench.py --workload W --write-counter-table NAME DIR [DIR ...]
    python bench.py --write-default-trace TRACE_DIR BENCH_LOG
write the committed summaries under profiles/ from rocprofv3 csv output
(each summary names the rocprofv3 command that made it).
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
DEFAULT_WORKLOAD = "prefill_echo_large"
SUB_WORKLOAD = "decode_peaked"
DEFAULT_STEPS = {"no_echo_next_token": 200, "ragged_echo_mix": 200, "decode_peaked": 200,
                 "prefill_echo_large": 20, "tie_edge_stress": 30}
# untimed warmup steps when --warmup is not given: about 100 ms of launches,
# after which short launches run at their steady-state rate
DEFAULT_WARMUP = {"no_echo_next_token": 10000, "ragged_echo_mix": 6000, "decode_peaked": 4000,
                  "prefill_echo_large": 5, "tie_edge_stress": 5}
MAX_CPU_WORKERS = 16          # the host share of one GPU on the GPU machines
CPU_BUDGET_S = 8.0            # oracle seconds per CPU leg (one core, then all cores)
CPU_ROWS_PER_WORKER = 24      # rows a worker draws and then runs in repeated passes
PARITY_ROWS = 8               # timed output rows the oracle recomputes per workload
SUB_WARM_S = 0.1              # side legs: untimed launches for at least this long first


def algorithmic_bytes(plan_info, vocab):
    """Bytes a perfect implementation moves per launch: each read row once
    (4 V), C columns of fp32 + uint32 output (64 B at C = 8) and a 16 B
    descriptor per output row."""
    cols = int(plan_info["columns"])
    return int(plan_info["read_rows"]) * 4 * vocab + int(plan_info["out_rows"]) * (8 * cols + 16)


# ---------------------------------------------------------------- CPU baseline leg

def _host_facts():
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "cores_available": int(avail), "cpu_count": os.cpu_count()}


def _sample_tasks(case, requests, k, cols):
    """(row, chosen, top_n) for the first min(k, count) output rows of each
    given request, with the rows drawn on the host (gen.request_rows_sample):
    exactly the rows the workload reads for echo and next-token requests,
    rows of the same distribution for a non-echo request with full logits."""
    import gen
    import oracle.logprob_oracle as LO

    tasks_all = LO.row_tasks(case.offsets, case.echo, case.top_n, case.tokens, case.sampled,
                             case.has_logits)
    counts, out_off = LO.output_counts_and_offsets(case.offsets, case.echo)
    out = []
    for n in requests:
        rows = gen.request_rows_sample(case, n, k)
        for j in range(min(k, int(counts[n]), rows.shape[0])):
            t = tasks_all[int(out_off[n]) + j]
            out.append((rows[j], t.chosen, t.top_n))
    return out


def _oracle_passes(tasks, cols, budget_s):
    """Runs the oracle's row computation over `tasks` in repeated passes
    until budget_s has been spent; returns (rows done, seconds)."""
    import oracle.logprob_oracle as LO

    done, t0 = 0, time.perf_counter()
    while True:
        for row, chosen, top_n in tasks:
            LO.compute_row(row, chosen, top_n, cols)
            done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return done, el


def _cpu_worker(case, requests, k, cols, budget_s, barrier, queue):
    # a forked child: `case` is the parent's object, not a pickled copy
    tasks = _sample_tasks(case, requests, k, cols)
    barrier.wait()
    queue.put(_oracle_passes(tasks, cols, budget_s))


def cpu_baseline(case, cols, budget_s=CPU_BUDGET_S, rows_per_worker=CPU_ROWS_PER_WORKER):
    """The oracle as it stands (never tuned for this), on the host cores, on
    a bounded sample of the workload: first one process, then one process
    per available core (at most MAX_CPU_WORKERS) started together, each
    running its own rows in repeated passes for budget_s.  Must run before
    this process touches the GPU: the pool is forked."""
    import multiprocessing as mp

    live = [n for n in range(case.batch) if int(case.top_n[n]) > 0]
    facts = _host_facts()
    if not live:
        return {"value": 0.0, "unit": "rows/s", "cores": 0, "kind": "oracle",
                "sample": "no request reads a row", "host": facts}
    one = _sample_tasks(case, live[:1] if case.echo[live[0]] else live[:rows_per_worker],
                        rows_per_worker, cols)
    n1, t1 = _oracle_passes(one, cols, budget_s)

    workers = max(1, min(MAX_CPU_WORKERS, facts["cores_available"]))
    ctx = mp.get_context("fork")
    barrier, queue = ctx.Barrier(workers), ctx.Queue()
    procs = []
    for w in range(workers):
        if case.echo[live[w % len(live)]]:
            reqs = [live[w % len(live)]]
        else:
            reqs = [live[(w * rows_per_worker + i) % len(live)] for i in range(rows_per_worker)]
        p = ctx.Process(target=_cpu_worker, args=(case, reqs, rows_per_worker, cols,
                                                  budget_s, barrier, queue))
        p.start()
        procs.append(p)
    results = [queue.get(timeout=600) for _ in procs]
    for p in procs:
        p.join(timeout=60)
    rows_all = sum(r[0] for r in results)
    span = max(r[1] for r in results)
    rate = rows_all / span
    v = case.vocab
    return {
        "value": rate, "unit": "rows/s", "cores": workers, "kind": "oracle",
        "gbs": rate * 4 * v / 1e9,
        "sample": (f"{case.name}: each of {workers} processes draws up to {rows_per_worker} "
                   f"read rows on the host (of one echo request, else one row from each of "
                   f"{rows_per_worker} requests; each request's own seed and distribution) "
                   f"and runs the oracle over them in repeated passes for {budget_s:.0f} s, all "
                   f"starting together; {rows_all} rows in {span:.1f} s (float64 log-softmax and "
                   f"a full stable sort per row)"),
        "one_core": {"value": n1 / t1, "unit": "rows/s", "rows": n1, "seconds": t1,
                     "gbs": n1 / t1 * 4 * v / 1e9},
        "host": facts,
    }


def cpu_check_timed_rows(case, src, lp_dev, ids_dev, cols, nrows=PARITY_ROWS, seed=7):
    """The oracle on a few of the timed output rows: their logits copied back
    from the device tensor the GPU read, the oracle's row recomputed on one
    thread, ids compared bit for bit and logprobs within 1e-5 (NaN and
    infinities exactly).  Returns the counts and the oracle's one-thread
    rate on these rows."""
    import oracle.logprob_oracle as LO

    tasks = LO.row_tasks(case.offsets, case.echo, case.top_n, case.tokens, case.sampled,
                         case.has_logits)
    live = [o for o, t in enumerate(tasks) if t.top_n > 0]
    if not live:
        return {"rows_checked": 0, "mismatches": 0}
    rng = np.random.default_rng(seed)
    pick = sorted(set([live[0], live[-1]] +
                      [int(x) for x in rng.choice(live, size=min(nrows, len(live)), replace=False)]))
    pick = pick[:max(nrows, 2)]
    mism, worst, t_or = 0, 0.0, 0.0
    for o in pick:
        t = tasks[o]
        row = src[t.src_row].cpu().numpy()
        t0 = time.perf_counter()
        want_lp, want_id = LO.compute_row(row, t.chosen, t.top_n, cols)
        t_or += time.perf_counter() - t0
        got_lp = lp_dev[o].cpu().numpy()
        got_id = ids_dev[o].cpu().numpy()
        ok = np.array_equal(got_id, want_id)
        nan_g, nan_w = np.isnan(got_lp), np.isnan(want_lp)
        ok &= np.array_equal(nan_g, nan_w)
        inf = np.isinf(want_lp) | np.isinf(got_lp)
        ok &= np.array_equal(got_lp[inf & ~nan_g], want_lp[inf & ~nan_w])
        fin = ~nan_g & ~nan_w & ~inf
        d = float(np.max(np.abs(got_lp[fin].astype(np.float64) - want_lp[fin]), initial=0.0))
        worst = max(worst, d)
        ok &= d <= 1e-5
        mism += 0 if ok else 1
    return {"rows_checked": len(pick), "mismatches": mism, "max_abs_lp_diff": worst,
            "rows": pick, "oracle_one_thread_rows_per_s": len(pick) / t_or}


def cpu_full(names):
    """The oracle on every read row of each workload, on the host, one process
    per available core (at most MAX_CPU_WORKERS) over requests, rows drawn on
    the host per request (gen.request_logits_host)."""
    import multiprocessing as mp

    facts = _host_facts()
    workers = max(1, min(MAX_CPU_WORKERS, facts["cores_available"]))
    ctx = mp.get_context("fork")
    for name in names:
        import gen

        case = gen.WORKLOADS[name]()
        live = [n for n in range(case.batch) if int(case.top_n[n]) > 0]
        t0 = time.perf_counter()
        with ctx.Pool(workers) as pool:
            res = pool.map(_full_request, [(name, n) for n in live], chunksize=1)
        wall = time.perf_counter() - t0
        rows = sum(r[0] for r in res)
        busy = sum(r[1] for r in res)
        print(json.dumps({"workload": name, "rows": rows, "wall_s": wall, "cores": workers,
                          "rows_per_s": rows / wall, "gbs": rows * 4 * case.vocab / wall / 1e9,
                          "oracle_busy_s": busy, "one_core_rows_per_s": rows / busy,
                          "host": facts,
                          "note": "oracle over every read row; wall time includes drawing the "
                                  "rows on the host; one_core_rows_per_s excludes it"}),
              flush=True)


def _full_request(arg):
    import gen
    import oracle.logprob_oracle as LO

    name, n = arg
    case = gen.WORKLOADS[name]()
    tasks = LO.row_tasks(case.offsets, case.echo, case.top_n, case.tokens, case.sampled,
                         case.has_logits)
    counts, out_off = LO.output_counts_and_offsets(case.offsets, case.echo)
    r0, _ = case.request_rows(n)
    x = gen.request_logits_host(case, n)
    busy, done = 0.0, 0
    for j in range(int(counts[n])):
        t = tasks[int(out_off[n]) + j]
        t0 = time.perf_counter()
        LO.compute_row(x[t.src_row - r0], t.chosen, t.top_n, 8)
        busy += time.perf_counter() - t0
        done += 1
    return done, busy


# ---------------------------------------------------------------- GPU legs

def _stats_us(ms_list):
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return {"mean_us": float(a.mean()), "median_us": float(np.median(a)),
            "p10_us": float(np.percentile(a, 10)), "p90_us": float(np.percentile(a, 90))}


def _timed_calls(calls, n_copies, steps, stream, torch):
    """Runs steps calls back to back on `stream`, an event pair around each;
    returns (per-call ms list, total ms from the first event to the last)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[2 * i].record(stream)
        calls[i % n_copies]()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]
    return per, ev[0].elapsed_time(ev[-1])


def _grouped_ms(calls, n_copies, steps, stream, torch):
    """Mean ms per call over steps calls with no event between them."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        calls[i % n_copies]()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _warm(calls, n_copies, steps, min_s, torch):
    """`steps` untimed calls, then more in groups until `min_s` seconds have
    passed.  Back to back after an idle spell (drawing a workload, another
    leg's setup) the first milliseconds of launches run slower than the
    steady state (decode, 256 rows of 128256: 24.6 against 23.0 us per
    launch after 10 warmup launches, and 23.0 after 100 ms of them)."""
    i = 0
    for i in range(steps):
        calls[i % n_copies]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_s:
        for _ in range(32):
            i += 1
            calls[i % n_copies]()
        torch.cuda.synchronize()


NOALLOC_WORKSPACE_BYTES = 4 << 20   # lp_compute_ragged_noalloc's fixed workspace

PROBE_SHAPES = [(segs, threads, loads) for segs in (1, 2, 4) for threads in (256, 512, 1024)
                for loads in (1, 2, 4, 8)]


def probe_sweep(R, torch, dev, stream, case, args):
    """The plain-read probe (lp_bench_stream_read_shape) in every launch
    shape of PROBE_SHAPES over the workload's read rows, on the same cycled
    copies as the bench: one JSON line per shape, then the fastest."""
    import gen

    base = gen.device_logits(case, dev, torch)
    plan = make_plan(R, case, args)
    rows = int(plan.info()["read_rows"])
    plan.close()
    read_bytes = rows * 4 * case.vocab
    n_copies = max(1, math.ceil(ROTATE_BYTES / max(read_bytes, 1)))
    copies = [base] + [base.clone() for _ in range(n_copies - 1)]
    steps = args.steps or DEFAULT_STEPS.get(case.name, 50)
    best = None
    for segs, threads, loads in PROBE_SHAPES:
        partial = torch.empty(rows * segs, dtype=torch.float32, device=dev)
        launch = [R.binding.stream_read_shape_launcher(c, rows, case.vocab, segs, threads, loads,
                                                       partial, stream) for c in copies]
        _warm(launch, n_copies, 3, SUB_WARM_S, torch)
        us = _grouped_ms(launch, n_copies, steps, stream, torch) * 1e3
        rec = {"workload": case.name, "rows": rows, "row_len": case.vocab, "segments": segs,
               "threads": threads, "loads_per_thread": loads, "us": us,
               "gbs": read_bytes / (us * 1e-6) / 1e9,
               "frac": read_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
               "copies_cycled": n_copies, "steps": steps}
        print(json.dumps(rec), flush=True)
        if best is None or us < best["us"]:
            best = rec
    print(json.dumps({"probe_sweep_best": best, "shapes": len(PROBE_SHAPES)}), flush=True)


def make_plan(R, case, args):
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
    return plan


def measure(R, torch, dev, stream, case, args, steps, warmup, probe=True, extras=True,
            warm_s=SUB_WARM_S):
    """Times one workload: kernel path with resident descriptors (the step),
    lp_compute_ragged per step, the probe; returns the record and what the
    parity check needs."""
    import gen

    base = gen.device_logits(case, dev, torch)
    plan = make_plan(R, case, args)
    info = plan.info()
    read_rows = int(info["read_rows"])
    read_bytes = read_rows * 4 * case.vocab
    alg = algorithmic_bytes(info, case.vocab)
    n_copies = max(1, math.ceil(ROTATE_BYTES / max(read_bytes, 1)))
    copies = [base] + [base.clone() for _ in range(n_copies - 1)]
    with torch.cuda.stream(stream):
        lp, ids, ws = R.alloc_outputs(plan, dev, torch)
    torch.cuda.synchronize()
    plan.stage(case.tokens, case.sampled, ws, stream)     # descriptors resident in HBM

    def srcs(c):
        return (c, None) if case.has_logits else (None, c)

    launch = [plan.launcher(*srcs(c), lp, ids, ws, stream) for c in copies]
    _warm(launch, n_copies, warmup, warm_s, torch)
    t0 = time.perf_counter()
    ms_per_step = _grouped_ms(launch, n_copies, steps, stream, torch)
    wall = time.perf_counter() - t0
    per, _ = _timed_calls(launch, n_copies, steps, stream, torch)
    st = _stats_us(per)
    rec = {
        "workload": case.name, "batch": case.batch, "vocab": case.vocab, "levels": args.levels,
        "max_top_n": int(np.max(case.top_n)) if case.batch else 0,
        "out_rows": int(info["out_rows"]), "read_rows": read_rows,
        "split": int(info["split"]), "waves": int(info["waves"]), "depth": int(info["depth"]),
        "direct_rows": int(info["direct_rows"]), "logits_copies_cycled": n_copies,
        "algorithmic_bytes_per_launch": alg, "steps": steps, "ms_per_step": ms_per_step,
        "host_wall_s": wall, "rows_per_s": read_rows / (ms_per_step * 1e-3),
        "launch_with_event_pairs": st,
        "gbs": alg / (ms_per_step * 1e-3) / 1e9,
    }
    rec["frac"] = rec["gbs"] / HBM_PEAK_GBS
    if extras:
        # lp_compute_ragged per step: host descriptors, their upload (or, up
        # to 262144 rows, the kernels' reads of them in pinned host memory),
        # the launch
        comp = [plan.computer(*srcs(c), case.tokens, case.sampled, lp, ids, ws, stream)
                for c in copies]
        _warm(comp, n_copies, 3, SUB_WARM_S, torch)
        cper, _ = _timed_calls(comp, n_copies, steps, stream, torch)
        cs = _stats_us(cper)
        rec["compute_ragged"] = dict(cs, rows_per_s=read_rows / (cs["median_us"] * 1e-6),
                                     gbs=alg / (cs["median_us"] * 1e-6) / 1e9,
                                     note="lp_compute_ragged per step (host descriptor build, "
                                          "upload or, up to 262144 rows, reads from pinned host "
                                          "memory, launch); event interval on the stream")
        # lp_compute_ragged_noalloc per step, where the plan fits its fixed
        # workspace: up to 1984 rows the descriptors go in upload launches
        # and the call waits for nothing; larger plans copy them
        # synchronously, so the host waits for the stream at every call
        if int(info["workspace_bytes"]) <= NOALLOC_WORKSPACE_BYTES:
            na = [plan.noalloc_computer(*srcs(c), case.tokens, case.sampled, lp, ids, stream)
                  for c in copies]
            _warm(na, n_copies, 3, SUB_WARM_S, torch)
            nper, _ = _timed_calls(na, n_copies, steps, stream, torch)
            ns = _stats_us(nper)
            rec["compute_noalloc"] = dict(
                ns, rows_per_s=read_rows / (ns["median_us"] * 1e-6),
                note="lp_compute_ragged_noalloc per step (the library's fixed workspace; up to "
                     "1984 rows descriptors in upload-kernel arguments, else a synchronous "
                     "copy); event interval on the stream")
        # leave the resident descriptors in place for the parity check
        plan.stage(case.tokens, case.sampled, ws, stream)
        launch[0]()
        torch.cuda.synchronize()
    if probe and case.vocab % 4 == 0 and read_rows > 0:
        rec["probe"] = bench_probe(copies, n_copies, read_rows, case.vocab, steps, stream, torch,
                                   dev, R, ms_per_step * 1e3)
        best = stored_probe_best(case.name) if args.levels == 3 and args.top_n is None else None
        if best is not None:
            best["kernel_time_over_best"] = ms_per_step * 1e3 / best["us"]
            rec["probe"]["sweep_best"] = best
            if "segments" in best:
                # the sweep's fastest shape, timed again here on this machine
                segs, thr, loads = best["segments"], best["threads"], best["loads"]
                partial = torch.empty(read_rows * segs, dtype=torch.float32, device=dev)
                pl = [R.binding.stream_read_shape_launcher(c, read_rows, case.vocab, segs, thr, loads,
                                                           partial, stream) for c in copies]
                _warm(pl, n_copies, 3, SUB_WARM_S, torch)
                us = _grouped_ms(pl, n_copies, steps, stream, torch) * 1e3
                gbs = read_bytes / (us * 1e-6) / 1e9
                rec["probe"]["best_shape_live"] = {
                    "us": us, "gbs": gbs, "frac": gbs / HBM_PEAK_GBS,
                    "kernel_time_over_best": ms_per_step * 1e3 / us,
                    "note": "the sweep's fastest plain-read shape, timed in this run"}
    return rec, plan, info, base, lp, ids, ws, copies


def bench_probe(copies, n_copies, rows, vocab, steps, stream, torch, dev, R, kernel_us):
    """The plain streaming read (lp_bench_stream_read: one workgroup per row,
    nontemporal 16-byte loads, a sum per row) over as many rows of the same
    width, cycling through the same copies: what the memory system gives a
    kernel that only reads these bytes."""
    partial = torch.empty(max(rows, 1), dtype=torch.float32, device=dev)
    launch = [R.binding.stream_read_launcher(c, rows, vocab, partial, stream) for c in copies]
    _warm(launch, n_copies, 3, SUB_WARM_S, torch)
    us = _grouped_ms(launch, n_copies, steps, stream, torch) * 1e3
    gbs = rows * vocab * 4 / (us * 1e-6) / 1e9
    return {"us": us, "gbs": gbs, "frac": gbs / HBM_PEAK_GBS,
            "kernel_time_over_probe": kernel_us / us,
            "note": "plain read of the same number of rows and row width, same copies cycled, "
                    "steps back to back between two events"}


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

    rec_calls = [[plan.shard_records_launcher(bounds[k][0], t if case.has_logits else None,
                                              None if case.has_logits else t, rec[k], ws, stream)
                  for k, t in enumerate(copy_shards)] for copy_shards in shards]
    merge = plan.merge_launcher(S, rec, lp, ids, ws, stream)

    def records(i, k):
        rec_calls[i % len(rec_calls)][k]()

    steps = 50
    for i in range(3):
        records(i, 0)
    merge()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for i in range(steps):
        records(i, i % S)
    ev[1].record(stream)
    for i in range(steps):
        merge()
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps before the K timed ones (default: about 100 ms "
                         "of launches of the workload, 5 for the large batches)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
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
    ap.add_argument("--probe-sweep", action="store_true",
                    help="time the plain-read probe in every launch shape (1, 2 or 4 workgroups "
                         "per row; 256, 512 or 1024 threads; 1-8 loads in flight per thread) "
                         "over the workload's read rows, print one JSON line per shape, exit")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the plain-read probe over the same rows (the practical ceiling)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode sub-record")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle on every workload in full on the host, then exit")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run 3 plain device copies of this many MiB "
                         "(a known-size kernel for calibrating FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="print the rows of rocprofv3 csv output directories")
    ap.add_argument("--write-counter-table", nargs="+", metavar="ARG",
                    help="NAME DIR [DIR ...]: write profiles/NAME.txt, the per-dispatch mean of "
                         "every counter in these rocprofv3 --pmc runs of this workload, per kernel")
    ap.add_argument("--write-default-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                    help="write profiles/bench_default_trace.txt from a kernel-trace run of the "
                         "default bench line and that run's output")
    ap.add_argument("--write-profile", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/row_kernel_<workload>_{trace,counters}.txt from a "
                         "kernel-trace run and FETCH_SIZE / WRITE_SIZE runs of this workload")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.write_default_trace:
        write_default_trace(*args.write_default_trace)
        return
    if args.write_profile:
        write_profile(args.workload, *args.write_profile, split=args.split, waves=args.waves)
        return
    if args.write_counter_table:
        write_counter_table(args.workload, args.write_counter_table[0], args.write_counter_table[1:])
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark drives one GPU; --gpus must be 1 (rows "
                                   "shard across GPUs with no exchange, but no multi-GPU "
                                   "path is provided)", "n_gpus": args.gpus}),
              flush=True)
        sys.exit(2)

    import gen

    if args.cpu_full:
        cpu_full(list(gen.WORKLOADS))
        return

    case = gen.WORKLOADS[args.workload]()
    if args.top_n is not None:
        case.top_n = np.where(np.asarray(case.top_n) > 0, args.top_n, 0).astype(np.int32)
    cols = 1 << args.levels if args.levels > 0 else 1
    cpu = None
    if not args.no_cpu_baseline and not args.probe_sweep:
        # before anything touches the GPU: the pool forks this process
        cpu = cpu_baseline(case, cols)

    import torch

    import ragged_token_log_amd as R

    R.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    steps = args.steps or DEFAULT_STEPS.get(args.workload, 50)
    warmup = args.warmup if args.warmup is not None else DEFAULT_WARMUP.get(args.workload, 5)
    if args.probe_sweep:
        probe_sweep(R, torch, dev, stream, case, args)
        return

    main_rec, plan, info, base, lp, ids, ws, copies = measure(
        R, torch, dev, stream, case, args, steps, warmup, probe=not args.no_probe,
        warm_s=0.0)
    ms_per_step = main_rec["ms_per_step"]
    read_rows = main_rec["read_rows"]
    st = main_rec["launch_with_event_pairs"]
    alg = main_rec["algorithmic_bytes_per_launch"]
    achieved = main_rec["gbs"]

    result = {
        "metric": METRIC,
        "value": read_rows / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded draws with the workload's shapes and distributions)",
        "config": {k: main_rec[k] for k in ("workload", "batch", "vocab", "levels", "max_top_n",
                                            "out_rows", "read_rows", "split", "waves", "depth",
                                            "direct_rows", "logits_copies_cycled")},
        "hbm_gbs": alg / (ms_per_step * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "row_kernel",
                     "algorithmic_bytes_per_launch": alg,
                     "avg_launch_us": ms_per_step * 1e3,
                     "median_launch_us_event_pairs": st["median_us"],
                     "p10_launch_us_event_pairs": st["p10_us"],
                     "p90_launch_us_event_pairs": st["p90_us"]},
    }
    result["config"]["temperature"] = args.temperature if args.temperature is not None else 1.0
    result["config"]["top_k"] = args.top_k
    for k in ("compute_ragged", "compute_noalloc", "probe"):
        if k in main_rec:
            result[k] = main_rec[k]

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

    if args.shards:
        result["shards"] = bench_shards(args, case, plan, info, copies, len(copies), torch, dev,
                                        stream, ws)

    traffic = stored_traffic(case.name, info, algorithmic_bytes(info, case.vocab))
    if traffic is not None:
        result["roofline"]["traffic"] = traffic

    checks = []
    if cpu is not None:
        checks.append(cpu_check_timed_rows(case, base, lp, ids, cols))
    del copies, base

    if not args.no_decode and args.workload != SUB_WORKLOAD:
        dcase = gen.WORKLOADS[SUB_WORKLOAD]()
        if args.top_n is not None:
            dcase.top_n = np.where(np.asarray(dcase.top_n) > 0, args.top_n, 0).astype(np.int32)
        drec, dplan, dinfo, dbase, dlp, dids, _, dcopies = measure(
            R, torch, dev, stream, dcase, args, DEFAULT_STEPS[SUB_WORKLOAD], warmup,
            probe=not args.no_probe)
        dtraffic = stored_traffic(dcase.name, dinfo, algorithmic_bytes(dinfo, dcase.vocab))
        drec["traffic"] = dtraffic
        result["decode"] = drec
        if cpu is not None:
            checks.append(cpu_check_timed_rows(dcase, dbase, dlp, dids, cols))
        del dcopies, dbase

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        a = torch.ones(n, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if cpu is not None:
        cpu["timed_rows_check"] = checks
        result["cpu_baseline"] = cpu
        result["parity_rows_checked"] = sum(c["rows_checked"] for c in checks)
        result["mismatches"] = sum(c["mismatches"] for c in checks)

    print(json.dumps(result), flush=True)
    if result.get("mismatches"):
        sys.exit(1)


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


def stored_traffic(workload, info, alg):
    """HBM bytes per launch of the row kernel from the committed counter
    summary for this workload, if it was taken on the current kernel source,
    the same kernel shape and the same algorithmic bytes (rows, width and
    columns: another --levels moves other bytes); else None."""
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
    if vals.get("algorithmic_bytes_per_launch") != str(int(alg)):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stored_probe_best(workload):
    """The fastest plain-read shape in the committed sweep for this workload
    (profiles/probe_sweep_<workload>.txt, written from `bench.py
    --probe-sweep`), as {"us", "frac", "shape"}; None without one."""
    import re

    path = os.path.join(PROFILES, f"probe_sweep_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        for line in f:
            m = re.match(r"fastest: (.*): ([0-9.]+) us, ([0-9.]+) of 8 TB/s", line.strip())
            if m:
                shape = re.match(r"(\d+) segment\(s\), (\d+) threads, (\d+) load\(s\) per thread",
                                 m.group(1))
                rec = {"us": float(m.group(2)), "frac": float(m.group(3)), "shape": m.group(1),
                       "source": f"profiles/probe_sweep_{workload}.txt"}
                if shape:
                    rec["segments"], rec["threads"], rec["loads"] = (int(g) for g in shape.groups())
                return rec
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
                f"-- python bench.py --workload {workload} --no-cpu-baseline --no-decode{flags}\n")
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
                    f"--no-decode --no-probe --copy-probe-mb 256{flags}\n")
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


def write_default_trace(trace_dir, bench_log):
    """profiles/bench_default_trace.txt: the kernel-trace statistics of one
    rocprofv3 run of the default bench line (`bench.py` with no flags) and
    that run's JSON line, the row kernel of each workload matched by its
    shape (slot count, waves, depth) as the line reports it."""
    with open(bench_log, encoding="utf-8") as f:
        line = [x for x in f if x.startswith("{")][-1]
    d = json.loads(line)
    legs = [("prefill_echo_large", d["config"], d["roofline"]["algorithmic_bytes_per_launch"]),
            ("decode_peaked", d["decode"], d["decode"]["algorithmic_bytes_per_launch"])]
    out = ["rocprofv3 kernel trace of the default bench line (prefill_echo_large, with the "
           "decode_peaked sub-record)",
           "command: rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o default "
           "-- python3 bench.py",
           f"kernel_source_sha256: {kernel_source_hash()}"]
    for r in _kernel_rows(trace_dir, "kernel_stats.csv"):
        name = r["Name"]
        if not any(t in name for t in ("row_kernel", "stream_read_kernel", "merge_kernel")):
            continue
        avg = float(r["AverageNs"])
        out.append(f"kernel: {name}")
        out.append(f"  calls={r['Calls']} avg_ns={avg:.0f} min_ns={r['MinNs']} max_ns={r['MaxNs']}")
        for wl, cfg, alg in legs:
            k = (1 << int(cfg["levels"])) - 1
            if f"row_kernel<{k}, {int(cfg['waves'])}, {int(cfg['depth'])}," in name:
                out.append(f"  workload {wl}: algorithmic_bytes_per_launch={alg}  GB/s at avg = "
                           f"{alg / avg:.1f}  fraction of 8 TB/s = {alg / avg / HBM_PEAK_GBS:.4f}")
                break
        else:
            if "stream_read_kernel" in name:
                out.append("  (the plain-read probe over both workloads' rows: calls of both "
                           "sizes averaged together)")
    out.append(f"bench line of the same run: headline avg_launch_us = "
               f"{d['roofline']['avg_launch_us']:.1f} (frac {d['roofline']['frac']:.4f}); decode "
               f"ms_per_step = {d['decode']['ms_per_step'] * 1e3:.2f} us (frac "
               f"{d['decode']['frac']:.4f})")
    with open(os.path.join(PROFILES, "bench_default_trace.txt"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def write_counter_table(workload, name, dirs):
    """profiles/<name>.txt: for each rocprofv3 --pmc output directory (one
    run each, of `bench.py --workload <workload> --no-cpu-baseline
    --no-decode --steps 50 --warmup 5`), the per-dispatch mean of every counter, for
    the log-probability kernels and the plain-read probe."""
    rows = {}
    cmds = []
    for d in dirs:
        names = set()
        for r in _kernel_rows(d, "counter_collection.csv"):
            k = r["Kernel_Name"]
            if not any(t in k for t in ("row_kernel", "merge_kernel", "stream_read_kernel")):
                continue
            names.add(r["Counter_Name"])
            rows.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        cmds.append(f"rocprofv3 --pmc {' '.join(sorted(names))} --output-format csv -d <dir> -o <name> "
                    f"-- python bench.py --workload {workload} --no-cpu-baseline --no-decode --steps 50 "
                    f"--warmup 5")
    with open(os.path.join(PROFILES, f"{name}.txt"), "w") as f:
        f.write(f"rocprofv3 counters: {workload} (per-dispatch mean over the run's dispatches)\n")
        for c in cmds:
            f.write(f"command: {c}\n")
        f.write(f"kernel_source_sha256: {kernel_source_hash()}\n")
        for k, cs in sorted(rows.items()):
            f.write(f"kernel: {k}\n")
            for c, v in sorted(cs.items()):
                f.write(f"  {c}: {sum(v) / len(v):.1f}  (dispatches={len(v)})\n")
    print(f"wrote profiles/{name}.txt")


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
