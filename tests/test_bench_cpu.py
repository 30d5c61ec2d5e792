"""Host logic of bench.py (no GPU): the algorithmic bytes it prices a launch
at, the kernel-source hash that ties stored counters to the kernels, the
lookups of stored traffic and of the plain-read sweep's fastest shape, the
writers of the profile summaries (traffic scaled by the copy probe), and the
one-GPU refusal.  Fixture files
are written to a temporary directory, so the committed profiles are only
read, never changed."""
import json
import os
import subprocess
import sys

import pytest

import bench
import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_closed_form():
    """Rows read x V x 4, plus per output row C fp32 + C uint32 and a 16-byte
    descriptor."""
    info = {"columns": 8, "read_rows": 520, "out_rows": 530}
    assert bench.algorithmic_bytes(info, 32000) == 520 * 4 * 32000 + 530 * (8 * 8 + 16)
    info = {"columns": 1, "read_rows": 0, "out_rows": 7}
    assert bench.algorithmic_bytes(info, 5) == 7 * (8 + 16)


def test_kernel_source_hash_follows_device_code_only(tmp_path, monkeypatch):
    """Comments in the device namespace and host code outside it leave the
    hash alone; a change of device code moves it."""
    with open(bench.KERNEL_SOURCE, encoding="utf-8") as f:
        src = f.read()
    h0 = bench.kernel_source_hash()
    i = src.index("namespace dev {") + len("namespace dev {")
    edited = src[:i] + "\n    // a comment\n\n" + src[i:] + "\nstatic int host_only_addition = 0;\n"
    p = tmp_path / "kernels.hip"
    p.write_text(edited, encoding="utf-8")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(p))
    assert bench.kernel_source_hash() == h0
    j = edited.index("namespace dev {") + len("namespace dev {")
    p.write_text(edited[:j] + "\n__device__ int changed_device_code;\n" + edited[j:],
                 encoding="utf-8")
    assert bench.kernel_source_hash() != h0


def test_stored_traffic_only_for_the_same_source_shape_and_bytes(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    info = {"split": 1, "waves": 16, "depth": 1, "direct_rows": 1}
    alg = 131354624

    def write(source_hash, shape, alg_bytes):
        (tmp_path / "row_kernel_decode_peaked_counters.txt").write_text(
            "rocprofv3 counters: decode_peaked\n"
            f"shape: {shape}\n"
            f"kernel_source_sha256: {source_hash}\n"
            "traffic_bytes_per_launch: 131542471\n"
            f"algorithmic_bytes_per_launch: {alg_bytes}\n", encoding="utf-8")

    h = bench.kernel_source_hash()
    write(h, bench.shape_text(info), alg)
    assert bench.stored_traffic("decode_peaked", info, alg) == 131542471.0
    write("0" * 16, bench.shape_text(info), alg)                       # other kernels
    assert bench.stored_traffic("decode_peaked", info, alg) is None
    write(h, bench.shape_text(dict(info, waves=8)), alg)               # another shape
    assert bench.stored_traffic("decode_peaked", info, alg) is None
    write(h, bench.shape_text(info), alg + 64)                         # other bytes (levels)
    assert bench.stored_traffic("decode_peaked", info, alg) is None
    assert bench.stored_traffic("no_such_workload", info, alg) is None


def test_stored_probe_best_parses_the_sweep_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "probe_sweep_x.txt").write_text(
        "plain-read probe sweep: x\n"
        "fastest: 2 segment(s), 1024 threads, 1 load(s) per thread: 20.56 us, 0.798 of 8 TB/s\n",
        encoding="utf-8")
    r = bench.stored_probe_best("x")
    assert (r["us"], r["frac"]) == (20.56, 0.798)
    assert (r["segments"], r["threads"], r["loads"]) == (2, 1024, 1)
    assert bench.stored_probe_best("missing") is None


@pytest.mark.parametrize("workload", sorted(gen.WORKLOADS))
def test_committed_sweeps_name_a_shape_of_the_sweep(workload):
    """Every workload has a committed sweep whose fastest shape is one the
    probe runs, so the bench can time it again."""
    r = bench.stored_probe_best(workload)
    assert r is not None, workload
    assert (r["segments"], r["threads"], r["loads"]) in bench.PROBE_SHAPES


def test_write_default_trace_matches_kernels_by_shape(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(tmp_path / "profiles")
    trace = tmp_path / "trace"
    trace.mkdir()
    (trace / "default_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void lp::dev::row_kernel<7, 4, 2, true, false>(lp::dev::RowArgs)",133,1,3002000,50,'
        '2990000,3100000,0\n'
        '"void lp::dev::row_kernel<7, 16, 1, true, true>(lp::dev::RowArgs)",8000,1,22300,40,'
        '20000,40000,0\n'
        '"lp::dev::stream_read_kernel(float const*, unsigned int, float*)",800,1,10000,10,9000,'
        '11000,0\n'
        '"__amd_rocclr_fillBufferAligned",3,1,1000,0,900,1100,0\n', encoding="utf-8")
    line = {"config": {"levels": 3, "waves": 4, "depth": 2},
            "roofline": {"algorithmic_bytes_per_launch": 21053199888, "avg_launch_us": 3010.0,
                         "frac": 0.874},
            "decode": {"levels": 3, "waves": 16, "depth": 1,
                       "algorithmic_bytes_per_launch": 131354624, "ms_per_step": 0.0223,
                       "frac": 0.736}}
    log = tmp_path / "default.log"
    log.write_text("a line of rocprofv3 output\n" + json.dumps(line) + "\n", encoding="utf-8")
    bench.write_default_trace(str(trace), str(log))
    text = (tmp_path / "profiles" / "bench_default_trace.txt").read_text(encoding="utf-8")
    assert (f"workload prefill_echo_large: algorithmic_bytes_per_launch=21053199888  "
            f"GB/s at avg = {21053199888 / 3002000:.1f}") in text
    assert (f"workload decode_peaked: algorithmic_bytes_per_launch=131354624  "
            f"GB/s at avg = {131354624 / 22300:.1f}") in text
    assert "plain-read probe" in text
    assert "fillBuffer" not in text
    assert f"kernel_source_sha256: {bench.kernel_source_hash()}" in text


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["n_gpus"] == 2 and "one GPU" in d["error"]


def test_write_profile_scales_counters_by_the_copy_probe(tmp_path, monkeypatch):
    """Traffic = the row kernel's FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, averaged) each scaled by 256 MiB over what the same counter
    read for the 256 MiB device copy; the summaries carry the source hash,
    the plan's shape and the algorithmic bytes that stored_traffic checks."""
    import ragged_token_log_amd as R

    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(tmp_path / "profiles")
    wl = "ragged_echo_mix"
    kname = "void lp::dev::row_kernel<7, 8, 1, false, true>(lp::dev::RowArgs)"
    copy = "__amd_rocclr_copyBuffer"
    dirs = {}
    for d, (kvals, cval) in {"fetch": ((32000.0, 33000.0), 131072.0),
                             "write": ((40.0, 44.0), 262144.0)}.items():
        p = tmp_path / d
        p.mkdir()
        rows = [f'"{kname}","{d.upper()}_SIZE",{v}' for v in kvals] + [f'"{copy}","X",{cval}']
        (p / f"{d}_counter_collection.csv").write_text(
            '"Kernel_Name","Counter_Name","Counter_Value"\n' + "\n".join(rows) + "\n",
            encoding="utf-8")
        dirs[d] = str(p)
    t = tmp_path / "trace"
    t.mkdir()
    (t / "trace_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        f'"{kname}",200,1,15000,60,14000,17000,0\n', encoding="utf-8")
    bench.write_profile(wl, str(t), dirs["fetch"], dirs["write"])
    case = gen.WORKLOADS[wl]()
    info = R.Plan(case.offsets, case.echo, case.top_n, case.vocab, case.has_logits).info()
    alg = bench.algorithmic_bytes(info, case.vocab)
    want = 32500.0 * 1024 * (bench.COPY_PROBE_BYTES / (131072.0 * 1024)) + \
        42.0 * 1024 * (bench.COPY_PROBE_BYTES / (262144.0 * 1024))
    assert bench.stored_traffic(wl, info, alg) == pytest.approx(round(want), abs=1)
    text = (tmp_path / "profiles" / f"row_kernel_{wl}_trace.txt").read_text(encoding="utf-8")
    assert f"algorithmic GB/s at avg = {alg / 15000:.1f}" in text
