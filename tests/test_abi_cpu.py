"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host planning agrees with the oracle.  No GPU call is made here."""
import os
import re
import subprocess

import numpy as np
import pytest

import gen
import oracle.logprob_oracle as LO
import ragged_token_log_amd as R
from ragged_token_log_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "liblogprob.h")


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lp_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    R.load()
    declared = _declared()
    assert declared, "no declarations parsed"
    assert sorted(binding.EXPORTED) == declared
    out = subprocess.run(["nm", "-D", "--defined-only", R.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lp_[a-z_0-9]+)\b", out))
    missing = [s for s in declared if s not in exported]
    assert not missing, missing


def test_status_strings():
    for code, name in binding.STATUS_NAMES.items():
        assert R.status_string(code) == name


def _random_batch(rng, batch, vocab, has_logits, p_echo=0.5):
    lengths = rng.integers(1, 9, size=batch)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    echo = (rng.random(batch) < p_echo) if has_logits else np.zeros(batch, bool)
    top_n = rng.integers(0, 8, size=batch)
    tokens = rng.integers(0, vocab, size=int(off[-1])).astype(np.uint32)
    sampled = rng.integers(0, vocab, size=batch).astype(np.uint32)
    return off, echo, top_n, tokens, sampled


@pytest.mark.parametrize("seed", range(20))
def test_plan_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    has_logits = bool(seed % 3)
    batch = int(rng.integers(1, 12))
    off, echo, top_n, tokens, sampled = _random_batch(rng, batch, 50, has_logits)
    plan = R.Plan(off, echo, top_n, 50, has_logits)
    counts, out_off = LO.output_counts_and_offsets(off, echo)
    assert plan.out_off.dtype == np.uint32 and np.array_equal(plan.out_off, out_off)
    assert plan.out_rows == int(out_off[-1])
    desc = plan.descriptors(tokens, sampled)
    tasks = LO.row_tasks(off, echo, top_n, tokens, sampled, has_logits)
    one = int(np.array([1.0], np.float32).view(np.uint32)[0])
    want = np.array([[t.src_row, t.chosen, t.top_n, one] for t in tasks], dtype=np.uint32)
    assert np.array_equal(desc, want)
    info = plan.info()
    assert info["read_rows"] == sum(int(c) for c, t in zip(counts, top_n) if t > 0)
    assert info["columns"] == 8 and info["levels"] == 3


@pytest.mark.parametrize("seed", range(24))
def test_direct_rows_flag(seed):
    """The plan marks a batch direct exactly when output row o reads logits
    row o for every o and no request has top_n == 0 (then the kernel takes
    the row from its own index instead of the descriptor)."""
    rng = np.random.default_rng(100 + seed)
    has_logits = seed % 4 != 0
    batch = int(rng.integers(1, 10))
    off, echo, top_n, tokens, sampled = _random_batch(rng, batch, 40, has_logits,
                                                      p_echo=(1.0, 0.5, 0.0)[seed % 3])
    if seed % 2:
        top_n = np.maximum(top_n, 1)
    plan = R.Plan(off, echo, top_n, 40, has_logits)
    tasks = LO.row_tasks(off, echo, top_n, tokens, sampled, has_logits)
    want = all(t.src_row == o and t.top_n > 0 for o, t in enumerate(tasks))
    assert plan.info()["direct_rows"] == int(want)


def test_direct_rows_on_named_workloads():
    expect = {"no_echo_next_token": 1, "ragged_echo_mix": 0, "decode_peaked": 1,
              "prefill_echo_large": 1, "tie_edge_stress": 1}
    for name, make in gen.WORKLOADS.items():
        c = make()
        plan = R.Plan(c.offsets, c.echo, c.top_n, c.vocab, c.has_logits)
        assert plan.info()["direct_rows"] == expect[name], name


@pytest.mark.parametrize("levels", range(0, 8))
def test_levels_columns_and_caps(levels):
    """[MAX] log_probabilities_ragged_graph: 2**levels columns (1 at levels
    0), top_n up to columns - 1; the library serves levels 0..6."""
    off = np.array([0, 2, 3], np.uint32)
    if levels > 6:
        _expect("LP_ERR_UNSUPPORTED", lambda: R.Plan(off, [1, 0], [0, 0], 100, True, levels=levels))
        return
    cols = LO.columns_for_levels(levels)
    cap = LO.max_top_n(levels)
    plan = R.Plan(off, [1, 0], [cap, 0], 100, True, levels=levels)
    assert plan.columns == cols and plan.info()["columns"] == cols
    _expect("LP_ERR_TOP_N_TOO_LARGE", lambda: R.Plan(off, [1, 0], [cap + 1, 0], 100, True,
                                                     levels=levels))
    # the split cap keeps a row's records within the merge wave's 1024 keys
    wide = R.Plan(np.array([0, 1], np.uint32), [0], [cap], 1 << 20, False, levels=levels)
    limit = 64 if cap == 0 else min(64, 1024 // cap)
    wide.set_split(limit)
    _expect("LP_ERR_UNSUPPORTED", lambda: wide.set_split(limit + 1))
    assert wide.workspace_bytes == 256 + limit * 8 * (cap + 2)
    assert wide.info()["record_words"] == cap + 2


def test_plan_on_named_workloads():
    for name, make in gen.WORKLOADS.items():
        c = make()
        plan = R.Plan(c.offsets, c.echo, c.top_n, c.vocab, c.has_logits)
        _, out_off = LO.output_counts_and_offsets(c.offsets, c.echo)
        assert np.array_equal(plan.out_off, out_off), name
        desc = plan.descriptors(c.tokens, c.sampled)
        tasks = LO.row_tasks(c.offsets, c.echo, c.top_n, c.tokens, c.sampled, c.has_logits)
        assert np.array_equal(desc[:, 0], [t.src_row for t in tasks]), name
        assert np.array_equal(desc[:, 1], [t.chosen for t in tasks]), name
        assert plan.info()["split"] >= 1


def test_split_and_workspace():
    plan = R.Plan([0, 1, 2], [0, 0], [7, 7], 128256, False)
    s = plan.split
    assert s > 1                      # two rows cannot fill the chip
    ws = plan.workspace_bytes
    assert ws == 256 + 2 * s * 72                  # records of 9 words at levels 3
    assert plan.info()["record_words"] == 9
    plan.set_split(1)
    assert plan.split == 1 and plan.workspace_bytes == 256
    with pytest.raises(R.LogprobError) as e:
        plan.set_split(65)
    assert e.value.name == "LP_ERR_UNSUPPORTED"
    plan.set_waves(8)
    assert plan.info()["waves"] == 8
    plan.set_waves(16)
    assert plan.info()["waves"] == 16
    plan.set_depth(1)
    assert plan.info()["depth"] == 1
    with pytest.raises(R.LogprobError):
        plan.set_depth(4)
    with pytest.raises(R.LogprobError) as e:
        plan.set_waves(6)
    assert e.value.name == "LP_ERR_UNSUPPORTED"
    big = R.Plan(np.arange(2001, dtype=np.uint32), np.ones(2000, bool), np.full(2000, 5), 32000,
                 True)
    assert big.split == 1


@pytest.mark.parametrize("vocab,waves,depth", [(8192, 4, 1), (18992, 4, 1), (20480, 4, 1),
                                               (20481, 8, 1), (32000, 8, 1), (65536, 8, 1), (65537, 16, 1),
                                               (128256, 16, 1), (131072, 16, 1), (131073, 4, 2),
                                               (151936, 4, 2)])
def test_many_rows_shape_by_row_length(vocab, waves, depth):
    """Plans of many rows pick the workgroup shape by row length."""
    plan = R.Plan(np.arange(1025, dtype=np.uint32), np.ones(1024, bool), np.full(1024, 5), vocab,
                  True)
    info = plan.info()
    assert (info["split"], info["waves"], info["depth"]) == (1, waves, depth)


@pytest.mark.parametrize("rows,vocab,shape", [
    (4, 32000, (1, 16, 1)), (32, 32000, (1, 16, 1)), (200, 32000, (1, 16, 1)),
    (32, 8192, (1, 8, 1)), (200, 16000, (1, 8, 1)), (32, 24000, (1, 8, 1)), (32, 24576, (1, 16, 1)),
    (32, 128256, (8, 8, 1)), (32, 151936, (8, 8, 1)), (64, 151936, (4, 16, 1)),
    (32, 256000, (8, 16, 1)), (8, 65536, (2, 16, 1)), (8, 65537, (4, 8, 1)),
    (40, 128256, (6, 8, 1)), (8, 1 << 20, (32, 16, 1)), (8, 256000, (8, 16, 1)), (4, 294912, (9, 16, 1)), (96, 256000, (2, 16, 1)), (111, 151936, (2, 16, 1)),
    (112, 151936, (2, 16, 1)), (127, 256000, (2, 16, 1)), (128, 128256, (2, 16, 1)),
    (129, 128256, (1, 16, 1)), (128, 32000, (1, 16, 1)), (256, 128256, (1, 16, 1)), (256, 32000, (1, 16, 1)),
    (257, 128256, (1, 8, 1)), (600, 151936, (1, 8, 1))])
def test_few_rows_shape(rows, vocab, shape):
    """Plans of at most 1023 read rows: (split, waves, depth) from the row
    count and the row length; long rows of small batches are cut into at
    most one workgroup per compute unit, over 8 waves at 7 slots when a
    segment holds fewer than 24576 entries, else 16."""
    plan = R.Plan(np.arange(rows + 1, dtype=np.uint32), np.zeros(rows, bool), np.full(rows, 7),
                  vocab, False)
    info = plan.info()
    assert (info["split"], info["waves"], info["depth"]) == shape
    assert rows * info["split"] <= 256 or info["split"] == 1


@pytest.mark.parametrize("levels,rows,vocab,shape", [
    (5, 2048, 32000, (1, 4, 2)), (6, 2048, 128256, (1, 4, 2)), (5, 1024, 256000, (1, 4, 2)),
    (5, 512, 128256, (1, 8, 2)), (5, 513, 128256, (1, 8, 1)), (6, 520, 32000, (1, 8, 1)),
    (6, 300, 128256, (1, 8, 2)), (6, 300, 16000, (1, 8, 1)),
    (6, 200, 16000, (1, 8, 1)), (5, 256, 128256, (1, 16, 1)), (6, 129, 32000, (1, 8, 2)),
    (6, 32, 256000, (4, 16, 1)), (6, 96, 151936, (2, 16, 1)), (6, 16, 151936, (4, 16, 1)),
    (5, 32, 256000, (4, 16, 1)), (5, 64, 151936, (4, 16, 1)), (5, 32, 128256, (4, 16, 1)),
    (5, 96, 70001, (2, 16, 1)), (5, 80, 128256, (3, 16, 1)), (5, 128, 256000, (2, 16, 1)),
    (5, 32, 65536, (1, 8, 2)), (6, 16, 32000, (1, 8, 2)), (6, 64, 32000, (1, 8, 2)),
    (6, 64, 24000, (1, 8, 2)), (6, 65, 32000, (1, 8, 2)), (5, 128, 32000, (1, 8, 2)),
    (6, 8, 1 << 29, (4, 16, 1)), (6, 200, 1 << 29, (2, 16, 1)),
    (4, 32, 151936, (8, 16, 1)), (4, 80, 128256, (3, 16, 1)),
    (4, 96, 128256, (2, 16, 1)), (4, 2048, 128256, (1, 16, 1)),
    (1, 520, 32000, (1, 4, 1)), (2, 800, 128256, (1, 4, 1)), (2, 511, 128256, (1, 8, 1)),
    (1, 300, 16000, (1, 8, 1)), (3, 520, 32000, (1, 8, 1))])
def test_shape_by_ranked_slots(levels, rows, vocab, shape):
    """With 31 or more ranked slots: 4 waves two deep for many rows, 8 one
    deep above one row per compute unit, rows of at most 65536 entries over 8
    waves two deep below, long rows over 16 waves one deep with up to 4
    segments a row at most 128 rows; 15 slots keep the segments of 7 over 16
    waves.  A row beyond the streamed range is always cut."""
    plan = R.Plan(np.arange(rows + 1, dtype=np.uint32), np.zeros(rows, bool),
                  np.full(rows, (1 << levels) - 1), vocab, False, levels=levels)
    info = plan.info()
    assert (info["split"], info["waves"], info["depth"]) == shape


@pytest.mark.parametrize("levels,rows,vocab,shape", [
    (6, 520, 32000, (1, 8, 2)), (5, 300, 151936, (1, 8, 2)), (5, 600, 16000, (1, 8, 1)),
    (6, 1024, 32000, (1, 4, 2)), (6, 200, 32000, (1, 8, 2)), (6, 200, 128256, (1, 16, 1))])
def test_shape_by_ranked_slots_rows_through_descriptors(levels, rows, vocab, shape):
    """Requests that read their last row only (no echo, full logits): above
    one row per compute unit the rows are found through their descriptors,
    the kernel holds no copy of its first chunk, and 8 waves go two deep."""
    off = np.arange(0, 2 * rows + 1, 2, dtype=np.uint32)
    plan = R.Plan(off, np.zeros(rows, bool), np.full(rows, (1 << levels) - 1), vocab, True,
                  levels=levels)
    info = plan.info()
    assert info["direct_rows"] == 0 and info["read_rows"] == rows
    assert (info["split"], info["waves"], info["depth"]) == shape


def test_segments_stay_within_the_streamed_range():
    # one workgroup streams at most 2^28 elements of a row: a wider row is
    # always cut into segments, and a split leaving longer segments is refused
    many = 3000
    wide = R.Plan(np.arange(many + 1, dtype=np.uint32), np.zeros(many, bool), np.full(many, 1),
                  (1 << 31) + 1, False)
    assert wide.split == 9
    assert wide.workspace_bytes == ((many * 16 + 255) // 256) * 256 + many * 9 * 72
    with pytest.raises(R.LogprobError) as e:
        wide.set_split(8)
    assert e.value.name == "LP_ERR_UNSUPPORTED"
    edge = R.Plan(np.arange(many + 1, dtype=np.uint32), np.zeros(many, bool), np.full(many, 1),
                  1 << 31, False)
    assert edge.split == 8
    edge.set_split(64)
    assert edge.split == 64


def _expect(name, fn):
    with pytest.raises(R.LogprobError) as e:
        fn()
    assert e.value.name == name, e.value.name


def test_error_codes_match_oracle_readings():
    off = [0, 2, 3]
    _expect("LP_ERR_TOP_N_NEGATIVE", lambda: R.Plan(off, [1, 0], [-1, 1], 5, True))
    _expect("LP_ERR_TOP_N_TOO_LARGE", lambda: R.Plan(off, [1, 0], [8, 1], 5, True))
    _expect("LP_ERR_ECHO_NEEDS_LOGITS", lambda: R.Plan(off, [1, 0], [1, 1], 5, False))
    _expect("LP_ERR_OFFSETS", lambda: R.Plan([0, 3, 3], [1, 0], [1, 1], 5, True))
    _expect("LP_ERR_OFFSETS", lambda: R.Plan([1, 2, 3], [1, 0], [1, 1], 5, True))
    _expect("LP_ERR_SHAPE", lambda: R.Plan(off, [1, 0], [1, 1], 5, True, logits_rows=4))
    _expect("LP_ERR_SHAPE", lambda: R.Plan(off, [0, 0], [1, 1], 5, False, logits_rows=3))
    _expect("LP_ERR_SHAPE", lambda: R.Plan(off, [1, 0], [1, 1], 0, True))
    _expect("LP_ERR_UNSUPPORTED", lambda: R.Plan(off, [1, 0], [1, 1], 5, True, levels=7))
    plan = R.Plan(off, [1, 0], [1, 7], 5, True)
    _expect("LP_ERR_TOKEN_RANGE", lambda: plan.descriptors([1, 2, 5], [4, 0]))
    _expect("LP_ERR_TOKEN_RANGE", lambda: plan.descriptors([1, 2, 3], [4, 5]))
    _expect("LP_ERR_NULL_ARG", lambda: plan.descriptors(None, [4, 0]))   # echo needs tokens
    # the oracle rejects the same calls with the same names
    ok = dict(input_row_offsets=np.array(off, np.uint32), logits=np.zeros((3, 5), np.float32),
              next_token_logits=np.zeros((2, 5), np.float32), tokens=np.array([1, 2, 3], np.uint32),
              sampled_tokens=np.array([4, 0], np.uint32), batch_top_n=[1, 7], batch_echo=[True, False])
    for code, kw in (("LP_ERR_TOP_N_NEGATIVE", {"batch_top_n": [-1, 1]}),
                     ("LP_ERR_TOP_N_TOO_LARGE", {"batch_top_n": [8, 1]}),
                     ("LP_ERR_ECHO_NEEDS_LOGITS", {"logits": None}),
                     ("LP_ERR_OFFSETS", {"input_row_offsets": np.array([0, 3, 3], np.uint32)}),
                     ("LP_ERR_TOKEN_RANGE", {"tokens": np.array([1, 2, 5], np.uint32)})):
        args = dict(ok, **kw)
        with pytest.raises(LO.OracleError) as e:
            LO.compute_log_probabilities_ragged(**args)
        assert e.value.code == code


def test_empty_batch():
    plan = R.Plan([0], [], [], 10, True)
    assert plan.out_rows == 0 and plan.out_off.tolist() == [0]
    assert plan.descriptors([], []).shape == (0, 4)


def test_no_echo_request_with_full_logits_needs_no_tokens():
    plan = R.Plan([0, 4, 6], [0, 0], [3, 3], 9, True)
    d = plan.descriptors(None, [1, 2])
    assert d[:, :2].tolist() == [[3, 1], [5, 2]]


@pytest.mark.parametrize("seed", range(16))
def test_assembly_matches_oracle(seed):
    """lp_assemble_ragged (host code, no GPU) against the oracle's
    compute_top on random device-shaped outputs: shuffled columns, padding,
    ties, sampled tokens inside and outside the top columns."""
    rng = np.random.default_rng(200 + seed)
    levels = int(rng.integers(1, 7))
    cols = 2 ** levels
    batch = int(rng.integers(1, 8))
    vocab = int(rng.integers(cols, 4 * cols + 2))
    off, echo, top_n, tokens, sampled = _random_batch(rng, batch, vocab, True)
    top_n = rng.integers(0, cols, size=batch)
    plan = R.Plan(off, echo, top_n, vocab, True, levels=levels)
    R_rows = plan.out_rows
    ids = rng.integers(0, vocab + 3, size=(R_rows, cols)).astype(np.uint32)
    ids[rng.random((R_rows, cols)) < 0.2] = binding.PAD_ID
    ids[:, -1] = rng.integers(0, vocab, size=R_rows)
    take = rng.random(R_rows) < 0.5            # sampled token among the columns
    ids[take, -1] = ids[take, 0] % vocab
    lp = (rng.integers(-6, 1, size=(R_rows, cols)) / 2).astype(np.float32)
    toks, vals, counts = plan.assemble(lp, ids)
    want = LO.assemble(lp, ids, plan.out_off, top_n, vocab)
    for n in range(batch):
        rows = range(int(plan.out_off[n]), int(plan.out_off[n + 1]))
        if want[n] is None:
            assert all(counts[o] == 0 for o in rows)
            continue
        for k, o in enumerate(rows):
            got = list(zip(toks[o, :counts[o]].tolist(), vals[o, :counts[o]].tolist()))
            assert got == list(want[n][1][k].items()), (n, o, got, want[n][1][k])


def test_temperature_in_descriptors_and_errors():
    off = np.array([0, 2, 3], np.uint32)
    plan = R.Plan(off, [1, 0], [3, 2], 50, True)
    tokens = np.array([1, 2, 3], np.uint32)
    sampled = np.array([4, 5], np.uint32)
    plan.set_temperature([0.5, 2.0])
    desc = plan.descriptors(tokens, sampled)
    temp = desc[:, 3].view(np.float32)
    assert temp.tolist() == [0.5, 0.5, 2.0]          # rows of request 0, then request 1
    for bad in ([0.0, 1.0], [-1.0, 1.0], [np.inf, 1.0], [np.nan, 1.0], [1e-45, 1.0],
                [2.0 ** -127, 1.0], [1.0, 3.5e-39], [1.0, 2.0 ** 121], [3.0e38, 1.0]):
        _expect("LP_ERR_TEMPERATURE", lambda b=bad: plan.set_temperature(b))
    assert plan.descriptors(tokens, sampled)[:, 3].view(np.float32).tolist() == [0.5, 0.5, 2.0]
    # both ends of the accepted range [2^-126, 2^120]
    plan.set_temperature([2.0 ** -126, 2.0 ** 120])
    temp = plan.descriptors(tokens, sampled)[:, 3].view(np.float32).tolist()
    assert temp == [2.0 ** -126, 2.0 ** -126, 2.0 ** 120]
    plan.set_temperature(None)
    assert plan.descriptors(tokens, sampled)[:, 3].view(np.float32).tolist() == [1.0] * 3


def test_top_k_in_descriptors_and_errors():
    """The top-k front end rides in the high half of the descriptor's third
    word (rows of top_n 0 keep a zero word); values beyond the ranked slots
    are refused and leave the plan unchanged."""
    off = np.array([0, 2, 3, 4], np.uint32)
    plan = R.Plan(off, [1, 0, 0], [3, 2, 0], 50, True)
    tokens = np.arange(4, dtype=np.uint32)
    sampled = np.array([4, 5, 6], np.uint32)
    plan.set_top_k([5, 0, 7])
    desc = plan.descriptors(tokens, sampled)
    assert desc[:, 2].tolist() == [3 | 5 << 16, 3 | 5 << 16, 2, 0]
    for bad in ([8, 0, 0], [-1, 0, 0], [0, 0, 100]):
        _expect("LP_ERR_TOP_K", lambda b=bad: plan.set_top_k(b))
    assert plan.descriptors(tokens, sampled)[:, 2].tolist() == [3 | 5 << 16, 3 | 5 << 16, 2, 0]
    plan.set_top_k(2)
    assert plan.descriptors(tokens, sampled)[:, 2].tolist() == [3 | 2 << 16, 3 | 2 << 16, 2 | 2 << 16, 0]
    plan.set_top_k(None)
    assert plan.descriptors(tokens, sampled)[:, 2].tolist() == [3, 3, 2, 0]
    wide = R.Plan(off, [1, 0, 0], [3, 2, 0], 500, True, levels=6)
    wide.set_top_k([63, 1, 0])
    _expect("LP_ERR_TOP_K", lambda: wide.set_top_k([64, 0, 0]))


def test_plain_c_caller(tmp_path):
    """The header compiles as C11 and a C program linked against the library
    plans, inspects, assembles and reports errors with no GPU."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.dirname(R.binding.LIB_PATH)
    exe = tmp_path / "c_abi_check"
    build = subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-I",
                            os.path.join(root, "include"),
                            os.path.join(root, "tests", "native", "c_abi_check.c"),
                            "-L", lib_dir, "-llogprob", "-lm", f"-Wl,-rpath,{lib_dir}",
                            "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr


def test_out_of_range_integers_are_rejected_not_wrapped():
    # a cast to uint32 would turn 2^32 + 1 into 1 and -1 into 2^32 - 1
    _expect("LP_ERR_OFFSETS", lambda: R.Plan([0, (1 << 32) + 1], [1], [1], 5, True))
    _expect("LP_ERR_OFFSETS", lambda: R.Plan(np.array([-1, 1], np.int64), [1], [1], 5, True))
    _expect("LP_ERR_SHAPE", lambda: R.Plan([0.0, 1.5], [1], [1], 5, True))
    _expect("LP_ERR_TOP_N_TOO_LARGE", lambda: R.Plan([0, 1], [1], [(1 << 32) + 1], 5, True))
    _expect("LP_ERR_TOP_N_NEGATIVE", lambda: R.Plan([0, 1], [1], [-(1 << 32) + 1], 5, True))
    _expect("LP_ERR_SHAPE", lambda: R.Plan([0, 1], [1], [0.5], 5, True))
    plan = R.Plan([0, 2], [1], [1], 5, True)
    _expect("LP_ERR_TOKEN_RANGE", lambda: plan.descriptors([0, (1 << 32) + 1], [1]))
    _expect("LP_ERR_TOKEN_RANGE", lambda: plan.descriptors([0, 1], np.array([-4], np.int64)))
    # whole numbers in range still pass, whatever their dtype
    d = plan.descriptors(np.array([0, 3], np.int64), np.array([2.0]))
    assert d[:, :2].tolist() == [[0, 3], [1, 2]]


def test_token_arrays_must_match_the_batch():
    """The library reads input_row_offsets[-1] tokens and batch sampled
    tokens; a shorter, longer or 2-D array is refused before any call reads
    it (descriptors, staging and compute share the check)."""
    plan = R.Plan([0, 64], [1], [3], 2 ** 32 - 1, True)
    good = np.arange(64, dtype=np.uint32)
    assert plan.descriptors(good, [1]).shape == (64, 4)
    for bad in (np.array([0, 1, 2], np.uint32), np.arange(65, dtype=np.uint32),
                np.arange(64, dtype=np.uint32).reshape(8, 8)):
        _expect("LP_ERR_SHAPE", lambda b=bad: plan.descriptors(b, [1]))
        _expect("LP_ERR_SHAPE", lambda b=bad: plan.stage(b, [1], None))
        _expect("LP_ERR_SHAPE", lambda b=bad: plan.compute(None, None, b, [1], None, None, None))
    for bad in ([], [1, 2], np.array([[1]], np.uint32), 5):
        _expect("LP_ERR_SHAPE", lambda b=bad: plan.descriptors(good, b))


def test_noalloc_refuses_plans_beyond_its_workspace_before_any_hip_call():
    """The no-allocation entry point's workspace is 4 MiB: a plan asking for
    more is refused before any HIP call (so this runs without a GPU)."""
    n = 300_000
    plan = R.Plan(np.array([0, n], np.uint32), [1], [7], 32, True)
    assert plan.workspace_bytes > 4 << 20
    _expect("LP_ERR_WORKSPACE", lambda: plan.compute_noalloc(None, None, np.zeros(n, np.uint32),
                                                             [0], None, None))


def test_deterministic_flag_round_trips():
    plan = R.Plan([0, 3, 5], [1, 0], [3, 2], 100, True)
    assert plan.info()["deterministic"] == 0
    plan.set_deterministic(True)
    assert plan.info()["deterministic"] == 1
    plan.set_deterministic(False)
    assert plan.info()["deterministic"] == 0


def test_stream_read_shapes_are_checked_before_any_hip_call():
    """The plain-read probe refuses shapes it has no kernel for, a misaligned
    buffer and a null pointer before any HIP call (so this runs without a
    GPU); zero rows is a no-op."""
    lib = binding.load()
    names = {0: "LP_OK", 1: "LP_ERR_NULL_ARG", 8: "LP_ERR_UNSUPPORTED"}
    fake = 1 << 20                       # 16-byte aligned, never dereferenced

    def st(x, rows, row_len, segs, threads, loads, partial=fake):
        return names.get(lib.lp_bench_stream_read_shape(x, rows, row_len, segs, threads, loads,
                                                        partial, None), "other")

    assert binding.status_string(8) == "LP_ERR_UNSUPPORTED"
    assert st(fake, 0, 1024, 1, 512, 4) == "LP_OK"
    assert st(None, 4, 1024, 1, 512, 4) == "LP_ERR_NULL_ARG"
    assert st(fake, 4, 1024, 1, 512, 4, partial=None) == "LP_ERR_NULL_ARG"
    assert st(fake + 4, 4, 1024, 1, 512, 4) == "LP_ERR_UNSUPPORTED"   # misaligned
    assert st(fake, 4, 1022, 1, 512, 4) == "LP_ERR_UNSUPPORTED"       # row_len % 4
    for segs, threads, loads in ((0, 512, 4), (65, 512, 4), (1, 384, 4), (1, 2048, 4),
                                 (1, 512, 3), (1, 512, 16), (1, 512, 0)):
        assert st(fake, 4, 1024, segs, threads, loads) == "LP_ERR_UNSUPPORTED", (segs, threads,
                                                                                loads)
    assert st(fake, 1 << 26, 1024, 64, 512, 4) == "LP_ERR_UNSUPPORTED"  # rows * segs >= 2^31


def test_device_buffers_are_checked_before_any_hip_call():
    """The binding hands the kernels bare pointers, so it refuses host
    tensors, non-contiguous ones and ones of the wrong element type before
    any HIP call (LP_ERR_SHAPE); a missing buffer is left to the library."""
    import torch

    plan = R.Plan([0, 3, 5], [1, 0], [3, 2], 100, True)
    host_logits = torch.zeros(5, 100)
    _expect("LP_ERR_SHAPE", lambda: plan.launch(host_logits, None, None, None, None))
    _expect("LP_ERR_SHAPE", lambda: plan.launcher(host_logits, None, None, None, None))
    _expect("LP_ERR_SHAPE", lambda: plan.compute(host_logits, None, np.arange(5), [1, 2], None,
                                                 None, None))
    _expect("LP_ERR_SHAPE", lambda: plan.compute_noalloc(host_logits, None, np.arange(5), [1, 2],
                                                         None, None))
    with pytest.raises(binding.LogprobError):
        binding._check_device_tensor(torch.zeros(4, 4).t(), "x", (4,), 16)
    binding._check_device_tensor(None, "x", (4,), 16)   # missing: the library reports it
