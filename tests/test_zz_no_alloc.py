"""lp_compute_ragged_noalloc (the library's fixed device workspace, no
allocation) against lp_compute_ragged on the same inputs, through the C ABI:
two calls in a row, the second on a smaller batch, then a third of another
shape; ids bit for bit, log-probabilities within 1e-5, and both against the
oracle.  Plans of up to 1984 output rows send their descriptors in the
arguments of up to 8 upload launches (248 each) and do not wait; larger ones
copy them synchronously: both sides of that limit, and the waiting, are
checked."""
import numpy as np
import pytest

import gen
from tests.gpu_helpers import assert_parity, log, oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_token_log_amd as lib
    lib.load()
    return lib


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _both(R, case, split=None, levels=3):
    """Runs the batch through lp_compute_ragged and lp_compute_ragged_noalloc
    (outputs of the latter pre-filled with NaN and 0xAAAAAAAA, so a row it
    does not write shows) and returns both host results and the oracle's."""
    logits = gen.host_logits(case)
    ntl = gen.next_token_rows(case, logits)
    dl = _dev(logits) if case.has_logits else None
    dn = _dev(ntl)
    plan = R.Plan(case.offsets, case.echo, case.top_n, case.vocab, case.has_logits, levels=levels)
    if split:
        plan.set_split(split)
    stream = torch.cuda.current_stream()
    lp1, ids1, ws = R.alloc_outputs(plan, dn.device, torch)
    plan.compute(dl, dn, case.tokens, case.sampled, lp1, ids1, ws, stream)
    lp2 = torch.full_like(lp1, float("nan"))
    ids2 = torch.full_like(ids1, 0xAAAAAAAA)
    plan.compute_noalloc(dl, dn, case.tokens, case.sampled, lp2, ids2, stream)
    torch.cuda.synchronize()
    ref = oracle(case.offsets, logits if case.has_logits else None, ntl, case.tokens,
                 case.sampled, case.top_n, case.echo, levels=levels)
    info = plan.info()
    plan.close()
    return (lp1.cpu().numpy(), ids1.cpu().numpy()), (lp2.cpu().numpy(), ids2.cpu().numpy()), \
        plan.out_off, ref, info


def _check(R, case, where, split=None, levels=3):
    (lp1, ids1), (lp2, ids2), off, ref, info = _both(R, case, split, levels)
    log(f"{where}: rows {info['out_rows']} split {info['split']} workspace {info['workspace_bytes']}")
    assert info["split"] == (split or info["split"])
    assert np.array_equal(ids2, ids1), where
    assert_parity(lp2, ids2, off, (lp1, ids1, off), f"{where}: noalloc vs compute")
    assert_parity(lp2, ids2, off, ref, f"{where}: noalloc vs oracle")


def test_noalloc_matches_compute_two_calls_then_a_third(R):
    # 1) 24 rows of 100003 split in 8 segments: descriptors and records in the scratch
    big = gen.decode_peaked(seed=41, batch=24, vocab=100003)
    _check(R, big, "first call (24 rows, split records)", split=8)
    # 2) a smaller batch right after: fewer descriptors, fewer records, other layout
    small = gen.ragged_echo_mix(seed=42, batch=3, lmin=2, lmax=9, vocab=5003)
    small.top_n[1] = 0          # a padding-only request among them
    _check(R, small, "second call (smaller echo batch)", split=3)
    # 3) another shape again, whole rows at levels 5
    mid = gen.ragged_echo_mix(seed=43, batch=5, lmin=4, lmax=40, vocab=30011)
    mid.top_n = np.minimum(mid.top_n * 4, 31).astype(np.int32)
    _check(R, mid, "third call (levels 5)", levels=5)


def test_noalloc_refuses_plans_beyond_its_workspace(R):
    n = 300_000                 # 16 B of descriptor per output row: 4.8 MB > 4 MiB
    off = np.array([0, n], np.uint32)
    plan = R.Plan(off, [1], [7], 32, True)
    lp = torch.empty((n, 8), dtype=torch.float32, device="cuda")
    ids = torch.empty((n, 8), dtype=torch.uint32, device="cuda")
    logits = torch.zeros((n, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(R.LogprobError) as e:
        plan.compute_noalloc(logits, logits[:1], np.zeros(n, np.uint32), [0], lp, ids)
    assert e.value.name == "LP_ERR_WORKSPACE"


def _next_token_case(rows, vocab, seed):
    """`rows` one-row requests over next-token logits only (no echo)."""
    c = gen.decode_peaked(seed=seed, batch=rows, vocab=vocab)
    c.top_n = np.random.default_rng(seed).integers(0, 8, rows).astype(np.int32)
    return c


@pytest.mark.parametrize("rows", [248, 249, 700, 1984, 1985])
def test_noalloc_upload_launch_counts(R, rows):
    """One launch of descriptors (248 rows), one more row (two launches),
    three with a short last one (700), the most sent in launch arguments
    (1984 = 8 x 248) and one past it (1985: the synchronous copy)."""
    _check(R, _next_token_case(rows, 3001, 60 + rows), f"{rows} rows")


def test_noalloc_waits_only_past_the_launch_argument_limit(R):
    """With about 12 ms of reads queued ahead on the stream, a call of 1984
    rows returns before they end (its descriptors travel in launch
    arguments); a call of 1985 rows copies them synchronously and returns
    only after the stream has drained.  Both results match lp_compute_ragged."""
    stream = torch.cuda.current_stream()
    x = torch.zeros(8192 * 131072, dtype=torch.float32, device="cuda")    # 4 GiB
    partial = torch.empty(8192, dtype=torch.float32, device="cuda")
    read = R.binding.stream_read_launcher(x, 8192, 131072, partial, stream)
    for rows, waits in ((1984, False), (1985, True)):
        case = _next_token_case(rows, 2003, 90 + rows)
        ntl = _dev(gen.next_token_rows(case, gen.host_logits(case)))
        plan = R.Plan(case.offsets, case.echo, case.top_n, case.vocab, False)
        lp1, ids1, ws = R.alloc_outputs(plan, ntl.device, torch)
        plan.compute(None, ntl, None, case.sampled, lp1, ids1, ws, stream)
        lp2 = torch.full_like(lp1, float("nan"))
        ids2 = torch.full_like(ids1, 0xAAAAAAAA)
        torch.cuda.synchronize()
        for _ in range(20):
            read()
        ahead = torch.cuda.Event()
        ahead.record(stream)
        plan.compute_noalloc(None, ntl, None, case.sampled, lp2, ids2, stream)
        drained = ahead.query()
        torch.cuda.synchronize()
        log(f"{rows} rows: the queued reads had ended when the call returned: {drained}")
        assert drained == waits, rows
        assert np.array_equal(ids2.cpu().numpy(), ids1.cpu().numpy()), rows
        assert_parity(lp2.cpu().numpy(), ids2.cpu().numpy(), plan.out_off,
                      (lp1.cpu().numpy(), ids1.cpu().numpy(), plan.out_off), f"{rows} rows")
        plan.close()


@pytest.mark.parametrize("i", range(100))
def test_noalloc_random_plans(R, i):
    """Seeded random plans (row widths from a few entries to past 128K,
    degenerate rows, heap depths 0-6, forced shapes and splits) through the
    no-allocation entry point, one after another on the same fixed
    workspace: against the oracle."""
    from tests.test_gpu_random import _draw_case

    c = _draw_case(4000 + i)
    echo = c["echo"] if c["has_logits"] else np.zeros_like(c["echo"])
    logits = c["logits"] if c["has_logits"] else None
    ref = oracle(c["off"], logits, c["ntl"], c["tokens"], c["sampled"], c["top_n"], echo,
                 levels=c["levels"])
    plan = R.Plan(c["off"], echo, c["top_n"], c["vocab"], c["has_logits"], levels=c["levels"])
    if c["split"]:
        plan.set_split(c["split"])
        plan.set_waves(c["waves"])
        plan.set_depth(c["depth"])
    plan.set_deterministic(c["deterministic"])
    dl = _dev(c["logits"]) if c["has_logits"] else None
    dn = _dev(c["ntl"])
    lp = torch.full((plan.out_rows, plan.columns), float("nan"), device="cuda")
    ids = torch.full((plan.out_rows, plan.columns), 0xAAAAAAAA, dtype=torch.uint32, device="cuda")
    plan.compute_noalloc(dl, dn, c["tokens"], c["sampled"], lp, ids)
    torch.cuda.synchronize()
    assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), plan.out_off, ref, f"noalloc random {i}")
    plan.close()
