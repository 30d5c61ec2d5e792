"""Seeded random plans against the oracle (needs an MI355X).

Each case draws a batch of requests (row counts, echo flags, top_n up to the
heap depth's cap), a row width from tiny to past 128K entries, rows of the
degenerate kinds the parity suite uses (ties, all -inf, +-0.0, a boosted
token), and, for some cases, a forced kernel shape (waves, depth, segments)
or the deterministic chunk order.  Ids and offsets must match the oracle bit
for bit and logprobs within 1e-5.  The draws cover the paths a fixed grid can
miss: large-K bulk merges with keys still pending at a wave's end, seeds over
two chunks, segments of a few elements, rows shorter than one chunk.  The
same draws also go through the options (temperatures, top-k front ends) and
through the vocabulary-shard path (records per shard, then the merge).
"""
import numpy as np
import pytest

import oracle.logprob_oracle as LO
from tests.gpu_helpers import (assert_close_rel, assert_parity, log, oracle, run_library,
                               run_sharded, shard_bounds, special_rows)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 1000


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_token_log_amd as lib
    lib.load()
    return lib


def _draw_case(i):
    rng = np.random.default_rng(9000 + i)
    levels = int(rng.integers(0, 7))
    cap = LO.max_top_n(levels)
    kind = i % 4
    if kind == 0:
        vocab = int(rng.integers(1, 300))
    elif kind == 1:
        vocab = int(rng.integers(900, 9000))
    elif kind == 2:
        vocab = int(rng.integers(20000, 70000))
    else:
        vocab = int(rng.choice([128256, 131073, 151936]))
    batch = int(rng.integers(1, 7))
    lengths = rng.integers(1, 6 if vocab < 100000 else 3, batch)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    echo = rng.random(batch) < 0.5
    top_n = rng.integers(0, cap + 1, batch) if cap > 0 else np.zeros(batch, int)
    if cap > 0 and rng.random() < 0.7:
        top_n[int(rng.integers(batch))] = cap
    logits = special_rows(rng, int(off[-1]), vocab)
    ntl = logits[off[1:].astype(np.int64) - 1]
    tokens = rng.integers(0, vocab, int(off[-1])).astype(np.uint32)
    sampled = rng.integers(0, vocab, batch).astype(np.uint32)
    split = waves = depth = None
    if rng.random() < 0.5:
        waves = int(rng.choice([4, 8, 16]))
        depth = int(rng.integers(1, 3))
        most = min(64, 1024 // max(cap, 1))
        split = int(rng.choice([s for s in (1, 2, 3, 4, 7) if s <= most]))
    deterministic = bool(rng.random() < 0.25)
    has_logits = bool(rng.random() < 0.6)
    return dict(levels=levels, vocab=vocab, off=off, echo=echo, top_n=top_n, logits=logits,
                ntl=ntl, tokens=tokens, sampled=sampled, split=split, waves=waves, depth=depth,
                deterministic=deterministic, has_logits=has_logits)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_plan(R, i):
    c = _draw_case(i)
    echo = c["echo"] if c["has_logits"] else np.zeros_like(c["echo"])
    log(f"random case {i}: levels={c['levels']} vocab={c['vocab']} rows={int(c['off'][-1])} "
        f"logits={c['has_logits']} shape={(c['waves'], c['depth'], c['split'])} "
        f"deterministic={c['deterministic']}")
    logits = c["logits"] if c["has_logits"] else None
    ref = oracle(c["off"], logits, c["ntl"], c["tokens"], c["sampled"], c["top_n"], echo,
                 levels=c["levels"])
    dl = torch.from_numpy(c["logits"]).cuda() if c["has_logits"] else None
    dn = torch.from_numpy(np.ascontiguousarray(c["ntl"])).cuda()
    got = run_library(R, torch, c["off"], dl, dn, c["tokens"], c["sampled"], c["top_n"], echo,
                      c["split"], c["waves"], c["depth"], levels=c["levels"],
                      deterministic=c["deterministic"])
    assert_parity(*got, ref, f"random case {i}")


N_OPTION_CASES = 400


@pytest.mark.parametrize("i", range(N_OPTION_CASES))
def test_random_plan_with_options(R, i):
    """The same draws with per-request temperatures (some 1, some far from
    it) and top-k front ends (0 = off, up to the heap cap), through the torch
    front end: ids and offsets bit for bit, logprobs within 1e-5 (plus one
    ulp where |lp| >= 128, as the temperature tests allow)."""
    c = _draw_case(1000 + i)
    rng = np.random.default_rng(5000 + i)
    batch = len(c["top_n"])
    cap = LO.max_top_n(c["levels"])
    temps = rng.choice(np.array([1.0, 0.25, 0.7, 1.0, 1.9, 6.0], np.float32), batch)
    top_k = rng.integers(0, cap + 1, batch) if cap > 0 else np.zeros(batch, int)
    top_k[rng.random(batch) < 0.4] = 0
    echo = c["echo"] if c["has_logits"] else np.zeros_like(c["echo"])
    log(f"random option case {i}: levels={c['levels']} vocab={c['vocab']} rows={int(c['off'][-1])} "
        f"shape={(c['waves'], c['depth'], c['split'])} temps={temps.tolist()} top_k={top_k.tolist()}")
    logits = c["logits"] if c["has_logits"] else None
    ref = LO.compute_log_probabilities_ragged(c["off"], logits, c["ntl"], c["tokens"], c["sampled"],
                                              list(c["top_n"]), list(echo), levels=c["levels"],
                                              batch_temperature=temps, batch_top_k=top_k)
    dl = torch.from_numpy(c["logits"]).cuda() if c["has_logits"] else None
    dn = torch.from_numpy(np.ascontiguousarray(c["ntl"])).cuda()
    lp, ids, out_off = R.compute_log_probabilities_ragged(
        c["off"], dl, dn, c["tokens"], c["sampled"], c["top_n"], echo, split=c["split"],
        waves=c["waves"], depth=c["depth"], levels=c["levels"], temperature=temps, top_k=top_k,
        deterministic=c["deterministic"])
    torch.cuda.synchronize()
    assert np.array_equal(out_off, ref[2]), f"option case {i}: offsets"
    assert np.array_equal(ids.cpu().numpy(), ref[1]), f"option case {i}: ids"
    assert_close_rel(lp.cpu().numpy(), ref[0], f"option case {i}")


N_SHARD_CASES = 200


@pytest.mark.parametrize("i", range(N_SHARD_CASES))
def test_random_plan_through_vocab_shards(R, i):
    """The same draws through the vocabulary-shard path: 1 to 16 uneven
    shards (as many as the merge takes at the draw's heap depth), records
    per shard, then the merge, some with a top-k front end: ids and offsets
    bit for bit, logprobs within 1e-5 (plus one ulp where |lp| >= 128)."""
    c = _draw_case(2000 + i)
    rng = np.random.default_rng(7000 + i)
    echo = c["echo"] if c["has_logits"] else np.zeros_like(c["echo"])
    logits = c["logits"] if c["has_logits"] else None
    cap = LO.max_top_n(c["levels"])
    most = min(64, 1024 // max(cap, 1), c["vocab"])
    n = int(rng.integers(1, min(most, 16) + 1))
    bounds = shard_bounds(c["vocab"], n, rng) if n > 1 else [(0, c["vocab"])]
    top_k = rng.integers(0, cap + 1, len(c["top_n"])) if cap > 0 and rng.random() < 0.4 else None
    log(f"random shard case {i}: levels={c['levels']} vocab={c['vocab']} rows={int(c['off'][-1])} "
        f"shards={len(bounds)} top_k={top_k is not None}")
    ref = LO.compute_log_probabilities_ragged(c["off"], logits, c["ntl"], c["tokens"], c["sampled"],
                                              list(c["top_n"]), list(echo), levels=c["levels"],
                                              batch_top_k=top_k)
    got = run_sharded(R, torch, c["off"], logits, c["ntl"], c["tokens"], c["sampled"], c["top_n"],
                      echo, c["levels"], bounds, top_k)
    assert np.array_equal(got[2], ref[2]), f"shard case {i}: offsets"
    assert np.array_equal(got[1], ref[1]), f"shard case {i}: ids"
    assert_close_rel(got[0], ref[0], f"shard case {i}")


N_STAGED_CASES = 100


@pytest.mark.parametrize("i", range(N_STAGED_CASES))
def test_random_plan_staged_then_launched(R, i):
    """The same draws through lp_stage_ragged (descriptors uploaded into the
    workspace) and lp_launch_ragged, the path a caller takes to keep
    descriptors resident or to capture the launch: against the oracle."""
    c = _draw_case(3000 + i)
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
    dl = torch.from_numpy(c["logits"]).cuda() if c["has_logits"] else None
    dn = torch.from_numpy(np.ascontiguousarray(c["ntl"])).cuda()
    lp, ids, ws = R.alloc_outputs(plan, dn.device, torch)
    plan.stage(c["tokens"], c["sampled"], ws)
    plan.launch(dl, dn, lp, ids, ws)
    torch.cuda.synchronize()
    assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), plan.out_off, ref, f"staged case {i}")
    plan.close()


N_BATCH_CASES = 20


@pytest.mark.parametrize("i", range(N_BATCH_CASES))
def test_random_serving_batch(R, i):
    """Serving-sized batches: 16-200 requests of 1-64 rows, vocabularies of
    7919 to 151936, echo on about half the requests (or next-token logits
    only), top_n and heap depth drawn, per-request temperatures and top-k
    front ends on some; the device draws the logits.  Offsets bit for bit
    and 64 sampled rows (plus the first and last) against the oracle."""
    from tests.gpu_helpers import DeviceRows

    rng = np.random.default_rng(600000 + i)
    B = int(rng.integers(16, 201))
    V = int(rng.choice([32000, 50257, 128256, 151936, 7919]))
    levels = int(rng.integers(1, 7))
    cap = LO.max_top_n(levels)
    lengths = rng.integers(1, 65, B)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    T = int(off[-1])
    has_logits = bool(rng.random() < 0.8)
    echo = (rng.random(B) < 0.5) if has_logits else np.zeros(B, bool)
    top_n = rng.integers(0, cap + 1, B)
    temps = rng.choice(np.array([1.0, 0.5, 0.8, 1.5, 3.0], np.float32), B) \
        if rng.random() < 0.3 else None
    top_k = rng.integers(0, cap + 1, B) if rng.random() < 0.3 else None
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(600000 + i)
    logits = torch.randn((T if has_logits else B, V), generator=g, device=dev) * 2.0
    ntl = logits.index_select(0, torch.from_numpy(off[1:].astype(np.int64) - 1).to(dev)) \
        if has_logits else logits
    tokens = rng.integers(0, V, T).astype(np.uint32)
    sampled = rng.integers(0, V, B).astype(np.uint32)
    log(f"serving batch {i}: B={B} V={V} levels={levels} rows={T} logits={has_logits} "
        f"temps={temps is not None} top_k={top_k is not None}")
    lp, ids, out_off = R.compute_log_probabilities_ragged(
        off, logits if has_logits else None, ntl, tokens, sampled, top_n, echo, levels=levels,
        temperature=temps, top_k=top_k)
    torch.cuda.synchronize()
    nrows = lp.shape[0]
    rows = sorted(set(rng.choice(nrows, size=min(64, nrows), replace=False).tolist())
                  | {0, nrows - 1})
    ref = LO.compute_log_probabilities_ragged(
        off, DeviceRows(logits) if has_logits else None, DeviceRows(ntl), tokens, sampled,
        list(top_n), list(echo), levels=levels, rows=rows, batch_temperature=temps,
        batch_top_k=top_k)
    assert np.array_equal(out_off, ref[2]), f"serving batch {i}: offsets"
    assert np.array_equal(ids.cpu().numpy()[rows], ref[1][rows]), f"serving batch {i}: ids"
    assert_close_rel(lp.cpu().numpy()[rows], ref[0][rows], f"serving batch {i}")
