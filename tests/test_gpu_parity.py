"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

Ids and output offsets must match bit for bit; logprobs within 1e-5 absolute
(NaN and infinities exactly).  Small cases compare every element; the full
prefill and tie-stress workloads compare sampled rows with the oracle and
check every row through properties that hold at any size.
"""
import numpy as np
import pytest

import gen
import oracle.logprob_oracle as LO
from tests.gpu_helpers import (DeviceRows, assert_close_rel, assert_lp_close, assert_parity,
                               check_all_rows_properties,
                               log, oracle, run_library, run_sharded, shard_bounds)
from tests.gpu_helpers import special_rows as _special_rows

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


def _edge_batch(seed, vocab):
    rng = np.random.default_rng(seed)
    lengths = np.array([1, 3, 1, 5, 2, 7, 1, 4])
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    echo = np.array([1, 1, 0, 1, 0, 1, 1, 0], bool)
    top_n = np.array([7, 0, 5, 1, 7, 3, 2, 6])
    logits = _special_rows(rng, int(off[-1]), vocab)
    ntl = logits[off[1:].astype(np.int64) - 1]
    tokens = rng.integers(0, vocab, int(off[-1])).astype(np.uint32)
    sampled = rng.integers(0, vocab, len(lengths)).astype(np.uint32)
    return off, logits, ntl, tokens, sampled, top_n, echo


@pytest.mark.parametrize("vocab", [1, 2, 3, 7, 8, 9, 111, 1000, 1027, 4099, 8193, 20011, 70001])
@pytest.mark.parametrize("split,waves,depth", [(None, None, None), (1, 4, 2), (2, 8, 1), (5, 4, 1),
                                               (64, 8, 2), (1, 16, 1), (3, 16, 2), (1, 8, 1)])
def test_edge_cases(R, vocab, split, waves, depth):
    log(f"edge cases vocab={vocab} split={split} waves={waves} depth={depth}")
    off, logits, ntl, tokens, sampled, top_n, echo = _edge_batch(vocab * 7 + 1, vocab)
    ref = oracle(off, logits, ntl, tokens, sampled, top_n, echo)
    got = run_library(R, torch, off, _dev(logits), _dev(ntl), tokens, sampled, top_n, echo, split,
                      waves, depth)
    assert_parity(*got, ref, f"edge vocab={vocab} split={split} waves={waves}")


def test_adversarial_orders(R):
    """Rows sorted ascending (every chunk beats the running threshold),
    descending, and a sawtooth: the candidate buffer must compress often."""
    vocab = 50000
    base = np.linspace(-5, 5, vocab, dtype=np.float32)
    rows = np.stack([base, base[::-1].copy(), np.tile(base[:1000], vocab // 1000),
                     np.round(base * 2) / 2])
    off = np.arange(5, dtype=np.uint32)
    for split, waves, depth in ((1, 4, 2), (1, 8, 1), (3, 4, 1), (1, 16, 2), (2, 16, 1), (1, 4, 1)):
        ref = oracle(off, rows, rows, np.zeros(4, np.uint32), np.array([0, 1, 2, 3], np.uint32),
                     np.full(4, 7), np.ones(4, bool))
        got = run_library(R, torch, off, _dev(rows), _dev(rows), np.zeros(4, np.uint32),
                          np.array([0, 1, 2, 3], np.uint32), np.full(4, 7), np.ones(4, bool),
                          split, waves, depth)
        assert_parity(*got, ref, f"adversarial split={split} waves={waves} depth={depth}")


@pytest.mark.parametrize("split", [None, 1, 3])
def test_no_echo_next_token_path(R, split):
    c = gen.no_echo_next_token()
    ntl = gen.host_logits(c)
    log(f"no_echo_next_token split={split}")
    ref = oracle(c.offsets, None, ntl, c.tokens, c.sampled, c.top_n, c.echo)
    got = run_library(R, torch, c.offsets, None, _dev(ntl), c.tokens, c.sampled, c.top_n, c.echo,
                      split)
    assert_parity(*got, ref, "no_echo_next_token")


@pytest.mark.parametrize("split", [None, 2])
def test_ragged_echo_mix(R, split):
    c = gen.ragged_echo_mix()
    logits = gen.host_logits(c)
    ntl = gen.next_token_rows(c, logits)
    log(f"ragged_echo_mix rows={c.total_tokens} split={split}")
    ref = oracle(c.offsets, logits, ntl, c.tokens, c.sampled, c.top_n, c.echo)
    got = run_library(R, torch, c.offsets, _dev(logits), _dev(ntl), c.tokens, c.sampled, c.top_n,
                      c.echo, split)
    assert_parity(*got, ref, "ragged_echo_mix")


@pytest.mark.parametrize("split,waves,depth", [(None, None, None), (1, 4, 2), (16, 8, 1), (1, 16, 1),
                                               (1, 8, 2)])
def test_decode_peaked(R, split, waves, depth):
    c = gen.decode_peaked()
    ntl = gen.host_logits(c)
    log(f"decode_peaked split={split} waves={waves} depth={depth}")
    ref = oracle(c.offsets, None, ntl, c.tokens, c.sampled, c.top_n, c.echo)
    got = run_library(R, torch, c.offsets, None, _dev(ntl), c.tokens, c.sampled, c.top_n, c.echo,
                      split, waves, depth)
    assert_parity(*got, ref, "decode_peaked")
    # the chosen slot holds the sampled (boosted) token in every row
    assert np.array_equal(got[1][:, 7], c.sampled)


def _levels_batch(seed, vocab, levels, rows_per_req=(1, 4, 1, 6, 2, 3)):
    rng = np.random.default_rng(seed)
    lengths = np.array(rows_per_req)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    cap = LO.max_top_n(levels)
    echo = np.array([1, 1, 0, 1, 0, 1], bool)[: len(lengths)]
    top_n = rng.integers(0, cap + 1, len(lengths)) if cap > 0 else np.zeros(len(lengths), int)
    if cap > 0:
        top_n[0] = cap
        top_n[-1] = 0
    logits = _special_rows(rng, int(off[-1]), vocab)
    ntl = logits[off[1:].astype(np.int64) - 1]
    tokens = rng.integers(0, vocab, int(off[-1])).astype(np.uint32)
    sampled = rng.integers(0, vocab, len(lengths)).astype(np.uint32)
    return off, logits, ntl, tokens, sampled, top_n, echo


@pytest.mark.parametrize("levels", [0, 1, 2, 4, 5, 6])
@pytest.mark.parametrize("vocab", [3, 77, 1027, 40001])
@pytest.mark.parametrize("split,waves,depth", [(None, None, None), (1, 4, 1), (3, 8, 2), (1, 16, 2),
                                               (16, 4, 2), (1, 16, 1), (2, 16, 1)])
def test_levels(R, levels, vocab, split, waves, depth):
    """[MAX] log_probabilities_ragged_graph: 2**levels columns, top_n up to
    2**levels - 1, every heap depth the library serves."""
    log(f"levels={levels} vocab={vocab} split={split} waves={waves} depth={depth}")
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(levels * 100 + vocab, vocab, levels)
    ref = oracle(off, logits, ntl, tokens, sampled, top_n, echo, levels=levels)
    got = run_library(R, torch, off, _dev(logits), _dev(ntl), tokens, sampled, top_n, echo, split,
                      waves, depth, levels=levels)
    assert got[0].shape[1] == LO.columns_for_levels(levels)
    assert_parity(*got, ref, f"levels={levels} vocab={vocab} split={split}")


@pytest.mark.parametrize("vocab", [1, 2, 5, 62, 63, 64, 65])
def test_levels6_small_vocab(R, vocab):
    """63 ranked slots over vocabularies around and below 63 (the rest pads)."""
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(vocab + 900, vocab, 6)
    top_n = np.where(top_n > 0, 63, 0)
    ref = oracle(off, logits, ntl, tokens, sampled, top_n, echo, levels=6)
    for split in (None, 2, 16):
        got = run_library(R, torch, off, _dev(logits), _dev(ntl), tokens, sampled, top_n, echo, split,
                          levels=6)
        assert_parity(*got, ref, f"levels 6 vocab={vocab} split={split}")


@pytest.mark.parametrize("levels", [1, 5, 6])
def test_levels_direct_rows(R, levels):
    """Next-token rows (the direct-row kernels) at other heap depths, with the
    split path at its largest split for the depth."""
    c = gen.decode_peaked(seed=30 + levels, batch=24, vocab=70001)
    ntl = gen.host_logits(c)
    cap = LO.max_top_n(levels)
    top_n = np.full(c.batch, cap)
    ref = oracle(c.offsets, None, ntl, c.tokens, c.sampled, top_n, c.echo, levels=levels)
    for split in (None, 1, min(64, 1024 // cap)):
        log(f"direct rows levels={levels} split={split}")
        got = run_library(R, torch, c.offsets, None, _dev(ntl), c.tokens, c.sampled, top_n, c.echo,
                          split, levels=levels)
        assert_parity(*got, ref, f"direct levels={levels} split={split}")


@pytest.mark.parametrize("levels", [3, 5])
@pytest.mark.parametrize("vocab", [1027, 40001])
@pytest.mark.parametrize("split", [None, 3, 16])
def test_temperature(R, levels, vocab, split):
    """log_softmax(x / T) per request (the temperature of the FlashInfer
    page's Temperature processor), ranking on the raw logits."""
    log(f"temperature levels={levels} vocab={vocab} split={split}")
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(3 * vocab + levels, vocab, levels)
    temps = np.array([0.25, 0.7, 1.0, 1.9, 5.0, 0.4], np.float32)[: len(top_n)]
    ref = LO.compute_log_probabilities_ragged(off, logits, ntl, tokens, sampled, list(top_n),
                                              list(echo), levels=levels, batch_temperature=temps)
    lp, ids, out_off = R.compute_log_probabilities_ragged(
        off, _dev(logits), _dev(ntl), tokens, sampled, top_n, echo, split=split, levels=levels,
        temperature=temps)
    torch.cuda.synchronize()
    assert np.array_equal(out_off, ref[2])
    assert np.array_equal(ids.cpu().numpy(), ref[1]), "ids"
    assert_close_rel(lp.cpu().numpy(), ref[0], f"temperature levels={levels} split={split}")


@pytest.mark.parametrize("levels", [1, 3, 5, 6])
@pytest.mark.parametrize("vocab", [5, 1027, 40001])
@pytest.mark.parametrize("split", [None, 3])
def test_top_k_front_end(R, levels, vocab, split):
    """The FlashInfer page's TopK on logits then Softmax, per request, with
    temperatures: kept set, renormalised log-probabilities, dropped chosen
    tokens at -inf."""
    log(f"top-k front end levels={levels} vocab={vocab} split={split}")
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(5 * vocab + levels, vocab, levels)
    cap = LO.max_top_n(levels)
    rng = np.random.default_rng(vocab + 17 * levels)
    top_k = rng.integers(0, cap + 1, len(top_n))
    top_k[0], top_k[1] = 1, cap
    temps = np.array([0.5, 1.0, 2.0, 0.8, 1.3, 3.0], np.float32)[: len(top_n)]
    ref = LO.compute_log_probabilities_ragged(off, logits, ntl, tokens, sampled, list(top_n),
                                              list(echo), levels=levels, batch_temperature=temps,
                                              batch_top_k=top_k)
    lp, ids, out_off = R.compute_log_probabilities_ragged(
        off, _dev(logits), _dev(ntl), tokens, sampled, top_n, echo, split=split, levels=levels,
        temperature=temps, top_k=top_k)
    torch.cuda.synchronize()
    assert np.array_equal(out_off, ref[2])
    assert np.array_equal(ids.cpu().numpy(), ref[1]), "ids"
    assert_close_rel(lp.cpu().numpy(), ref[0], f"top-k levels={levels} split={split}")


@pytest.mark.parametrize("top_k", [1, 3, 7])
def test_top_k_decode_shape(R, top_k):
    """Decode rows (direct rows): the sampled token is the boosted id, kept
    (finite renormalised log-probability) in the rows where it ranks within
    k and -inf elsewhere, as the oracle says row by row."""
    c = gen.decode_peaked()
    ntl = gen.host_logits(c)
    ref = LO.compute_log_probabilities_ragged(c.offsets, None, ntl, c.tokens, c.sampled,
                                              list(c.top_n), list(c.echo),
                                              batch_top_k=[top_k] * c.batch)
    lp, ids, _ = R.compute_log_probabilities_ragged(c.offsets, None, _dev(ntl), c.tokens, c.sampled,
                                                    c.top_n, c.echo, top_k=top_k)
    torch.cuda.synchronize()
    got_lp = lp.cpu().numpy()
    assert np.array_equal(ids.cpu().numpy(), ref[1])
    assert np.isfinite(ref[0][:, 7]).any()        # some rows keep their sampled token
    assert_lp_close(got_lp, ref[0], f"decode top_k={top_k}")


def test_temperature_decode_shape(R):
    """The decode workload (direct rows) at T = 0.6 and T = 1.5."""
    c = gen.decode_peaked()
    ntl = gen.host_logits(c)
    for T in (0.6, 1.5):
        log(f"decode_peaked temperature={T}")
        ref = LO.compute_log_probabilities_ragged(c.offsets, None, ntl, c.tokens, c.sampled,
                                                  list(c.top_n), list(c.echo),
                                                  batch_temperature=[T] * c.batch)
        lp, ids, _ = R.compute_log_probabilities_ragged(c.offsets, None, _dev(ntl), c.tokens,
                                                        c.sampled, c.top_n, c.echo, temperature=T)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ref[1])
        assert_close_rel(lp.cpu().numpy(), ref[0], f"decode T={T}")


def _run_sharded(R, off, logits, ntl, tokens, sampled, top_n, echo, levels, bounds, top_k=None):
    return run_sharded(R, torch, off, logits, ntl, tokens, sampled, top_n, echo, levels, bounds,
                       top_k)


@pytest.mark.parametrize("levels", [1, 3, 5])
@pytest.mark.parametrize("n_shards", [1, 2, 3, 8])
def test_vocab_shards(R, levels, n_shards):
    """Vocabulary-sharded logits: per-shard records (global ids), gathered
    and merged, give the unsharded results."""
    vocab = 40001
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(11 * n_shards + levels, vocab,
                                                                   levels)
    bounds = shard_bounds(vocab, n_shards, np.random.default_rng(n_shards))
    log(f"vocab shards levels={levels} shards={bounds}")
    ref = oracle(off, logits, ntl, tokens, sampled, top_n, echo, levels=levels)
    got = _run_sharded(R, off, logits, ntl, tokens, sampled, top_n, echo, levels, bounds)
    assert_parity(*got, ref, f"shards levels={levels} n={n_shards}")
    whole = run_library(R, torch, off, _dev(logits), _dev(ntl), tokens, sampled, top_n, echo,
                        levels=levels)
    assert np.array_equal(got[1], whole[1])


@pytest.mark.parametrize("vocab,n_shards,levels", [(7, 3, 3), (64, 64, 1), (130, 16, 6), (5, 5, 2),
                                                   (1027, 64, 4)])
def test_vocab_shards_edges(R, vocab, n_shards, levels):
    """Shards narrower than one 16-byte load, one shard per id, 64 shards,
    the deepest heap with fewer ids than slots."""
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(vocab + n_shards, vocab, levels)
    bounds = shard_bounds(vocab, n_shards, np.random.default_rng(vocab))
    log(f"shard edges vocab={vocab} shards={n_shards} levels={levels}")
    ref = oracle(off, logits, ntl, tokens, sampled, top_n, echo, levels=levels)
    got = _run_sharded(R, off, logits, ntl, tokens, sampled, top_n, echo, levels, bounds)
    assert_parity(*got, ref, f"shard edges vocab={vocab} n={n_shards}")


@pytest.mark.parametrize("levels", [3, 5])
def test_vocab_shards_top_k(R, levels):
    """The top-k front end applied after the shard merge."""
    vocab = 20011
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(41 + levels, vocab, levels)
    cap = LO.max_top_n(levels)
    top_k = np.array([1, cap, 2, 0, cap // 2, 3])[: len(top_n)]
    bounds = shard_bounds(vocab, 4, np.random.default_rng(levels))
    ref = LO.compute_log_probabilities_ragged(off, logits, ntl, tokens, sampled, list(top_n),
                                              list(echo), levels=levels, batch_top_k=top_k)
    got = _run_sharded(R, off, logits, ntl, tokens, sampled, top_n, echo, levels, bounds, top_k)
    assert_parity(*got, ref, f"shards top_k levels={levels}")


def test_vocab_shards_padding_only(R):
    """Every top_n 0: the merge pads every row without reading records."""
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(5, 300, 3)
    top_n = np.zeros_like(top_n)
    ref = oracle(off, logits, ntl, tokens, sampled, top_n, echo)
    got = _run_sharded(R, off, logits, ntl, tokens, sampled, top_n, echo, 3, [(0, 100), (100, 300)])
    assert_parity(*got, ref, "shards, padding only")


def test_vocab_shards_decode_tp8(R):
    """The decode workload's next-token rows cut into 8 equal vocabulary
    shards, the shape of an 8-way tensor-parallel LM head."""
    c = gen.decode_peaked()
    ntl = gen.host_logits(c)
    w = c.vocab // 8
    bounds = [(k * w, (k + 1) * w if k < 7 else c.vocab) for k in range(8)]
    ref = oracle(c.offsets, None, ntl, c.tokens, c.sampled, c.top_n, c.echo)
    got = _run_sharded(R, c.offsets, None, ntl, c.tokens, c.sampled, c.top_n, c.echo, 3, bounds)
    assert_parity(*got, ref, "decode tp8 shards")


def _same_value(a, b):
    return (np.isnan(a) and np.isnan(b)) or a == b or abs(a - b) <= 1e-5


@pytest.mark.parametrize("levels", [1, 3, 5])
@pytest.mark.parametrize("vocab", [5, 1027, 32000])
@pytest.mark.parametrize("with_top_k", [False, True])
def test_log_probabilities_objects(R, levels, vocab, with_top_k):
    """The whole call: device path, copy back and host assembly
    (lp_assemble_ragged) against the oracle's rows and its compute_top."""
    log(f"log_probabilities_ragged levels={levels} vocab={vocab} top_k={with_top_k}")
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(7 * levels + vocab, vocab, levels)
    top_k = None
    if with_top_k:
        top_k = np.minimum(np.array([2, 1, 3, 5, 1, 4])[: len(top_n)], LO.max_top_n(levels))
    got = R.log_probabilities_ragged(off, _dev(logits), _dev(ntl), tokens, sampled, top_n, echo,
                                     levels=levels, top_k=top_k)
    ref_lp, ref_ids, ref_off = LO.compute_log_probabilities_ragged(
        off, logits, ntl, tokens, sampled, list(top_n), list(echo), levels=levels,
        batch_top_k=top_k)
    want = LO.assemble(ref_lp, ref_ids, ref_off, top_n, vocab)
    assert len(got) == len(want)
    for n, (g, w) in enumerate(zip(got, want)):
        if w is None:
            assert g is None, n
            continue
        assert isinstance(g, R.LogProbabilities)
        w_tlp, w_tops = w
        assert len(g.token_log_probabilities) == len(w_tlp)
        assert all(_same_value(a, b) for a, b in zip(g.token_log_probabilities, w_tlp)), n
        for gd, wd in zip(g.top_log_probabilities, w_tops):
            assert list(gd.keys()) == list(wd.keys()), (n, gd, wd)
            assert all(_same_value(gd[k], wd[k]) for k in wd), (n, gd, wd)


def _full_size(R, c, n_sample, seed):
    dev = torch.device("cuda")
    logits = gen.device_logits(c, dev, torch)
    ntl = logits.index_select(0, torch.from_numpy(c.offsets[1:].astype(np.int64) - 1).to(dev))
    torch.cuda.synchronize()
    log(f"{c.name}: rows={c.total_tokens} vocab={c.vocab} generated")
    lp, ids, out_off = R.compute_log_probabilities_ragged(
        c.offsets, logits, ntl, c.tokens, c.sampled, c.top_n, c.echo)
    torch.cuda.synchronize()
    log(f"{c.name}: library done")
    nrows = lp.shape[0]
    rng = np.random.default_rng(seed)
    rows = sorted(set(rng.choice(nrows, size=min(n_sample, nrows), replace=False).tolist())
                  | {0, nrows - 1})
    if c.dist.get("kind") == "quant":      # every all-equal row too
        tasks = LO.row_tasks(c.offsets, c.echo, c.top_n, c.tokens, c.sampled, True)
        eq = c.dist["equal_rows"]
        rows = sorted(set(rows) | {o for o, t in enumerate(tasks) if eq[t.src_row]})
    ref = oracle(c.offsets, DeviceRows(logits), DeviceRows(ntl), c.tokens, c.sampled, c.top_n,
                 c.echo, rows=rows)
    log(f"{c.name}: oracle done on {len(rows)} rows")
    assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), out_off, ref, c.name, rows=rows)
    desc = LO.row_tasks(c.offsets, c.echo, c.top_n, c.tokens, c.sampled, True)
    check_all_rows_properties(torch, logits, desc, lp, ids, c.vocab)
    log(f"{c.name}: all-row properties hold")
    del logits, ntl, lp, ids
    torch.cuda.empty_cache()


@pytest.mark.parametrize("levels", [5, 6])
@pytest.mark.parametrize("name,n_sample", [("decode_peaked", 256), ("ragged_echo_mix", 520),
                                           ("tie_edge_stress", 200)])
def test_full_size_at_large_k(R, name, n_sample, levels):
    """The named workloads at full size with every read request asking for
    all 31 or 63 ranked slots (bulk merges, the published bound, the
    two-buffer stream at 16 waves): every row of decode and the ragged mix,
    200 sampled rows of the tie workload, against the oracle."""
    c = gen.WORKLOADS[name]()
    cap = (1 << levels) - 1
    top_n = np.where(np.asarray(c.top_n) > 0, cap, 0).astype(np.int32)
    dev = torch.device("cuda")
    logits = gen.device_logits(c, dev, torch)
    ntl = logits.index_select(0, torch.from_numpy(c.offsets[1:].astype(np.int64) - 1).to(dev))
    lp, ids, out_off = R.compute_log_probabilities_ragged(
        c.offsets, logits if c.has_logits else None, ntl, c.tokens, c.sampled, top_n, c.echo,
        levels=levels)
    torch.cuda.synchronize()
    nrows = lp.shape[0]
    rng = np.random.default_rng(levels)
    rows = sorted(set(rng.choice(nrows, size=min(n_sample, nrows), replace=False).tolist())
                  | {0, nrows - 1})
    log(f"{name} at levels {levels}: {len(rows)} of {nrows} rows compared")
    ref = oracle(c.offsets, DeviceRows(logits) if c.has_logits else None, DeviceRows(ntl),
                 c.tokens, c.sampled, top_n, c.echo, levels=levels, rows=rows)
    assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), out_off, ref, f"{name} levels {levels}",
                  rows=rows)
    del logits, ntl, lp, ids
    torch.cuda.empty_cache()


def test_prefill_echo_large_full_size(R):
    _full_size(R, gen.prefill_echo_large(), 600, 41)


def test_tie_edge_stress_full_size(R):
    _full_size(R, gen.tie_edge_stress(), 400, 51)


_BEYOND_2P24 = {}


def _beyond_2p24_case():
    """Three rows of 2^24 + 37 entries and the oracle's result for them
    (computed once: the oracle sorts each row in full)."""
    if not _BEYOND_2P24:
        vocab = (1 << 24) + 37
        b = 1 << 24
        rng = np.random.default_rng(24)
        x0 = (rng.standard_normal(vocab) * 2).astype(np.float32)
        for i in (vocab - 1, b + 1, b - 1, 5):
            x0[i] = 20.0                         # equal maxima on both sides of 2^24
        x1 = (rng.integers(-3, 4, vocab) * 0.5).astype(np.float32)
        x1[b - 3: b + 30] = 9.0                   # a run of ties straddling 2^24
        x2 = np.full(vocab, -np.inf, np.float32)
        x2[[b, b + 2, vocab - 1, vocab - 5]] = np.array([1.0, 2.0, 2.0, -1.0], np.float32)
        logits = np.stack([x0, x1, x2])
        off = np.array([0, 1, 3], np.uint32)      # request 0: one row; request 1: two rows, echo
        echo = np.array([False, True])
        top_n = np.array([7, 7])
        ntl = logits[off[1:].astype(np.int64) - 1]
        tokens = np.array([b + 7, 3, b + 2], np.uint32)
        sampled = np.array([vocab - 1, b + 5], np.uint32)
        args = (off, logits, ntl, tokens, sampled, top_n, echo)
        _BEYOND_2P24.update(vocab=vocab, args=args, ref=oracle(*args))
    return _BEYOND_2P24


@pytest.mark.parametrize("split", [None, 5])
def test_ids_beyond_float_exact_integers(R, split):
    """Rows of 2^24 + 37 entries: ids above 2^24, past the integers float32
    holds exactly, rank, break ties by id across that boundary, fill the
    chosen slot and pass through the segment records (split 5) like any
    other id.  Every row is compared with the oracle in full."""
    log(f"ids beyond 2^24: split={split}")
    case = _beyond_2p24_case()
    vocab, b = case["vocab"], 1 << 24
    off, logits, ntl, tokens, sampled, top_n, echo = case["args"]
    got = run_library(R, torch, off, _dev(logits), _dev(ntl), tokens, sampled, top_n, echo,
                      split=split)
    assert_parity(*got, case["ref"], f"ids beyond 2^24 split={split}")
    assert got[1][0, :4].tolist() == [5, b - 1, b + 1, vocab - 1]
    assert got[1][1, :7].tolist() == list(range(b - 3, b + 4))


@pytest.mark.parametrize("vocab,split", [((1 << 28) + 5, None), ((1 << 28) + 5, 2), (1 << 28, 1)])
def test_rows_at_the_segment_limit(R, vocab, split):
    """One row of 2^28 (+ 5) entries: the most one workgroup streams is 2^28
    (split 1 at 2^28), a longer row is cut into segments (the default plan,
    or 2 forced) and the record merge returns the planted maxima from all
    of them.  The planted values are the only entries at or above 9.5
    (counted on the host), which fixes the ranking; the log-probabilities
    are the oracle's log-softmax of the whole row."""
    log(f"row at the segment limit: vocab={vocab} split={split}")
    rng = np.random.default_rng(vocab)
    x = rng.standard_normal(vocab, dtype=np.float32)
    planted = [(3, 12.0), (vocab - 1, 12.0), (vocab - 4, 11.5), (vocab // 2 + 2, 11.0),
               (100, 10.0), (vocab - 2, 10.0), (77777777, 9.5)]
    for i, v in planted:
        x[i] = v
    assert np.count_nonzero(x >= 9.5) == len(planted)
    want_ids = [i for i, _ in sorted(planted, key=lambda p: (-p[1], p[0]))]
    off = np.array([0, 1], np.uint32)
    echo = np.array([False])
    top_n = np.array([7])
    chosen = vocab - 3
    plan = R.Plan(off, echo, top_n, vocab, False)
    if split is not None:
        plan.set_split(split)
    info = plan.info()
    plan.close()
    assert split is None or info["split"] == split
    assert vocab <= 1 << 28 or info["split"] >= 2
    xd = _dev(x[None, :])
    lp, ids, out_off = run_library(R, torch, off, None, xd, np.zeros(1, np.uint32),
                                   np.array([chosen], np.uint32), top_n, echo, split=split)
    del xd
    torch.cuda.empty_cache()
    log("row at the segment limit: library done")
    assert out_off.tolist() == [0, 1]
    assert ids[0].tolist() == want_ids + [chosen]
    ref_lp, _ = LO.log_softmax_f64(x)
    want_lp = ref_lp[np.array(want_ids + [chosen])].astype(np.float32)
    assert_lp_close(lp[0], want_lp, f"row at the segment limit vocab={vocab} split={split}")


@pytest.mark.parametrize("vocab,waves,depth", [(32000, 8, 1), (128256, 16, 1)])
def test_many_rows_row_length_shapes(R, vocab, waves, depth):
    """Thousands of rows of the widths whose default shape differs (8 waves
    one chunk deep, 16 waves one chunk deep), sampled rows against the
    oracle."""
    c = gen.prefill_echo_large(seed=44, batch=4, vocab=vocab)
    info = R.Plan(c.offsets, c.echo, c.top_n, c.vocab, True).info()
    assert info["read_rows"] >= 1024
    assert (info["split"], info["waves"], info["depth"]) == (1, waves, depth)
    _full_size(R, c, 40, 43)


def test_staging_pool_plans_in_flight(R):
    """Several plans staged and launched back to back on one stream, each
    destroyed as soon as its call returns (descriptors go through the
    process-wide pinned pool): every output matches the oracle."""
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    cases, outs = [], []
    for i in range(6):
        off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(500 + i, 3000 + 500 * i, 3,
                                                                       rows_per_req=(1 + i, 3, 2, 5))
        plan = R.Plan(off, echo, top_n, ntl.shape[1], True)
        lp, ids, ws = R.alloc_outputs(plan, dev, torch)
        lg, nt = _dev(logits), _dev(ntl)
        plan.compute(lg, nt, tokens, sampled, lp, ids, ws, stream)
        out_off = plan.out_off.copy()
        plan.close()
        cases.append((off, logits, ntl, tokens, sampled, top_n, echo))
        outs.append((lp, ids, out_off, lg, nt, ws))
    torch.cuda.synchronize()
    for i, (c, o) in enumerate(zip(cases, outs)):
        ref = oracle(*c)
        assert_parity(o[0].cpu().numpy(), o[1].cpu().numpy(), o[2], ref, f"plan {i} in flight")


@pytest.mark.parametrize("temperature", [2.0 ** -126, 0.01, 1.0, 100.0, 2.0 ** 120])
def test_extreme_values(R, temperature):
    """Logits at the ends of the fp32 range, subnormals and signed zeros, at
    temperatures where (x - max) / T overflows, up to both ends of the
    accepted range [2^-126, 2^120] (at 2^-126 the subnormal row becomes an
    ordinary distribution; at 2^120 logits 6e38 apart still differ by 451
    after the division): log-probabilities that overflow fp32 become -inf
    on both sides, the rest agree."""
    rng = np.random.default_rng(int(min(temperature, 1e4) * 100) + 5)
    vocab = 4099
    rows = []
    big = np.float32(3.0e38)
    for kind in range(6):
        x = (rng.standard_normal(vocab) * 3).astype(np.float32)
        if kind == 0:
            x[rng.integers(vocab, size=5)] = big
            x[rng.integers(vocab, size=5)] = -big
        elif kind == 1:
            x = (rng.standard_normal(vocab) * 1e30).astype(np.float32)
        elif kind == 2:
            x = (rng.standard_normal(vocab) * 1e-39).astype(np.float32)   # subnormals
        elif kind == 3:
            x = np.where(rng.random(vocab) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
            x[rng.integers(vocab)] = np.float32(1e-45)
        elif kind == 4:
            x[:] = -big
            x[rng.integers(vocab)] = big
        rows.append(x)
    logits = np.stack(rows)
    off = np.arange(len(rows) + 1, dtype=np.uint32)
    tokens = rng.integers(0, vocab, len(rows)).astype(np.uint32)
    sampled = rng.integers(0, vocab, len(rows)).astype(np.uint32)
    top_n = np.full(len(rows), 7)
    echo = np.ones(len(rows), bool)
    temps = [temperature] * len(rows)
    ref = LO.compute_log_probabilities_ragged(off, logits, logits, tokens, sampled, list(top_n),
                                              list(echo), batch_temperature=temps)
    lp, ids, out_off = R.compute_log_probabilities_ragged(off, _dev(logits), _dev(logits), tokens,
                                                          sampled, top_n, echo, temperature=temps)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref[1])
    assert_close_rel(lp.cpu().numpy(), ref[0], f"extreme values T={temperature}")


def test_staging_pool_two_threads(R):
    """Two host threads call the library at once, each on its own stream:
    the pinned staging pool (a mutex-guarded process-wide list) hands each
    upload its own slot, and every result matches the oracle."""
    import threading

    batches = [_levels_batch(700 + i, 5000 + 3000 * i, 3, rows_per_req=(2 + i, 5, 1, 3))
               for i in range(2)]
    refs = [oracle(*b) for b in batches]
    dev_inputs = [(_dev(b[1]), _dev(b[2])) for b in batches]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            off, _, _, tokens, sampled, top_n, echo = batches[i]
            lg, nt = dev_inputs[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for it in range(25):
                    lp, ids, out_off = R.compute_log_probabilities_ragged(
                        off, lg, nt, tokens, sampled, top_n, echo, stream=stream)
                    stream.synchronize()
                    assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), out_off, refs[i],
                                  f"thread {i} call {it}")
        except Exception as e:          # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors[0]


def test_one_plan_shared_by_two_threads(R):
    """Read-only calls on one plan may overlap: two host threads compute with
    the same plan at once, each on its own stream with its own outputs and
    workspace and its own sampled tokens, 25 calls each; every result
    matches the oracle for that thread's tokens."""
    import threading

    off, logits, ntl, tokens, sampled0, top_n, echo = _levels_batch(808, 7001, 3,
                                                                    rows_per_req=(3, 1, 4, 2))
    rng = np.random.default_rng(809)
    sampled = [sampled0, rng.integers(0, ntl.shape[1], len(sampled0)).astype(np.uint32)]
    refs = [oracle(off, logits, ntl, tokens, sampled[k], top_n, echo) for k in range(2)]
    plan = R.Plan(off, echo, top_n, ntl.shape[1], True)
    dl, dn = _dev(logits), _dev(ntl)
    torch.cuda.synchronize()
    errors = []

    def worker(k):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                lp, ids, ws = R.alloc_outputs(plan, dl.device, torch)
                for it in range(25):
                    plan.compute(dl, dn, tokens, sampled[k], lp, ids, ws, stream)
                    stream.synchronize()
                    assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), plan.out_off, refs[k],
                                  f"thread {k} call {it}")
        except Exception as e:          # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors[0]
    plan.close()


@pytest.mark.parametrize("direct", [False, True])
def test_deterministic_and_split_independent(R, direct):
    """With lp_plan_set_deterministic the outputs repeat bit for bit; by
    default the ids repeat exactly and the values within a few fp32 ulps
    (the chunks' assignment to waves follows timing).  Ids never depend on
    the split or shape, values only at that level."""
    c = gen.ragged_echo_mix(seed=9, batch=6, lmin=30, lmax=90)
    if direct:
        c.echo[:] = True
        c.top_n = np.maximum(c.top_n, 1).astype(np.int32)
    logits = _dev(gen.host_logits(c))
    ntl = logits.index_select(0, torch.from_numpy(c.offsets[1:].astype(np.int64) - 1).cuda())
    args = (c.offsets, logits, ntl, c.tokens, c.sampled, c.top_n, c.echo)
    for s, w, dp in ((None, None, None), (1, 8, 2), (1, 4, 1), (3, 16, 2)):
        a = run_library(R, torch, *args, split=s, waves=w, depth=dp, deterministic=True)
        b = run_library(R, torch, *args, split=s, waves=w, depth=dp, deterministic=True)
        assert np.array_equal(a[1], b[1]), (s, w, dp)
        assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32)), (s, w, dp)
        for _ in range(3):
            f = run_library(R, torch, *args, split=s, waves=w, depth=dp)
            assert np.array_equal(a[1], f[1]), (s, w, dp)
            np.testing.assert_allclose(a[0], f[0], rtol=0, atol=2e-6)
    a = run_library(R, torch, *args, deterministic=True)
    for s, w, dp in ((2, 4, 2), (4, 8, 1), (64, 4, 1), (1, 8, 2), (1, 16, 1), (5, 16, 2), (1, 8, 1)):
        for det in (True, False):
            d = run_library(R, torch, *args, split=s, waves=w, depth=dp, deterministic=det)
            assert np.array_equal(a[1], d[1]), (s, w, dp, det)
            np.testing.assert_allclose(a[0], d[0], rtol=0, atol=2e-6)


@pytest.mark.parametrize("levels", [4, 5, 6])
def test_shapes_agree_at_deep_levels(R, levels):
    """At 15, 31 and 63 slots the end of the row kernel and the record merge
    rank keys by binary search over sorted lists, and each row's bound uses
    the keys it needs (top_n drawn up to the cap): every shape and split
    gives the same ids and, within fp32 rounding, the same values, and the
    default one matches the oracle."""
    log(f"shapes agree at levels={levels}")
    cap = LO.max_top_n(levels)
    c = gen.ragged_echo_mix(seed=20 + levels, batch=6, lmin=20, lmax=70, vocab=20011)
    rng = np.random.default_rng(levels)
    top_n = rng.integers(0, cap + 1, len(c.top_n))
    top_n[0], top_n[1] = cap, 1
    logits_np = gen.host_logits(c)
    ntl_np = gen.next_token_rows(c, logits_np)
    logits, ntl = _dev(logits_np), _dev(ntl_np)
    args = (c.offsets, logits, ntl, c.tokens, c.sampled, top_n, c.echo)
    a = run_library(R, torch, *args, levels=levels)
    ref = oracle(c.offsets, logits_np, ntl_np, c.tokens, c.sampled, top_n, c.echo, levels=levels)
    assert_parity(*a, ref, f"deep levels={levels} default shape")
    max_split = min(64, 1024 // cap)     # the merge holds 1024 keys, at most 64 segments
    for s, w, dp in ((1, 4, 1), (1, 8, 2), (1, 16, 1), (2, 4, 2), (5, 8, 1),
                     (min(9, max_split), 16, 2), (max_split, 8, 1)):
        d = run_library(R, torch, *args, split=s, waves=w, depth=dp, levels=levels)
        assert np.array_equal(a[1], d[1]), (levels, s, w, dp)
        np.testing.assert_allclose(a[0], d[0], rtol=0, atol=2e-6)


def test_outputs_stay_in_bounds_and_plan_is_reusable(R):
    c = gen.ragged_echo_mix(seed=10, batch=5, lmin=5, lmax=40, vocab=3001)
    logits_np = gen.host_logits(c)
    logits = _dev(logits_np)
    ntl = _dev(gen.next_token_rows(c, logits_np))
    plan = R.Plan(c.offsets, c.echo, c.top_n, c.vocab, True)
    n = plan.out_rows
    canary_lp = torch.full((n + 4, 8), 123.0, device="cuda")
    canary_id = torch.full((n + 4, 8), 77, dtype=torch.uint32, device="cuda")
    ws = torch.empty(plan.workspace_bytes + 4096, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for trial in range(3):
        rng = np.random.default_rng(trial)
        tokens = rng.integers(0, c.vocab, c.total_tokens).astype(np.uint32)
        sampled = rng.integers(0, c.vocab, c.batch).astype(np.uint32)
        plan.compute(logits, ntl, tokens, sampled, canary_lp, canary_id, ws, stream)
        torch.cuda.synchronize()
        ref = oracle(c.offsets, logits_np, gen.next_token_rows(c, logits_np), tokens, sampled,
                     c.top_n, c.echo)
        lp = canary_lp.cpu().numpy()
        ids = canary_id.cpu().numpy()
        assert np.all(lp[n:] == 123.0) and np.all(ids[n:] == 77)
        assert_parity(lp[:n], ids[:n], plan.out_off, ref, f"reuse trial {trial}")
    plan.close()


def test_default_split_in_two(R):
    """120 next-token rows of 70001 entries (segments hold at least 32768):
    the default plan cuts each row in two (16 waves, one chunk deep) and
    merges the records; every row matches the oracle, special rows
    included."""
    vocab, rows = 70001, 120
    rng = np.random.default_rng(120)
    ntl_np = _special_rows(rng, rows, vocab)
    off = np.arange(rows + 1, dtype=np.uint32)
    echo = np.zeros(rows, bool)
    top_n = rng.integers(1, 8, rows)
    sampled = rng.integers(0, vocab, rows).astype(np.uint32)
    tokens = np.zeros(rows, np.uint32)
    plan = R.Plan(off, echo, top_n, vocab, False)
    info = plan.info()
    plan.close()
    assert (info["split"], info["waves"], info["depth"]) == (2, 16, 1)
    got = run_library(R, torch, off, None, _dev(ntl_np), tokens, sampled, top_n, echo)
    ref = oracle(off, None, ntl_np, tokens, sampled, top_n, echo)
    assert_parity(*got, ref, "default split in two")


@pytest.mark.parametrize("levels,shape", [(3, (8, 8, 1)), (4, (8, 16, 1)), (5, (4, 16, 1)),
                                          (6, (4, 16, 1))])
def test_default_segments_of_long_rows(R, levels, shape):
    """8 next-token rows of 128256 entries: the default plan cuts each row
    into 8 segments of at least 16000 entries (over 8 waves at 7 ranked
    slots, 16 at 15), or 4 from 31 slots up, and merges the records; every
    row matches the oracle, special rows included."""
    vocab, rows = 128256, 8
    rng = np.random.default_rng(80 + levels)
    ntl_np = _special_rows(rng, rows, vocab)
    off = np.arange(rows + 1, dtype=np.uint32)
    echo = np.zeros(rows, bool)
    top_n = rng.integers(1, 1 << levels, rows)
    top_n[0] = (1 << levels) - 1
    sampled = rng.integers(0, vocab, rows).astype(np.uint32)
    tokens = np.zeros(rows, np.uint32)
    plan = R.Plan(off, echo, top_n, vocab, False, levels=levels)
    info = plan.info()
    plan.close()
    assert (info["split"], info["waves"], info["depth"]) == shape
    got = run_library(R, torch, off, None, _dev(ntl_np), tokens, sampled, top_n, echo,
                      levels=levels)
    ref = oracle(off, None, ntl_np, tokens, sampled, top_n, echo, levels=levels)
    assert_parity(*got, ref, f"default segments, levels {levels}")


def test_empty_batch_and_padding_only_batch(R):
    """No request: empty outputs and offsets [0], nothing launched.  Every
    top_n 0 (levels 3): no logits row is read and every slot of every
    output row is padding (-inf, 0xFFFFFFFF), as the oracle gives."""
    vocab = 1000
    ntl = _dev(np.zeros((0, vocab), np.float32))
    lp, ids, out_off = run_library(R, torch, np.zeros(1, np.uint32), None, ntl,
                                   np.zeros(0, np.uint32), np.zeros(0, np.uint32),
                                   np.zeros(0, np.int32), np.zeros(0, bool))
    assert lp.shape == (0, 8) and ids.shape == (0, 8) and out_off.tolist() == [0]
    rng = np.random.default_rng(3)
    off = np.array([0, 3, 4, 9], np.uint32)
    logits = rng.standard_normal((9, vocab)).astype(np.float32)
    ntl_np = logits[off[1:].astype(np.int64) - 1]
    tokens = rng.integers(0, vocab, 9).astype(np.uint32)
    sampled = rng.integers(0, vocab, 3).astype(np.uint32)
    top_n = np.zeros(3, np.int32)
    echo = np.array([True, False, True])
    got = run_library(R, torch, off, _dev(logits), _dev(ntl_np), tokens, sampled, top_n, echo)
    ref = oracle(off, logits, ntl_np, tokens, sampled, top_n, echo)
    assert_parity(*got, ref, "padding only")
    assert np.all(got[1] == 0xFFFFFFFF) and np.all(np.isneginf(got[0]))


def test_errors_reported_before_launch(R):
    c = gen.no_echo_next_token()
    ntl = _dev(gen.host_logits(c))
    with pytest.raises(R.LogprobError) as e:
        R.compute_log_probabilities_ragged(c.offsets, None, ntl, c.tokens,
                                           np.array([0, 1, 2, 32000], np.uint32), c.top_n, c.echo)
    assert e.value.name == "LP_ERR_TOKEN_RANGE"
    plan = R.Plan(c.offsets, c.echo, c.top_n, c.vocab, False)
    lp, ids, ws = R.alloc_outputs(plan, ntl.device, torch)
    small = ws[:0]
    with pytest.raises(R.LogprobError) as e:
        plan.compute(None, ntl, c.tokens, c.sampled, lp, ids, small, torch.cuda.current_stream())
    assert e.value.name == "LP_ERR_WORKSPACE"
    with pytest.raises(R.LogprobError):
        R.compute_log_probabilities_ragged(c.offsets, None, ntl.double(), c.tokens, c.sampled,
                                           c.top_n, c.echo)


def test_calls_on_streams_other_than_the_current_one(R):
    """Outputs and workspace are allocated on the launch stream, so a call on
    a stream that is not the current one cannot have its workspace handed to
    the next call's allocation while its kernels still read it: back-to-back
    calls alternate between two such streams and every result matches the
    oracle."""
    c = gen.ragged_echo_mix(seed=31, batch=6, lmin=40, lmax=300, vocab=20011)
    logits = gen.host_logits(c)
    ntl = gen.next_token_rows(c, logits)
    ref = oracle(c.offsets, logits, ntl, c.tokens, c.sampled, c.top_n, c.echo)
    dl, dn = _dev(logits), _dev(ntl)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(6):
        s = s1 if i % 2 == 0 else s2
        log(f"call {i} on stream {1 + i % 2}")
        lp, ids, off = R.compute_log_probabilities_ragged(c.offsets, dl, dn, c.tokens, c.sampled,
                                                          c.top_n, c.echo, stream=s)
        outs.append((lp, ids, off))
    torch.cuda.synchronize()
    for i, (lp, ids, off) in enumerate(outs):
        assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), off, ref, f"stream call {i}")


def test_launcher_holds_its_buffers(R):
    """A launcher keeps the tensors it was made from: with every other
    reference dropped and the caching allocator handing out blocks of the
    same sizes (filled with garbage), its launches still read the staged
    descriptors and write outputs that match the oracle."""
    c = gen.ragged_echo_mix(seed=33, batch=5, lmin=20, lmax=80, vocab=12007)
    logits = gen.host_logits(c)
    ntl = gen.next_token_rows(c, logits)
    ref = oracle(c.offsets, logits, ntl, c.tokens, c.sampled, c.top_n, c.echo)
    plan = R.Plan(c.offsets, c.echo, c.top_n, c.vocab, True)
    lp, ids, ws = R.alloc_outputs(plan, torch.device("cuda"), torch)
    plan.stage(c.tokens, c.sampled, ws, torch.cuda.current_stream())
    launch = plan.launcher(_dev(logits), None, lp, ids, ws)
    shapes = [(t.shape, t.dtype) for t in (lp, ids, ws)]
    del lp, ids, ws
    churn = [torch.full(sh, 7, dtype=dt, device="cuda") for sh, dt in shapes for _ in range(3)]
    held = launch()
    torch.cuda.synchronize()
    del churn
    assert_parity(held[2].cpu().numpy(), held[3].cpu().numpy(), plan.out_off, ref, "launcher buffers")


@pytest.mark.parametrize("rows", [262144, 262145])
def test_compute_descriptors_either_side_of_the_zero_copy_limit(R, rows):
    """lp_compute_ragged lets the kernels read the descriptors of plans up to
    262144 output rows from pinned host memory and stages larger plans into
    the workspace: both sides of the limit match the oracle, and a staged
    launch of the same plan (lp_stage_ragged, then lp_launch_ragged)
    matches the compute call bit for bit (rows of 67 entries: one partial
    chunk, so no chunk order to differ)."""
    vocab = 67
    rng = np.random.default_rng(rows)
    lengths = np.full(rows // 1 if rows % 2 else rows // 2, 1 if rows % 2 else 2)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    echo = np.ones(len(lengths), bool) if rows % 2 == 0 else np.zeros(len(lengths), bool)
    top_n = rng.integers(1, 8, len(lengths))
    logits = _special_rows(rng, int(off[-1]), vocab)
    ntl = logits[off[1:].astype(np.int64) - 1]
    tokens = rng.integers(0, vocab, int(off[-1])).astype(np.uint32)
    sampled = rng.integers(0, vocab, len(lengths)).astype(np.uint32)
    log(f"zero-copy limit: rows={rows}")
    dl, dn = _dev(logits), _dev(ntl)
    plan = R.Plan(off, echo, top_n, vocab, True)
    assert plan.info()["out_rows"] == rows
    lp, ids, ws = R.alloc_outputs(plan, torch.device("cuda"), torch)
    plan.compute(dl, dn, tokens, sampled, lp, ids, ws)
    lp2, ids2, _ = R.alloc_outputs(plan, torch.device("cuda"), torch)
    plan.stage(tokens, sampled, ws)
    plan.launch(dl, dn, lp2, ids2, ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    assert torch.equal(lp.view(torch.int32), lp2.view(torch.int32))
    sample = sorted(set(rng.choice(rows, size=64, replace=False).tolist()) | {0, rows - 1})
    ref = oracle(off, logits, ntl, tokens, sampled, top_n, echo, rows=sample)
    assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), plan.out_off, ref, f"rows={rows}", rows=sample)
    plan.close()


@pytest.mark.parametrize("segs,threads,loads", [(1, 512, 4), (1, 256, 1), (2, 1024, 8), (4, 256, 2),
                                                (3, 512, 8)])
def test_stream_read_shapes_sum_rows(R, segs, threads, loads):
    """The plain-read probe in its launch shapes reads every float of each
    row once: the per-share sums add up to the row sums."""
    log(f"stream read shape segs={segs} threads={threads} loads={loads}")
    rng = np.random.default_rng(segs * 100 + loads)
    rows, row_len = 37, 128256 + 4 * 97
    x = _dev(rng.standard_normal((rows, row_len)).astype(np.float32))
    partial = torch.full((rows * segs,), float("nan"), dtype=torch.float32, device="cuda")
    R.binding.stream_read_shape_launcher(x, rows, row_len, segs, threads, loads, partial)()
    torch.cuda.synchronize()
    got = partial.view(rows, segs).double().sum(dim=1).cpu().numpy()
    want = x.double().sum(dim=1).cpu().numpy()
    assert np.all(np.abs(got - want) < 1e-3 * np.sqrt(row_len)), (got - want)


@pytest.mark.parametrize("levels", [5, 6])
@pytest.mark.parametrize("vocab", [15 * 1024, 16 * 1024, 17 * 1024 + 5, 33 * 1024 + 3, 128256])
@pytest.mark.parametrize("deterministic", [False, True])
def test_two_buffer_stream_at_large_k(R, levels, vocab, deterministic):
    """31 and 63 slots at 16 waves one chunk deep stream through two buffers
    taken in turn: chunk counts below, at and just past one per wave, and a
    decode-width row, in both chunk orders, against the oracle."""
    log(f"two-buffer stream levels={levels} vocab={vocab} deterministic={deterministic}")
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(vocab + levels, vocab, levels,
                                                                   rows_per_req=(1, 3, 1, 2))
    ref = oracle(off, logits, ntl, tokens, sampled, top_n, echo, levels=levels)
    for split in (1, 2):
        got = run_library(R, torch, off, _dev(logits), _dev(ntl), tokens, sampled, top_n, echo,
                          split, 16, 1, levels=levels, deterministic=deterministic)
        assert_parity(*got, ref, f"two-buffer levels={levels} vocab={vocab} split={split}")


def test_staging_slots_reused_across_streams(R):
    """Staging slots finish out of order: a long launch on one stream holds
    the oldest slot while many short ones on a second stream finish and are
    reused (the pool looks past a busy first slot).  Every short call writes
    its own outputs and they all match the oracle; so do sampled rows of the
    long one."""
    dev = torch.device("cuda")
    slow, fast = torch.cuda.Stream(), torch.cuda.Stream()
    # the long launch: 12000 rows of 32000 read through the zero-copy path
    rng = np.random.default_rng(77)
    n_long, v_long = 12000, 32000
    long_logits = torch.from_numpy(rng.standard_normal((n_long, v_long), dtype=np.float32) * 2).to(dev)
    long_off = np.array([0, n_long], np.uint32)
    long_tok = rng.integers(0, v_long, n_long).astype(np.uint32)
    long_smp = rng.integers(0, v_long, 1).astype(np.uint32)
    long_plan = R.Plan(long_off, [1], [7], v_long, True)
    with torch.cuda.stream(slow):
        llp, lids, lws = R.alloc_outputs(long_plan, dev, torch)
    torch.cuda.synchronize()
    # the short calls: 40 small batches, each with its own inputs and outputs
    shorts = []
    for i in range(40):
        off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(900 + i, 1000 + 37 * i, 3,
                                                                       rows_per_req=(1, 2, 1, 3))
        plan = R.Plan(off, echo, top_n, ntl.shape[1], True)
        with torch.cuda.stream(fast):
            lp, ids, ws = R.alloc_outputs(plan, dev, torch)
        shorts.append(((off, logits, ntl, tokens, sampled, top_n, echo), plan, _dev(logits),
                       _dev(ntl), lp, ids, ws))
    torch.cuda.synchronize()
    long_plan.compute(long_logits, None, long_tok, long_smp, llp, lids, lws, slow)
    for c, plan, lg, nt, lp, ids, ws in shorts:
        plan.compute(lg, nt, c[3], c[4], lp, ids, ws, fast)
    torch.cuda.synchronize()
    for i, (c, plan, lg, nt, lp, ids, ws) in enumerate(shorts):
        ref = oracle(*c)
        assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), plan.out_off.copy(), ref,
                      f"short call {i} beside a long one")
        plan.close()
    tasks = LO.row_tasks(long_off, [1], [7], long_tok, long_smp, True)
    for r in (0, 1, 4321, n_long - 1):
        t = tasks[r]
        want_lp, want_ids = LO.compute_row(long_logits[t.src_row].cpu().numpy(), t.chosen, t.top_n, 8)
        assert np.array_equal(lids[r].cpu().numpy(), want_ids), r
        assert_lp_close(llp[r].cpu().numpy(), want_lp, f"long row {r}")
    long_plan.close()


def test_staging_slots_not_refilled_under_queued_kernels(R):
    """Back-to-back lp_compute_ragged calls on one stream, each with its own
    sampled tokens and so its own descriptors, enqueued far faster than the
    GPU runs them (1024 rows of 131072 per call, read in place from the
    pinned staging slots): a slot is refilled only once the kernel that reads
    it has ended.  Every queued call's outputs equal those of the same call
    run alone, bit for bit (deterministic chunk order), and sampled rows of
    the first and last calls match the oracle."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(4711)
    B, V, calls = 1024, 131072, 24
    ntl_host = (rng.standard_normal((B, V), dtype=np.float32) * 2).astype(np.float32)
    ntl = _dev(ntl_host)
    off = np.arange(B + 1, dtype=np.uint32)
    plan = R.Plan(off, np.zeros(B, bool), np.full(B, 7, np.int32), V, False)
    plan.set_deterministic(True)
    assert plan.info()["out_rows"] <= 262144         # the in-place descriptor path
    sampled = [rng.integers(0, V, B).astype(np.uint32) for _ in range(calls)]
    stream = torch.cuda.current_stream()
    alone = []
    for i in range(calls):
        lp, ids, ws = R.alloc_outputs(plan, dev, torch)
        plan.compute(None, ntl, None, sampled[i], lp, ids, ws, stream)
        torch.cuda.synchronize()
        alone.append((lp.cpu().numpy(), ids.cpu().numpy()))
    queued = [R.alloc_outputs(plan, dev, torch) for _ in range(calls)]
    fns = [plan.computer(None, ntl, None, sampled[i], *queued[i], stream) for i in range(calls)]
    torch.cuda.synchronize()
    for f in fns:
        f()
    torch.cuda.synchronize()
    for i in range(calls):
        lp, ids, _ = queued[i]
        assert np.array_equal(ids.cpu().numpy(), alone[i][1]), f"call {i}: ids"
        assert np.array_equal(lp.cpu().numpy().view(np.uint32), alone[i][0].view(np.uint32)), \
            f"call {i}: logprobs"
    for i in (0, calls - 1):
        for r in (0, 517, B - 1):
            want_lp, want_ids = LO.compute_row(ntl_host[r], int(sampled[i][r]), 7, 8)
            assert np.array_equal(alone[i][1][r], want_ids), (i, r)
            assert_lp_close(alone[i][0][r], want_lp, f"call {i} row {r}")
    plan.close()


def test_short_or_mistyped_device_buffers_are_refused(R):
    """Device buffers smaller than the plan reads or writes, of the wrong
    element type or not contiguous are refused (LP_ERR_SHAPE) before any
    kernel runs; the same call with the right buffers matches the oracle."""
    off, logits, ntl, tokens, sampled, top_n, echo = _levels_batch(4242, 3001, 3)
    plan = R.Plan(off, echo, top_n, ntl.shape[1], True)
    dev = torch.device("cuda")
    lp, ids, ws = R.alloc_outputs(plan, dev, torch)
    lg, nt = _dev(logits), _dev(ntl)
    bad = [
        (lg[:-1], nt, lp, ids),                                    # one logits row short
        (lg.double(), nt, lp, ids),                                # fp64 logits
        (torch.empty(lg.shape[1], lg.shape[0], device=dev).t(), nt, lp, ids),   # not contiguous
        (lg, nt, lp[:-1], ids),                                    # one output row short
        (lg, nt, lp, ids.view(torch.float32)),                     # ids as floats
        (lg, nt, lp.view(torch.int32), ids),                       # logprobs as integers
    ]
    for k, (a, b, c, d) in enumerate(bad):
        with pytest.raises(R.LogprobError) as e:
            plan.compute(a, b, tokens, sampled, c, d, ws)
        assert e.value.name == "LP_ERR_SHAPE", (k, e.value.name)
    plan.compute(lg, nt, tokens, sampled, lp, ids, ws)
    torch.cuda.synchronize()
    ref = oracle(off, logits, ntl, tokens, sampled, top_n, echo)
    assert_parity(lp.cpu().numpy(), ids.cpu().numpy(), plan.out_off.copy(), ref, "after refusals")
    plan.close()
