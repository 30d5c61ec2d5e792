"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Each ``pin_*`` raises AssertionError when the oracle departs from a value
that does not come from the oracle itself: a hand-worked example, a closed
form, a 50-digit brute force, an exhaustive brute-force ranking or the
worked example printed on the SGLang page "logprob、finish reason 与 output
processing" (section "logprob 的数值形态").  The pins read the oracle's
functions through the module object at call time, so a test can plant a
mistake in the oracle (monkeypatch) and check that some pin catches it.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import mpmath
import numpy as np

import oracle.logprob_oracle as LO

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ brute forces

def brute_top_ids(xs, k):
    """Repeated argmax over a Python list, scanning ids upward and replacing
    only on a strictly larger value: ties keep the lowest id; -0.0 == +0.0."""
    remaining = list(range(len(xs)))
    out = []
    for _ in range(min(k, len(xs))):
        best = None
        for i in remaining:
            if best is None or xs[i] > xs[best]:
                best = i
        out.append(best)
        remaining.remove(best)
    return out


def mp_logprobs(xs, dps=50):
    """log p_i = x_i - log(sum_j e^{x_j}) at ``dps`` digits (finite xs only)."""
    with mpmath.workdps(dps):
        s = mpmath.fsum(mpmath.e ** mpmath.mpf(float(x)) for x in xs)
        lse = mpmath.log(s)
        return [mpmath.mpf(float(x)) - lse for x in xs], lse


# ------------------------------------------------------------------ offsets / mapping

def pin_offsets_hand_example():
    # L = (3, 1, 2), echo = (T, F, T) -> counts (3, 1, 2), offsets (0, 3, 4, 6)
    counts, out_off = LO.output_counts_and_offsets([0, 3, 4, 6], [True, False, True])
    assert counts.dtype == np.uint32 and out_off.dtype == np.uint32
    assert counts.tolist() == [3, 1, 2], counts
    assert out_off.tolist() == [0, 3, 4, 6], out_off
    # no echo: one row per request; all echo: the input offsets themselves
    _, o = LO.output_counts_and_offsets([0, 5, 6, 9], [False] * 3)
    assert o.tolist() == [0, 1, 2, 3], o
    _, o = LO.output_counts_and_offsets([0, 5, 6, 9], [True] * 3)
    assert o.tolist() == [0, 5, 6, 9], o
    assert LO.kernel_row_offsets([0, 5, 6, 9], False).tolist() == [0, 1, 2, 3]
    assert LO.kernel_row_offsets([0, 5, 6, 9], True).tolist() == [0, 5, 6, 9]


def pin_mapping_hand_example():
    # off (0,3,4,6), echo (T,F,T): request 0 reads rows 0,1,2 and predicts
    # tokens[1], tokens[2], sampled[0]; request 1 reads row 3 -> sampled[1];
    # request 2 reads rows 4,5 -> tokens[5], sampled[2].
    tokens = [100, 101, 102, 103, 104, 105]
    sampled = [900, 901, 902]
    tasks = LO.row_tasks([0, 3, 4, 6], [True, False, True], [7, 3, 1], tokens, sampled, True)
    got = [(t.src_row, t.chosen, t.top_n) for t in tasks]
    want = [(0, 101, 7), (1, 102, 7), (2, 900, 7), (3, 901, 3), (4, 105, 1), (5, 902, 1)]
    assert got == want, got
    # a non-echo request with full logits reads its last row
    tasks = LO.row_tasks([0, 3, 4, 6], [False, False, True], [1, 1, 1], tokens, sampled, True)
    got = [(t.src_row, t.chosen) for t in tasks]
    assert got == [(2, 900), (3, 901), (4, 105), (5, 902)], got
    # no full logits: row n of next_token_logits, chosen = sampled
    tasks = LO.row_tasks([0, 3, 4, 6], [False] * 3, [2, 2, 2], tokens, sampled, False)
    assert [(t.src_row, t.chosen) for t in tasks] == [(0, 900), (1, 901), (2, 902)]
    # L_n = 1 with echo: its only row predicts the sampled token
    tasks = LO.row_tasks([0, 1], [True], [2], [7], [8], True)
    assert [(t.src_row, t.chosen) for t in tasks] == [(0, 8)]


# ------------------------------------------------------------------ log-softmax

def pin_logsoftmax_bruteforce(rows):
    """Oracle float64 log-softmax against a 50-digit evaluation."""
    for xs in rows:
        lp, lse = LO.log_softmax_f64(np.asarray(xs, dtype=np.float32))
        ref, ref_lse = mp_logprobs(np.asarray(xs, dtype=np.float32).tolist())
        assert abs(lse - float(ref_lse)) <= 1e-12 * max(1.0, abs(float(ref_lse))), (xs, lse)
        for a, b in zip(lp, ref):
            assert abs(a - float(b)) <= 1e-12 * max(1.0, abs(float(b))), (xs, a, b)


def pin_logsoftmax_closed_forms():
    # uniform row -> -ln V
    for v in (1, 3, 111, 32000, 256000):
        lp, _ = LO.log_softmax_f64(np.full(v, 0.75, dtype=np.float32))
        assert np.allclose(lp, -math.log(v), rtol=0, atol=1e-12), v
    assert abs(-math.log(256000) - (-12.452933)) < 1e-6
    # two tokens at distance d: -log1p(e^-d) and -d - log1p(e^-d)
    for a, b in ((1.0, 0.0), (5.5, -3.25), (-20.0, -20.5), (0.0, -60.0)):
        lp, _ = LO.log_softmax_f64(np.array([a, b], dtype=np.float32))
        d = a - b
        assert abs(lp[0] - (-math.log1p(math.exp(-d)))) < 1e-14, (a, b, lp)
        assert abs(lp[1] - (-d - math.log1p(math.exp(-d)))) < 1e-12, (a, b, lp)
    # a row holding one finite entry among -inf: that entry has logprob 0
    lp, _ = LO.log_softmax_f64(np.array([-np.inf, 2.5, -np.inf], dtype=np.float32))
    assert lp[1] == 0.0 and np.isneginf(lp[0]) and np.isneginf(lp[2])


def pin_logsoftmax_invariants(rows):
    for xs in rows:
        x = np.asarray(xs, dtype=np.float32)
        lp, _ = LO.log_softmax_f64(x)
        assert np.all(lp <= 1e-15), lp              # a logprob is <= 0
        assert abs(np.sum(np.exp(lp)) - 1.0) < 1e-12
        for c in (-50.0, 3.5, 1e3):
            xs2 = x.astype(np.float64) + c            # exact in float64
            lp2, _ = LO.log_softmax_f64(xs2)
            assert np.allclose(lp, lp2, rtol=0, atol=1e-9 * max(1.0, abs(c))), c


def pin_worked_example():
    """The SGLang page's printed example: rebuilt rows give the printed values."""
    with open(os.path.join(GOLDEN, "sglang_worked_example.json"), encoding="utf-8") as f:
        g = json.load(f)
    for pos in (0, 1):
        (t1, a), (t2, b) = g["top_logprobs"][pos]
        rest = math.log((1.0 - math.exp(a) - math.exp(b)) / 8.0)
        row = np.array([a, b] + [rest] * 8, dtype=np.float64)
        lp, lse = LO.log_softmax_f64(row)
        assert abs(lse) < 1e-12, lse
        assert abs(lp[0] - a) < 1e-12 and abs(lp[1] - b) < 1e-12
        # top-2 through the full row path (float32 input)
        lp_out, id_out = LO.compute_row(row.astype(np.float32), 0, 2, 8)
        assert id_out[:2].tolist() == [0, 1], id_out
        assert abs(lp_out[0] - a) < 1e-6 and abs(lp_out[1] - b) < 1e-6, lp_out
        assert id_out[7] == 0 and abs(lp_out[7] - g["token_logprobs"][pos]) < 1e-6
        assert id_out[2:7].tolist() == [LO.PAD_ID] * 5
    pct = g["stated_percent"]
    assert round(100 * math.exp(g["top_logprobs"][1][0][1])) == pct[" cat"]
    assert round(100 * math.exp(g["top_logprobs"][1][1][1])) == pct[" dog"]
    (_, a), (_, b) = g["top_logprobs"][2]
    assert math.exp(a) + math.exp(b) > 1.0        # position 3 is not a distribution


# ------------------------------------------------------------------ ranking / rows

def pin_ranking_exhaustive(alphabet, vmax):
    for v in range(1, vmax + 1):
        for combo in itertools.product(alphabet, repeat=v):
            xs = list(combo)
            x = np.array(xs, dtype=np.float32)
            want_all = brute_top_ids(xs, v)
            got_all = LO.rank_descending(x)[:v].tolist()
            assert got_all == want_all, (xs, got_all, want_all)
            finite = np.isfinite(x).any()
            for k in range(0, 8):
                lp_out, id_out = LO.compute_row(x, v - 1, k, 8)
                kk = min(k, v)
                if k == 0:
                    assert id_out.tolist() == [LO.PAD_ID] * 8
                    continue
                assert id_out[:kk].tolist() == want_all[:kk], (xs, k, id_out)
                assert id_out[kk:7].tolist() == [LO.PAD_ID] * (7 - kk)
                assert np.all(np.isneginf(lp_out[kk:7]))
                assert id_out[7] == v - 1
                if finite:
                    lp, _ = LO.log_softmax_f64(x)
                    want = lp[want_all[:kk]].astype(np.float32)
                    assert np.array_equal(lp_out[:kk], want), (xs, lp_out)


def pin_ranking_special_cases():
    rng = np.random.default_rng(7)
    # all-equal row: ids 0..min(top_n, V)-1
    for v in (1, 3, 7, 8, 111):
        lp_out, id_out = LO.compute_row(np.full(v, -1.5, dtype=np.float32), 0, 7, 8)
        kk = min(7, v)
        assert id_out[:kk].tolist() == list(range(kk)), id_out
        assert np.allclose(lp_out[:kk], -math.log(v), atol=1e-6)
    # one boosted token ranks first
    x = rng.standard_normal(1000).astype(np.float32)
    x[417] = 50.0
    _, id_out = LO.compute_row(x, 3, 7, 8)
    assert id_out[0] == 417
    # -inf never enters the top-k while enough finite entries exist
    x = np.full(20, -np.inf, dtype=np.float32)
    x[[3, 9, 11]] = [1.0, 2.0, 0.5]
    lp_out, id_out = LO.compute_row(x, 0, 5, 8)
    assert id_out[:5].tolist() == [9, 3, 11, 0, 1], id_out
    assert np.all(np.isneginf(lp_out[3:5])) and np.isneginf(lp_out[7])
    # the chosen token also among the top columns holds the same value
    x = rng.standard_normal(50).astype(np.float32)
    lp_out, id_out = LO.compute_row(x, int(np.argmax(x)), 3, 8)
    assert id_out[0] == id_out[7] and lp_out[0] == lp_out[7]
    # an all -inf row: NaN logprobs, ids by the tie rule
    lp_out, id_out = LO.compute_row(np.full(4, -np.inf, dtype=np.float32), 2, 7, 8)
    assert id_out[:4].tolist() == [0, 1, 2, 3] and np.all(np.isnan(lp_out[:4]))
    assert id_out[4:7].tolist() == [LO.PAD_ID] * 3 and np.isnan(lp_out[7])


def pin_ranking_invariants(rows, k=7):
    for xs in rows:
        x = np.asarray(xs, dtype=np.float32)
        _, id_out = LO.compute_row(x, 0, k, 8)
        ids = [i for i in id_out[:7].tolist() if i != LO.PAD_ID]
        vals = x[ids].astype(np.float64)
        assert np.all(np.diff(vals) <= 0), vals
        for i in range(len(ids) - 1):
            if vals[i] == vals[i + 1]:
                assert ids[i] < ids[i + 1]
        # nothing outside the list beats its last member
        if ids:
            last_v, last_i = vals[-1], ids[-1]
            out = np.setdiff1d(np.arange(x.shape[0]), ids)
            assert not np.any((x[out] > last_v) | ((x[out] == last_v) & (out < last_i)))


def pin_batch_hand_example():
    """End to end over a tiny batch, expected values from closed forms.

    V = 4.  Request 0: echo, 3 tokens, top_n 2.  Request 1: no echo, 1 token,
    top_n 0.  Request 2: echo, 2 tokens, top_n 1.  Row r holds a spike s_r at
    id (r mod 4) over zeros, so lse_r = log(e^{s_r} + 3).
    """
    V = 4
    spikes = [2.0, -1.0, 0.5, 3.0, 1.0, 4.0]
    logits = np.zeros((6, V), dtype=np.float32)
    for r, s in enumerate(spikes):
        logits[r, r % V] = s
    ntl = logits[[2, 3, 5]]
    tokens = np.array([0, 1, 2, 3, 0, 2], dtype=np.uint32)
    sampled = np.array([3, 1, 0], dtype=np.uint32)
    lp, ids, off = LO.compute_log_probabilities_ragged(
        np.array([0, 3, 4, 6], dtype=np.uint32), logits, ntl, tokens, sampled,
        [2, 0, 1], [True, False, True])
    assert off.tolist() == [0, 3, 4, 6]
    lse = [math.log(math.exp(s) + 3.0) for s in spikes]
    P = LO.PAD_ID
    # (row, chosen, expected top ids)
    expect = {0: (0, 1, [0, 1]), 1: (1, 2, [0, 2]), 2: (2, 3, [2, 0]),
              4: (4, 2, [0]), 5: (5, 0, [1])}
    for o, (r, chosen, top) in expect.items():
        for j, t in enumerate(top):
            want = (spikes[r] if t == r % V else 0.0) - lse[r]
            assert ids[o, j] == t and abs(lp[o, j] - want) < 1e-6, (o, j, ids[o], lp[o])
        assert ids[o, len(top):7].tolist() == [P] * (7 - len(top))
        want = (spikes[r] if chosen == r % V else 0.0) - lse[r]
        assert ids[o, 7] == chosen and abs(lp[o, 7] - want) < 1e-6, (o, ids[o], lp[o])
    assert ids[3].tolist() == [P] * 8 and np.all(np.isneginf(lp[3]))   # top_n = 0


def pin_errors():
    ok = dict(input_row_offsets=np.array([0, 2, 3], np.uint32),
              logits=np.zeros((3, 5), np.float32), next_token_logits=np.zeros((2, 5), np.float32),
              tokens=np.array([1, 2, 3], np.uint32), sampled_tokens=np.array([4, 0], np.uint32),
              batch_top_n=[1, 7], batch_echo=[True, False])
    LO.compute_log_probabilities_ragged(**ok)

    def expect(code, **kw):
        args = dict(ok)
        args.update(kw)
        try:
            LO.compute_log_probabilities_ragged(**args)
        except LO.OracleError as e:
            assert e.code == code, (code, e.code)
            return
        raise AssertionError(f"no error, expected {code}")

    expect("LP_ERR_TOP_N_NEGATIVE", batch_top_n=[-1, 1])
    expect("LP_ERR_TOP_N_TOO_LARGE", batch_top_n=[8, 1])
    expect("LP_ERR_ECHO_NEEDS_LOGITS", logits=None)
    expect("LP_ERR_OFFSETS", input_row_offsets=np.array([0, 3, 3], np.uint32))
    expect("LP_ERR_OFFSETS", input_row_offsets=np.array([1, 2, 3], np.uint32))
    expect("LP_ERR_SHAPE", logits=np.zeros((4, 5), np.float32))
    expect("LP_ERR_SHAPE", logits=np.zeros((3, 6), np.float32))
    expect("LP_ERR_SHAPE", batch_echo=[True])
    expect("LP_ERR_TOKEN_RANGE", sampled_tokens=np.array([5, 0], np.uint32))
    expect("LP_ERR_TOKEN_RANGE", tokens=np.array([1, 2, 9], np.uint32))
    # levels widen the cap: 15 is fine at levels 4
    args = dict(ok)
    args["batch_top_n"] = [15, 1]
    lp, ids, _ = LO.compute_log_probabilities_ragged(levels=4, **args)
    assert lp.shape == (3, 16)


# ------------------------------------------------------------------ levels

def pin_levels_columns():
    """[MAX] §log_probabilities_ragged_graph: out_per_token is 2**levels, or 1
    when levels is 0; one column is the chosen token's, so top_n may reach
    columns - 1 ([MAX] §图支持的最大 top-n: levels 3 serves up to 7)."""
    for levels, cols in ((0, 1), (1, 2), (2, 4), (3, 8), (4, 16), (5, 32), (6, 64)):
        assert LO.columns_for_levels(levels) == cols, levels
        assert LO.max_top_n(levels) == cols - 1, levels


def pin_levels_bruteforce(rows, levels_list=(1, 2, 4, 5, 6)):
    """Every heap depth: the ranked columns are brute-force repeated argmax
    ids, padded past min(top_n, V), and the last column is the chosen token;
    a top_n beyond columns - 1 is rejected."""
    P = LO.PAD_ID
    for levels in levels_list:
        cols = 2 ** levels
        for x in rows:
            x = np.asarray(x, dtype=np.float32)
            V = x.shape[0]
            for top_n in sorted({0, 1, cols // 2, cols - 1}):
                chosen = V // 2
                lp, ids, off = LO.compute_log_probabilities_ragged(
                    np.array([0, 1], np.uint32), None, x[None, :], np.zeros(1, np.uint32),
                    np.array([chosen], np.uint32), [top_n], [False], levels=levels)
                assert lp.shape == (1, cols) and ids.shape == (1, cols)
                if top_n == 0:
                    assert ids[0].tolist() == [P] * cols
                    continue
                want = brute_top_ids([float(v) for v in x], min(top_n, V))
                got = ids[0, :len(want)].tolist()
                assert got == want, (levels, top_n, got, want)
                assert ids[0, len(want):cols - 1].tolist() == [P] * (cols - 1 - len(want))
                assert ids[0, cols - 1] == chosen
            try:
                LO.compute_log_probabilities_ragged(
                    np.array([0, 1], np.uint32), None, x[None, :], np.zeros(1, np.uint32),
                    np.array([0], np.uint32), [cols], [False], levels=levels)
            except LO.OracleError as e:
                assert e.code == "LP_ERR_TOP_N_TOO_LARGE"
            else:
                raise AssertionError(f"levels {levels}: top_n {cols} accepted")


def pin_levels_zero():
    """levels 0 keeps a single column and admits only top_n == 0, whose rows
    are padding (reading R6)."""
    x = np.array([[0.5, 1.5, -1.0]], np.float32)
    lp, ids, _ = LO.compute_log_probabilities_ragged(
        np.array([0, 1], np.uint32), None, x, np.zeros(1, np.uint32), np.array([1], np.uint32),
        [0], [False], levels=0)
    assert ids.shape == (1, 1) and ids[0, 0] == LO.PAD_ID and np.isneginf(lp[0, 0])
    try:
        LO.compute_log_probabilities_ragged(
            np.array([0, 1], np.uint32), None, x, np.zeros(1, np.uint32),
            np.array([1], np.uint32), [1], [False], levels=0)
    except LO.OracleError as e:
        assert e.code == "LP_ERR_TOP_N_TOO_LARGE"
    else:
        raise AssertionError("levels 0 accepted top_n 1")


# ------------------------------------------------------------------ host assembly

def pin_assembly_hand_examples():
    """[MAX] §compute_top 的结果组装, worked by hand: padding dropped, pairs
    sorted by logprob descending, top_n kept, the last column forced in
    (appended, or overwriting a present key in place)."""
    P = LO.PAD_ID
    lp = np.array([-1.2, -0.5, -2.0, -np.inf, -np.inf, -np.inf, -np.inf, -3.0], np.float32)
    ids = np.array([2, 5, 7, P, P, P, P, 9], np.uint32)
    d = LO.compute_top(lp, ids, 2, 10)
    assert list(d.items()) == [(5, -0.5), (2, np.float32(-1.2)), (9, -3.0)], d
    # the sampled token already among the top: its entry takes the last column's value
    ids2 = ids.copy()
    ids2[7] = 2
    d = LO.compute_top(lp, ids2, 3, 10)
    assert list(d.items()) == [(5, -0.5), (2, -3.0), (7, -2.0)], d
    # a sampled token outside the kept top_n is appended after them
    d = LO.compute_top(lp, np.array([2, 5, 7, P, P, P, P, 7], np.uint32), 1, 10)
    assert list(d.items()) == [(5, -0.5), (7, -3.0)], d
    # ids >= vocab are padding even when not the pad id
    d = LO.compute_top(lp, np.array([2, 10, 7, P, P, P, P, 9], np.uint32), 7, 10)
    assert list(d.keys()) == [2, 7, 9], d
    # a top_n = 0 request is None; token log-probabilities are the last column
    out_lp = np.stack([lp, lp, lp])
    out_ids = np.stack([ids, ids, ids])
    res = LO.assemble(out_lp, out_ids, np.array([0, 2, 3], np.uint32), [2, 0], 10)
    assert res[1] is None
    tlp, tops = res[0]
    assert tlp == [-3.0, -3.0] and len(tops) == 2
    for bad, code in ((-1, "LP_ERR_TOP_N_NEGATIVE"), (8, "LP_ERR_TOP_N_TOO_LARGE")):
        try:
            LO.compute_top(lp, ids, bad, 10)
        except LO.OracleError as e:
            assert e.code == code
        else:
            raise AssertionError(f"top_n {bad} accepted")


def pin_assembly_worked_example():
    """The SGLang page's printed response (section "logprob 的数值形态"):
    with each position's printed pair in its top columns and the printed
    token as the chosen one, the assembled result is the printed
    token_logprobs list and top_logprobs dicts (token names mapped to ids)."""
    with open(os.path.join(GOLDEN, "sglang_worked_example.json"), encoding="utf-8") as f:
        g = json.load(f)
    names = sorted({t for pos in g["top_logprobs"] for t, _ in pos} | set(g["tokens"]))
    tid = {t: i for i, t in enumerate(names)}
    P = LO.PAD_ID
    rows_lp, rows_id = [], []
    for pos, tok in enumerate(g["tokens"]):
        (t1, a), (t2, b) = g["top_logprobs"][pos]
        rows_lp.append([a, b] + [-np.inf] * 5 + [g["token_logprobs"][pos]])
        rows_id.append([tid[t1], tid[t2]] + [P] * 5 + [tid[tok]])
    out_lp = np.array(rows_lp, np.float32)
    out_ids = np.array(rows_id, np.uint32)
    res = LO.assemble(out_lp, out_ids, np.array([0, 3], np.uint32), [2], len(names))
    tlp, tops = res[0]
    assert np.allclose(tlp, g["token_logprobs"], atol=1e-6)
    for pos in range(3):
        want = {tid[t]: v for t, v in g["top_logprobs"][pos]}
        assert list(tops[pos].keys()) == list(want.keys()), (pos, tops[pos], want)
        assert all(abs(tops[pos][k] - want[k]) < 1e-6 for k in want)


# ------------------------------------------------------------------ temperature

def pin_temperature():
    """log_softmax(x / T): closed forms, a 50-digit brute force, the ranking
    untouched by T, and the rejected temperatures."""
    # two tokens apart by d: the lower one has -log(1 + e^(d/T)) at temperature T
    for d, T in ((1.0, 0.5), (3.0, 2.0), (0.25, 0.1), (5.0, 1.0)):
        x = np.array([0.0, -d], np.float32)
        lp, _ = LO.log_softmax_f64(x, T)
        assert abs(lp[1] - (-math.log1p(math.exp(d / T)))) < 1e-12, (d, T, lp)
        assert abs(lp[0] - (-math.log1p(math.exp(-d / T)))) < 1e-12, (d, T, lp)
    # uniform rows stay uniform at any temperature
    for T in (0.3, 4.0):
        lp, _ = LO.log_softmax_f64(np.full(1000, 2.5, np.float32), T)
        assert np.allclose(lp, -math.log(1000), atol=1e-12)
    # k tied maxima near the top of the float32 range, the rest far below:
    # each tie has p = 1/k exactly, so log p = -ln k at any T, however large
    # x / T gets (a log-sum added to a huge maximum would round ln k away)
    big = np.float32(3.0e38)
    for k in (2, 5, 64):
        x = np.concatenate([np.full(k, big, np.float32),
                            np.array([0.0, -big, 1e-45], np.float32)])
        for T in (0.01, 1.0, 100.0):
            lp, _ = LO.log_softmax_f64(x, T)
            assert np.all(np.abs(lp[:k] + math.log(k)) < 1e-12), (k, T, lp[:k])
            lo = LO.compute_row(x, k, 7, 8, T)[0]
            assert np.all(lo[:min(k, 7)] == np.float32(-math.log(k))), (k, T, lo)
            # the zero logit sits 3e38 / T below the ties
            with np.errstate(over="ignore"):          # -3e40 rounds to -inf
                want = np.float32(-3.0e38 / T - math.log(k))
            assert lo[7] == want, (k, T, lo[7])
    # brute force at 50 digits on x / T
    rng = np.random.default_rng(17)
    for T in (0.2, 0.7, 3.0):
        xs = (rng.standard_normal(9) * 3).astype(np.float32)
        want, _ = mp_logprobs([float(v) / T for v in xs])
        lp, _ = LO.log_softmax_f64(xs, T)
        assert max(abs(float(a) - float(b)) for a, b in zip(lp, want)) < 1e-12, T
    # the ids and the row layout do not depend on T; the values are the
    # float32 rounding of log_softmax(x / T)
    x = (rng.integers(-4, 5, 200) / 2).astype(np.float32)
    base_lp, base_id = LO.compute_row(x, 3, 7, 8)
    for T in (0.05, 0.5, 9.0):
        lp, ids = LO.compute_row(x, 3, 7, 8, T)
        assert ids.tolist() == base_id.tolist() == brute_top_ids([float(v) for v in x], 7) + [3]
        z = x.astype(np.float64) / T
        ref = z - (z.max() + math.log(np.exp(z - z.max()).sum()))
        assert np.allclose(lp[:7], ref[ids[:7]].astype(np.float32), atol=1e-6)
    # accepted: [2^-126, 2^120]
    for good in (2.0 ** -126, 2.0 ** 120, 1e-30, 1e30):
        assert LO.check_temperature(good) == float(np.float32(good))
    for bad in (0.0, -1.0, float("inf"), float("nan"), 1e-45, 2.0 ** -127, 3.5e-39,
                2.0 ** 121, 2.0 ** 126, 3.0e38):
        try:
            LO.check_temperature(bad)
        except LO.OracleError as e:
            assert e.code == "LP_ERR_TEMPERATURE"
        else:
            raise AssertionError(f"temperature {bad} accepted")


# ------------------------------------------------------------------ top-k front end

def pin_top_k():
    """The top-k front end (the FlashInfer page's TopK on logits, then
    Softmax): hand closed forms, boundary ties, a 50-digit brute force over
    the kept set, reductions to the untruncated row, and the rejected k."""
    pad = LO.PAD_ID
    # x = (1, 2, 3), k = 2: ids 2 and 1 are kept; log p = -log(1 + e^-1) and
    # -log(1 + e); id 0 is dropped (-inf)
    x = np.array([1.0, 2.0, 3.0], np.float32)
    a, b = -math.log1p(math.exp(-1.0)), -math.log1p(math.e)
    lp, ids = LO.compute_row(x, 0, 7, 8, 1.0, 2)
    assert ids.tolist() == [2, 1] + [pad] * 5 + [0], ids
    assert abs(lp[0] - a) < 1e-6 and abs(lp[1] - b) < 1e-6 and lp[7] == -np.inf, lp
    assert np.all(lp[2:7] == -np.inf)
    lp, ids = LO.compute_row(x, 1, 1, 8, 1.0, 2)       # top_n 1 lists one; chosen kept
    assert ids.tolist() == [2] + [pad] * 6 + [1] and abs(lp[7] - b) < 1e-6, (lp, ids)
    # at temperature 2 the kept pair differs by 1/2
    lp, _ = LO.compute_row(x, 2, 7, 8, 2.0, 2)
    assert abs(lp[0] + math.log1p(math.exp(-0.5))) < 1e-6, lp
    assert abs(lp[7] + math.log1p(math.exp(-0.5))) < 1e-6, lp
    # k = 1: the top token has log p = 0; anything else is -inf
    lp, ids = LO.compute_row(np.array([0.3, 5.0, -2.0, 5.0], np.float32), 3, 7, 8, 1.0, 1)
    assert ids[0] == 1 and lp[0] == 0.0 and lp[7] == -np.inf and ids[7] == 3, (lp, ids)
    # boundary ties: of three equal maxima, k = 2 keeps ids 0 and 1 (R23)
    lp, ids = LO.compute_row(np.array([1.0, 1.0, 1.0, 0.0], np.float32), 2, 7, 8, 1.0, 2)
    assert ids[:3].tolist() == [0, 1, pad], ids
    assert abs(lp[0] + math.log(2.0)) < 1e-6 and abs(lp[1] + math.log(2.0)) < 1e-6
    assert lp[7] == -np.inf
    # a kept -inf token keeps log p = -inf
    lp, ids = LO.compute_row(np.array([0.0, -np.inf, -np.inf], np.float32), 1, 7, 8, 1.0, 2)
    assert ids[:2].tolist() == [0, 1] and lp[0] == 0.0 and lp[1] == -np.inf and lp[7] == -np.inf
    # brute force at 50 digits over the kept values / T
    rng = np.random.default_rng(23)
    for trial in range(12):
        n = int(rng.integers(3, 40))
        xs = (rng.standard_normal(n) * 2).astype(np.float32)
        k = int(rng.integers(1, 8))
        T = float(rng.choice([0.5, 1.0, 1.7]))
        kept = brute_top_ids([float(v) for v in xs], k)
        want, _ = mp_logprobs([float(xs[i]) / T for i in kept])
        chosen = int(rng.integers(0, n))
        lp, ids = LO.compute_row(xs, chosen, 7, 8, T, k)
        listed = kept[:7]
        assert ids[: len(listed)].tolist() == listed, (trial, ids, kept)
        for j in range(len(listed)):
            assert abs(float(lp[j]) - float(want[j])) < 1e-6, (trial, j)
        if chosen in kept:
            assert abs(float(lp[7]) - float(want[kept.index(chosen)])) < 1e-6, trial
        else:
            assert lp[7] == -np.inf, trial
        # the kept probabilities sum to one
        assert abs(sum(math.exp(float(w)) for w in want) - 1.0) < 1e-12
    # k at or beyond V keeps every token: the untruncated row
    xs = np.array([0.5, -1.0, 2.0, 0.0, 1.5], np.float32)
    for k in (5, 7):
        got = LO.compute_row(xs, 4, 7, 8, 1.0, k)
        ref = LO.compute_row(xs, 4, 7, 8, 1.0, 0)
        assert np.array_equal(got[1], ref[1]) and np.allclose(got[0], ref[0], atol=1e-7), k
    # through the batch entry: one k per request, 0 = none
    off = np.array([0, 1, 3], np.uint32)
    logits = np.array([[1, 2, 3], [3, 2, 1], [0, 0, 5]], np.float32)
    lp, ids, _ = LO.compute_log_probabilities_ragged(
        off, logits, logits[[0, 2]], np.array([0, 1, 0], np.uint32), np.array([0, 2], np.uint32),
        [7, 7], [False, True], batch_top_k=[2, 0])
    assert ids[0, :3].tolist() == [2, 1, pad] and abs(lp[0, 0] - a) < 1e-6 and lp[0, 7] == -np.inf
    assert ids[1, :3].tolist() == [0, 1, 2] and ids[2, 0] == 2     # request 1 is untruncated
    for bad, cols in ((8, 8), (-1, 8), (2, 2)):
        try:
            LO.check_top_k(bad, cols)
        except LO.OracleError as e:
            assert e.code == "LP_ERR_TOP_K"
        else:
            raise AssertionError(f"top_k {bad} accepted with {cols} columns")
