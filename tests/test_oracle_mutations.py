"""Planted mistakes in the CPU oracle must each fail at least one pin.

Each mutant below replaces one oracle function with a plausible slip (a wrong
sign, index, tie rule or dropped term).  The test passes only if running the
pins against the mutated oracle raises AssertionError, i.e. the pins are
strong enough to catch that class of mistake.  Everything runs on the CPU.
"""
import numpy as np
import pytest

import oracle.logprob_oracle as LO
import tests.oracle_pins as P

_orig = {name: getattr(LO, name) for name in (
    "rank_descending", "log_softmax_f64", "row_tasks", "output_counts_and_offsets",
    "compute_row", "kernel_row_offsets")}


def _rank_ties_high_id_first(row_f32):
    x = np.asarray(row_f32, dtype=np.float32).astype(np.float64)
    x = np.where(x == 0, 0.0, x)
    n = x.shape[0]
    return np.lexsort((-np.arange(n), -x))


def _rank_negzero_below_poszero(row_f32):
    x = np.asarray(row_f32, dtype=np.float32).astype(np.float64)
    key = np.where((x == 0) & np.signbit(x), -1e-300, x)
    return np.argsort(-key, kind="stable")


def _lsm_no_shift(row, temperature=1.0):
    x = np.asarray(row, dtype=np.float64) / temperature
    with np.errstate(invalid="ignore", over="ignore"):
        lse = np.log(np.sum(np.exp(x)))
        return x - lse, float(lse)


def _lsm_wrong_sign(row, temperature=1.0):
    lp, lse = _orig["log_softmax_f64"](row, temperature)
    return -lp, lse


def _lsm_dropped_max(row, temperature=1.0):
    x = np.asarray(row, dtype=np.float64) / temperature
    m = np.max(x)
    with np.errstate(invalid="ignore"):
        lse = np.log(np.sum(np.exp(x - m)))
        return x - lse, float(lse)


def _lsm_sum_added_to_max(row, temperature=1.0):
    # the same log-softmax with the log-sum added to the maximum before the
    # subtraction: exact on paper, but ln k vanishes beside a maximum of 3e40
    x = np.asarray(row, dtype=np.float64) / temperature
    m = np.max(x)
    with np.errstate(invalid="ignore"):
        lse = m + np.log(np.sum(np.exp(x - m)))
        return x - lse, float(lse)


def _tasks_chosen_same_position(off, echo, top_n, tokens, sampled, has_logits):
    tasks = _orig["row_tasks"](off, echo, top_n, tokens, sampled, has_logits)
    out, o = [], 0
    counts, _ = _orig["output_counts_and_offsets"](off, echo)
    for n, c in enumerate(counts):
        length = int(off[n + 1] - off[n])
        for k in range(int(c)):
            p = length - int(c) + k
            t = tasks[o]
            out.append(LO.RowTask(t.src_row, int(tokens[int(off[n]) + p]), t.top_n))
            o += 1
    return out


def _tasks_first_rows(off, echo, top_n, tokens, sampled, has_logits):
    tasks = _orig["row_tasks"](off, echo, top_n, tokens, sampled, has_logits)
    counts, _ = _orig["output_counts_and_offsets"](off, echo)
    koff = _orig["kernel_row_offsets"](off, has_logits)
    out, o = [], 0
    for n, c in enumerate(counts):
        for k in range(int(c)):
            t = tasks[o]
            out.append(LO.RowTask(int(koff[n]) + k, t.chosen, t.top_n))
            o += 1
    return out


def _counts_swapped(off, echo):
    return _orig["output_counts_and_offsets"](off, [not bool(e) for e in echo])


def _row_pad_zero(row, chosen, top_n, cols, temperature=1.0, top_k=0):
    lp, ids = _orig["compute_row"](row, chosen, top_n, cols, temperature, top_k)
    ids = ids.copy()
    ids[ids == LO.PAD_ID] = 0
    return lp, ids


def _row_last_col_top1(row, chosen, top_n, cols, temperature=1.0, top_k=0):
    lp, ids = _orig["compute_row"](row, chosen, top_n, cols, temperature, top_k)
    if top_n > 0:
        lp = lp.copy()
        lp[cols - 1] = lp[0]
    return lp, ids


def _row_ignores_top_n(row, chosen, top_n, cols, temperature=1.0, top_k=0):
    return _orig["compute_row"](row, chosen, 7 if top_n > 0 else 0, cols, temperature, top_k)


def _row_topk_ignored(row, chosen, top_n, cols, temperature=1.0, top_k=0):
    return _orig["compute_row"](row, chosen, top_n, cols, temperature, 0)


def _row_topk_no_renormalise(row, chosen, top_n, cols, temperature=1.0, top_k=0):
    # plausible slip: mask the dropped tokens but keep the full-row softmax
    lp, ids = _orig["compute_row"](row, chosen, top_n, cols, temperature, 0)
    if top_k > 0 and top_n > 0:
        lp, ids = lp.copy(), ids.copy()
        lp[top_k:cols - 1] = -np.inf
        ids[top_k:cols - 1] = LO.PAD_ID
        if chosen not in _orig["rank_descending"](row)[:top_k]:
            lp[cols - 1] = -np.inf
    return lp, ids


def _row_topk_one_more(row, chosen, top_n, cols, temperature=1.0, top_k=0):
    return _orig["compute_row"](row, chosen, top_n, cols, temperature, top_k + 1 if top_k else 0)


def _row_topk_chosen_unmasked(row, chosen, top_n, cols, temperature=1.0, top_k=0):
    # plausible slip: a dropped chosen token still gets x/T - lse(kept)
    lp, ids = _orig["compute_row"](row, chosen, top_n, cols, temperature, top_k)
    if top_k > 0 and top_n > 0 and lp[cols - 1] == -np.inf:
        x = np.asarray(row, np.float64) / temperature
        kept = _orig["rank_descending"](row)[:top_k]
        m = np.max(x[kept])
        lp = lp.copy()
        with np.errstate(invalid="ignore"):
            lp[cols - 1] = np.float32(x[chosen] - (m + np.log(np.sum(np.exp(x[kept] - m)))))
    return lp, ids


def _top_no_overwrite(lp_row, id_row, top_n, vocab):
    # plausible slip: the sampled token only added when absent (no overwrite)
    cols = len(id_row)
    pairs = [(int(t), float(v)) for t, v in zip(id_row[: cols - 1], lp_row[: cols - 1])
             if int(t) < vocab]
    out = dict(sorted(pairs, key=lambda p: p[1], reverse=True)[:top_n])
    out.setdefault(int(id_row[cols - 1]), float(lp_row[cols - 1]))
    return out


def _top_truncate_before_sort(lp_row, id_row, top_n, vocab):
    cols = len(id_row)
    pairs = [(int(t), float(v)) for t, v in zip(id_row[: cols - 1], lp_row[: cols - 1])
             if int(t) < vocab][:top_n]
    out = dict(sorted(pairs, key=lambda p: p[1], reverse=True))
    out[int(id_row[cols - 1])] = float(lp_row[cols - 1])
    return out


def _lsm_temperature_multiplies(row, temperature=1.0):
    x = np.asarray(row, dtype=np.float64) * np.float64(temperature)
    m = np.max(x)
    with np.errstate(invalid="ignore"):
        lse = m + np.log(np.sum(np.exp(x - m)))
        return x - lse, float(lse)


def _cap_equals_columns(levels):
    # plausible slip: forgetting the column reserved for the chosen token
    return 2 ** levels if levels > 0 else 1


def _columns_two_to_levels_plus_one(levels):
    return 2 ** (levels + 1) if levels > 0 else 1


MUTANTS = {
    "temperature_multiplies": ("log_softmax_f64", _lsm_temperature_multiplies),
    "top_no_overwrite": ("compute_top", _top_no_overwrite),
    "top_truncate_before_sort": ("compute_top", _top_truncate_before_sort),
    "cap_equals_columns": ("max_top_n", _cap_equals_columns),
    "columns_off_by_level": ("columns_for_levels", _columns_two_to_levels_plus_one),
    "ties_high_id_first": ("rank_descending", _rank_ties_high_id_first),
    "negzero_ranks_low": ("rank_descending", _rank_negzero_below_poszero),
    "lse_no_shift": ("log_softmax_f64", _lsm_no_shift),
    "logprob_sign": ("log_softmax_f64", _lsm_wrong_sign),
    "lse_dropped_max": ("log_softmax_f64", _lsm_dropped_max),
    "lse_sum_added_to_max": ("log_softmax_f64", _lsm_sum_added_to_max),
    "chosen_same_position": ("row_tasks", _tasks_chosen_same_position),
    "echo_first_rows": ("row_tasks", _tasks_first_rows),
    "counts_swapped": ("output_counts_and_offsets", _counts_swapped),
    "pad_id_zero": ("compute_row", _row_pad_zero),
    "chosen_col_is_top1": ("compute_row", _row_last_col_top1),
    "top_n_ignored": ("compute_row", _row_ignores_top_n),
    "topk_ignored": ("compute_row", _row_topk_ignored),
    "topk_no_renormalise": ("compute_row", _row_topk_no_renormalise),
    "topk_one_more": ("compute_row", _row_topk_one_more),
    "topk_chosen_unmasked": ("compute_row", _row_topk_chosen_unmasked),
}


def _run_all_pins():
    rng = np.random.default_rng(3)
    P.pin_offsets_hand_example()
    P.pin_mapping_hand_example()
    P.pin_logsoftmax_bruteforce([[0.5, -1.0, 3.0], [2.0]])
    P.pin_logsoftmax_closed_forms()
    P.pin_logsoftmax_invariants([rng.standard_normal(300).astype(np.float32)])
    P.pin_worked_example()
    P.pin_ranking_exhaustive([-np.inf, 0.0, 1.0], 4)
    P.pin_ranking_exhaustive([-0.0, 0.0, 1.0], 4)
    P.pin_ranking_special_cases()
    P.pin_batch_hand_example()
    P.pin_errors()
    P.pin_levels_columns()
    P.pin_levels_bruteforce([rng.standard_normal(40).astype(np.float32)], levels_list=(1, 4))
    P.pin_levels_zero()
    P.pin_assembly_hand_examples()
    P.pin_assembly_worked_example()
    P.pin_temperature()
    P.pin_top_k()


def test_pins_pass_on_true_oracle():
    _run_all_pins()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(LO, attr, fn)
    with pytest.raises(AssertionError):
        _run_all_pins()
