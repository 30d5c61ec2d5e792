"""Plain, slow CPU oracle for ragged batched token log-probabilities.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, table or constant generator with
the HIP library; the two meet only in the seeded input generators of ``gen/``.

Pages this follows (cited by title and section, nothing else):

[MAX]  "MAX Python SDK 中 log_probabilities 模块解析：ragged 批量 Token 对数概率的
        计算图构建与执行"  (the method: graph contract, host orchestration, top-k
        semantics, result assembly)
[SGL]  "logprob、finish reason 与 output processing"  (definition of a logprob,
        worked example, where prompt-token logprobs come from)
[FI]   the FlashInfer ``logits_processor`` page (its test tolerance only)

What it computes, for every selected logits row, is a result with a plain
definition, so the oracle is that definition written out:
  * log-softmax in float64 (NumPy pairwise sum), rounded once to float32;
  * an exact top-k: a full stable sort of the raw float32 logits in
    descending order (lowest token id first among equal values, -0.0 == +0.0);
  * a gather of the chosen token's log-probability into the last column.

Readings taken where the pages are silent or garbled (each also listed in the
design notes):
  R1  echo row k of a request predicts prompt token k+1; the request's last
      row predicts its sampled token; the first prompt token gets no row.
  R2  with full logits, a request uses the *last* ``count`` rows of its token
      range (a non-echo request: its last row).
  R4  ranking is on raw float32 logits, descending, lowest id first on ties.
  R5  columns at or beyond ``min(top_n, V)`` are padding (-inf, 0xFFFFFFFF).
  R6  rows of ``top_n == 0`` requests keep their output rows; all columns are
      padding and no logits are read.
  R8  -inf logits rank lowest (ties by id); their logprob is -inf.
  R9  an all -inf row has NaN logprobs (IEEE x - lse with lse = -inf).
  R10 NaN or +inf logits are outside the contract and rejected.
  R11 an empty request (L_n = 0) is an error.
  R23 a top-k front end (the FlashInfer page's TopK processor on logits, then
      Softmax) keeps exactly the k best tokens of the ranking (R4 order, so
      ties at the boundary go to the lowest ids); k = 0 keeps all.
  R24 with a top-k front end, log-probabilities are renormalised over the
      kept tokens (after the temperature); only kept tokens are listed.
  R25 a chosen token outside the kept set has log-probability -inf.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(brute force, closed forms, invariants, the worked example of [SGL]).  The
exact float32 bits of the GPU log-probabilities are not fixed by the pages;
they are compared at 1e-5 absolute.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

PAD_ID = 0xFFFFFFFF
DEFAULT_LEVELS = 3  # [MAX] §图支持的最大 top-n: the default heap depth


class OracleError(ValueError):
    """A call the pages (or a stated reading) make invalid.

    ``code`` carries the name of the matching library status, so a test can
    check both sides reject the same call for the same reason.
    """

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


def columns_for_levels(levels: int) -> int:
    """Output columns per row.  [MAX] §log_probabilities_ragged_graph: a graph
    built with ``levels`` keeps 2**levels columns, or one when levels is 0."""
    if levels < 0:
        raise OracleError("LP_ERR_UNSUPPORTED", f"levels={levels} < 0")
    return 2 ** levels if levels > 0 else 1


def max_top_n(levels: int) -> int:
    """Largest servable top_n: one column is reserved for the chosen token,
    the rest hold the heap of capacity 2**levels - 1.  [MAX] §图支持的最大 top-n,
    §compute_top 的结果组装 (top_n above columns - 1 is rejected)."""
    return columns_for_levels(levels) - 1


def output_counts_and_offsets(input_row_offsets, batch_echo):
    """Echo-dependent output row counts and their offsets.

    [MAX] §ragged 数据编排：an echo request emits one row per input token, any
    other request exactly one; the output offsets are a leading zero followed
    by the running sum of the counts, all uint32.
    """
    off = np.asarray(input_row_offsets, dtype=np.int64)
    echo = [bool(e) for e in batch_echo]
    counts = np.array(
        [(off[i + 1] - off[i]) if e else 1 for i, e in enumerate(echo)],
        dtype=np.int64,
    )
    out_off = np.concatenate([np.zeros(1, dtype=np.int64), np.cumsum(counts)])
    if out_off[-1] >= 2 ** 32:
        raise OracleError("LP_ERR_SHAPE", "output rows do not fit uint32")
    return counts.astype(np.uint32), out_off.astype(np.uint32)


def kernel_row_offsets(input_row_offsets, has_logits: bool):
    """Row offsets into the logits the device op reads.

    [MAX] §ragged 数据编排: without full logits the op reads one
    next-token row per request and its row offsets are 0..batch; otherwise it
    reads the full logits with the input row offsets.
    """
    off = np.asarray(input_row_offsets, dtype=np.int64)
    if has_logits:
        return off.copy()
    return np.arange(off.shape[0], dtype=np.int64)


@dataclass(frozen=True)
class RowTask:
    """One output row: which logits row to read, the chosen token and top_n."""

    src_row: int
    chosen: int
    top_n: int


def validate(input_row_offsets, logits_shape, next_token_logits_shape, tokens,
             sampled_tokens, batch_top_n, batch_echo, levels=DEFAULT_LEVELS):
    """Argument checks.  [MAX] §compute_log_probabilities_ragged (entry
    assertions: 1-D offsets, 2-D logits, equal batch lengths, equal vocab),
    §compute_top 的结果组装 (top_n range), §echo 的前置条件 (echo needs full
    logits).  R11 and the token-range check are readings of our own."""
    off = np.asarray(input_row_offsets)
    if off.ndim != 1 or off.shape[0] < 1:
        raise OracleError("LP_ERR_SHAPE", "input_row_offsets must be 1-D, length batch+1")
    batch = off.shape[0] - 1
    if len(batch_top_n) != batch or len(batch_echo) != batch or len(sampled_tokens) != batch:
        raise OracleError("LP_ERR_SHAPE", "per-request arguments differ in length")
    offi = off.astype(np.int64)
    if offi[0] != 0 or np.any(np.diff(offi) <= 0):
        raise OracleError("LP_ERR_OFFSETS", "offsets must start at 0 and strictly increase")
    total = int(offi[-1])
    if len(next_token_logits_shape) != 2 or next_token_logits_shape[0] != batch:
        raise OracleError("LP_ERR_SHAPE", "next_token_logits must be (batch, vocab)")
    vocab = int(next_token_logits_shape[1])
    if vocab < 1:
        raise OracleError("LP_ERR_SHAPE", "vocab must be >= 1")
    if logits_shape is not None:
        if len(logits_shape) != 2 or logits_shape[0] != total:
            raise OracleError("LP_ERR_SHAPE", "logits must be (tokens, vocab)")
        if logits_shape[1] != vocab:
            raise OracleError("LP_ERR_SHAPE", "vocab of logits and next_token_logits differ")
    if len(tokens) != total:
        raise OracleError("LP_ERR_SHAPE", "tokens must hold input_row_offsets[-1] ids")
    cap = max_top_n(levels)
    for t in batch_top_n:
        if t < 0:
            raise OracleError("LP_ERR_TOP_N_NEGATIVE", f"top_n={t}")
        if t > cap:
            raise OracleError("LP_ERR_TOP_N_TOO_LARGE", f"top_n={t} > {cap}")
    if logits_shape is None and any(bool(e) for e in batch_echo):
        raise OracleError("LP_ERR_ECHO_NEEDS_LOGITS", "echo requires full logits")
    tok = np.asarray(tokens, dtype=np.int64)
    smp = np.asarray(sampled_tokens, dtype=np.int64)
    if (tok.size and (tok.min() < 0 or tok.max() >= vocab)) or \
            (smp.size and (smp.min() < 0 or smp.max() >= vocab)):
        raise OracleError("LP_ERR_TOKEN_RANGE", "token id outside [0, vocab)")
    return batch, vocab, total


def row_tasks(input_row_offsets, batch_echo, batch_top_n, tokens, sampled_tokens,
              has_logits: bool):
    """Per output row: source logits row, chosen token and top_n.

    Counts follow [MAX] §ragged 数据编排; the source rows and chosen tokens
    follow readings R1/R2, grounded in [SGL] §input logprob 和 output logprob
    来自哪里 (a prefill position's distribution is over the next token; a
    decode step reads the sampled token from the same logits) and in [MAX]
    §compute_top 的结果组装 (the last column is the sampled token's logprob).
    """
    off = np.asarray(input_row_offsets, dtype=np.int64)
    counts, _ = output_counts_and_offsets(off, batch_echo)
    koff = kernel_row_offsets(off, has_logits)
    tasks = []
    for n in range(len(counts)):
        c = int(counts[n])
        length = int(off[n + 1] - off[n])
        for k in range(c):
            src = int(koff[n + 1]) - c + k     # the last c rows of the range (R2)
            p = length - c + k                 # prompt position of this row
            if p + 1 < length:
                chosen = int(tokens[int(off[n]) + p + 1])   # next prompt token (R1)
            else:
                chosen = int(sampled_tokens[n])             # the sampled token
            tasks.append(RowTask(src, chosen, int(batch_top_n[n])))
    return tasks


def check_temperature(t) -> float:
    """A request's temperature (reading R19): positive, as the FlashInfer
    page's Temperature processor requires, and within [2^-126, 2^120].  There
    T, 1/T and log2(e)/T are normal fp32 numbers, and two logits whose
    difference exceeds the fp32 range (|x - y| > 3.4e38) differ by more than
    256 after the division, a weight below e^-256.  The bounds also reject
    NaN and infinities."""
    t = float(np.float32(t))
    if not (2.0 ** -126 <= t <= 2.0 ** 120):
        raise OracleError("LP_ERR_TEMPERATURE", f"temperature={t}")
    return t


def log_softmax_f64(row, temperature: float = 1.0) -> tuple[np.ndarray, float]:
    """log p = z - logsumexp(z), z = x / temperature, in float64.  [SGL]
    §logprob 的数值形态: a logprob is log of a probability in (0, 1], so it
    is <= 0; [SGL] §output 从 forward() 到响应对象的完整路径 and the FlashInfer
    page's Temperature processor: the softmax is of the logits divided by
    the temperature."""
    x = np.asarray(row, dtype=np.float64) / np.float64(temperature)
    m = np.max(x)
    with np.errstate(invalid="ignore"):
        d = x - m                           # exact for the max and its ties
        log_sum = np.log(np.sum(np.exp(d)))
        # (x - m) - log sum is log p with nothing absorbed into a huge m
        # (m + log sum would round log sum away once |m| passes ~1e16)
        return d - log_sum, float(m + log_sum)


def rank_descending(row_f32) -> np.ndarray:
    """Token ids ordered by raw float32 logit, largest first, lowest id first
    among equal values (-0.0 counts as +0.0).  Reading R4; [MAX]
    §compute_top 的结果组装 sorts (token, logit) pairs by logit, descending."""
    x = np.asarray(row_f32, dtype=np.float32)
    canon = np.where(x == 0, np.float32(0.0), x)
    return np.argsort(-canon.astype(np.float64), kind="stable")


def check_top_k(k, cols: int) -> int:
    """A request's top-k front end: 0 (none) up to the ranked slots
    (readings R23, R24)."""
    k = int(k)
    if k < 0 or k > cols - 1:
        raise OracleError("LP_ERR_TOP_K", f"top_k={k} outside [0, {cols - 1}]")
    return k


def compute_row(row_f32, chosen: int, top_n: int, cols: int, temperature: float = 1.0,
                top_k: int = 0):
    """One output row: ``cols - 1`` top slots (padded past min(top_n, V)) and
    the chosen token in the last slot.  [MAX] §log_probabilities_ragged_graph
    (lp_logits / lp_tokens) and §compute_top 的结果组装.  With ``top_k`` > 0,
    the FlashInfer page's TopK on logits and Softmax come first: the
    distribution is the softmax of the kept logits alone (R23-R25)."""
    lp_out = np.full(cols, -np.inf, dtype=np.float32)
    id_out = np.full(cols, PAD_ID, dtype=np.uint32)
    if top_n == 0:
        return lp_out, id_out                     # R6: nothing is read
    x = np.asarray(row_f32, dtype=np.float32)
    if np.any(np.isnan(x)) or np.any(np.isposinf(x)):
        raise OracleError("LP_ERR_UNSUPPORTED", "NaN or +inf logits (R10)")
    order = rank_descending(x)
    if top_k == 0:
        lp, _ = log_softmax_f64(x, temperature)
        listed = order
    else:
        kept = order[: min(top_k, x.shape[0])]
        lp = np.full(x.shape[0], -np.inf)
        lp[kept], _ = log_softmax_f64(x[kept], temperature)
        listed = kept
    take = listed[: min(top_n, x.shape[0], cols - 1)]
    with np.errstate(over="ignore"):      # beyond the fp32 range a logprob rounds to -inf
        for j, t in enumerate(take):
            lp_out[j] = np.float32(lp[t])
            id_out[j] = t
        lp_out[cols - 1] = np.float32(lp[chosen])
    id_out[cols - 1] = chosen
    return lp_out, id_out


def compute_log_probabilities_ragged(input_row_offsets, logits, next_token_logits,
                                     tokens, sampled_tokens, batch_top_n, batch_echo,
                                     levels=DEFAULT_LEVELS, rows=None, batch_temperature=None,
                                     batch_top_k=None):
    """The whole path for one batch.

    Arguments follow [MAX] §compute_log_probabilities_ragged：执行计算并组装结果.
    ``logits`` is (tokens, vocab) float32 or None (only when no request
    echoes); ``next_token_logits`` is (batch, vocab) float32.  Either may be
    any object whose rows index to 1-D float32 arrays (a NumPy array, or a
    lazy row source for very large inputs).

    Returns ``(out_lp (R, cols) float32, out_ids (R, cols) uint32,
    out_off (batch+1) uint32)``.  If ``rows`` is given, only those output rows
    are computed (the rest stay padding) -- used to check very large inputs
    row by row.  ``batch_top_k`` (one per request, 0 = none) adds the top-k
    front end of R23-R25.
    """
    has_logits = logits is not None
    lshape = tuple(logits.shape) if has_logits else None
    validate(input_row_offsets, lshape, tuple(next_token_logits.shape), tokens,
             sampled_tokens, batch_top_n, batch_echo, levels)
    cols = columns_for_levels(levels)
    _, out_off = output_counts_and_offsets(input_row_offsets, batch_echo)
    tasks = row_tasks(input_row_offsets, batch_echo, batch_top_n, tokens,
                      sampled_tokens, has_logits)
    src = logits if has_logits else next_token_logits
    n_out = len(tasks)
    batch = len(batch_top_n)
    if batch_temperature is None:
        temps = [1.0] * batch
    else:
        temps = [check_temperature(t) for t in batch_temperature]
        if len(temps) != batch:
            raise OracleError("LP_ERR_SHAPE", "one temperature per request")
    if batch_top_k is None:
        top_ks = [0] * batch
    else:
        top_ks = [check_top_k(k, cols) for k in batch_top_k]
        if len(top_ks) != batch:
            raise OracleError("LP_ERR_SHAPE", "one top_k per request")
    req = np.repeat(np.arange(batch), np.diff(out_off.astype(np.int64)))
    out_lp = np.full((n_out, cols), -np.inf, dtype=np.float32)
    out_ids = np.full((n_out, cols), PAD_ID, dtype=np.uint32)
    which = range(n_out) if rows is None else rows
    for o in which:
        t = tasks[o]
        row = src[t.src_row] if t.top_n > 0 else None
        out_lp[o], out_ids[o] = compute_row(row, t.chosen, t.top_n, cols, temps[req[o]],
                                            top_ks[req[o]])
    return out_lp, out_ids, out_off


# ------------------------------------------------------------------ host assembly

def compute_top(lp_row, id_row, top_n: int, vocab: int) -> dict:
    """One output row's top dict.  [MAX] §compute_top 的结果组装: drop the
    padding columns (token id >= vocab), sort the (token, logprob) pairs by
    logprob descending, keep top_n, then write the sampled token's entry
    from the row's last column into the dict, overwriting a duplicate key."""
    if top_n < 0:
        raise OracleError("LP_ERR_TOP_N_NEGATIVE", f"top_n={top_n}")
    cols = len(id_row)
    if top_n > cols - 1:
        raise OracleError("LP_ERR_TOP_N_TOO_LARGE", f"top_n={top_n} > {cols - 1}")
    pairs = [(int(t), float(v)) for t, v in zip(id_row[: cols - 1], lp_row[: cols - 1])
             if int(t) < vocab]
    pairs = sorted(pairs, key=lambda p: p[1], reverse=True)[:top_n]
    out = dict(pairs)
    out[int(id_row[cols - 1])] = float(lp_row[cols - 1])
    return out


def assemble(out_lp, out_ids, out_off, batch_top_n, vocab: int):
    """Per request: None when top_n == 0, else (token log-probabilities = the
    last column of each of its rows, top dicts per row).  [MAX]
    §compute_top 的结果组装 (the final paragraph: a LogProbabilities per
    batch item, None for top_n == 0)."""
    res = []
    for n, top_n in enumerate(batch_top_n):
        if int(top_n) == 0:
            res.append(None)
            continue
        rows = range(int(out_off[n]), int(out_off[n + 1]))
        cols = out_ids.shape[1]
        res.append(([float(out_lp[o, cols - 1]) for o in rows],
                    [compute_top(out_lp[o], out_ids[o], int(top_n), vocab) for o in rows]))
    return res
