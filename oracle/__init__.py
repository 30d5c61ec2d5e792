"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .logprob_oracle import (  # noqa: F401
    PAD_ID, DEFAULT_LEVELS, OracleError, RowTask, columns_for_levels, max_top_n,
    output_counts_and_offsets, kernel_row_offsets, validate, row_tasks,
    log_softmax_f64, rank_descending, compute_row, compute_log_probabilities_ragged,
)
