"""ragged_token_log_amd: ragged batched token log-probabilities on MI355X.

The computation lives in ``liblogprob.so`` (C ABI in ``include/liblogprob.h``,
HIP kernels for gfx950); this package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    COLUMNS, EXPORTED, LEVELS, LIB_PATH, MAX_LEVELS, MAX_TOP_N, PAD_ID, LogProbabilities,
    LogprobError, Plan, alloc_outputs, compute_log_probabilities_ragged, load,
    log_probabilities_ragged, status_string,
)
