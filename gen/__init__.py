"""Seeded synthetic input generators (random draws only, no method arithmetic)."""
from .configs import (  # noqa: F401
    Case, make_case, WORKLOADS, no_echo_next_token, ragged_echo_mix, decode_peaked,
    prefill_echo_large, tie_edge_stress, request_logits_host, request_rows_sample, host_logits,
    next_token_rows, device_logits,
)
