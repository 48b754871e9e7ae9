"""CPU oracle (test infrastructure): see verify_oracle.py."""
from .verify_oracle import (  # noqa: F401
    ancestors_or_self, attend, bf16_bits_to_f64, gather_rows, merge_partials,
    prefix_partial, tree_partial, verify, visibility,
)
