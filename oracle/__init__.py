"""CPU oracle for ragged paged attention -- test infrastructure only (see rpa_oracle)."""
from .rpa_oracle import (as_f64, forward, forward_inputs, forward_rows, sequence_probs,
                         softmax_rows, unpage, visible)

__all__ = ["as_f64", "forward", "forward_inputs", "forward_rows", "sequence_probs",
           "softmax_rows", "unpage", "visible"]
