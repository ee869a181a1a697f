"""CPU oracle for FLCE (test infrastructure only; see flce_oracle.py)."""
from .flce_oracle import (widen, logits, row_logsumexp, row_losses, dlogits, flce, flce_blocked,  # noqa: F401
                          flce_rows, flce_sparse_weight, flce_ext, rmsnorm, rmsnorm_backward, rmsnorm_flce,
                          logits_bytes)
