"""Float64 CPU oracle (test infrastructure only; see oracle.py)."""
from .oracle import (build, fir_direct, fir_direct_multi, fir_ols_blocks,
                     parity_bound, state_next)

__all__ = ["build", "fir_direct", "fir_direct_multi", "fir_ols_blocks",
           "parity_bound", "state_next"]
