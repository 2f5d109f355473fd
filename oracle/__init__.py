"""Float64 CPU oracles (test infrastructure only; see oracle.py and channelizer.py)."""
from .channelizer import pfb_channelize, pfb_parity_bound, pfb_state_next
from .oracle import (build, fir_direct, fir_direct_multi, fir_ols_blocks,
                     parity_bound, state_next)

__all__ = ["build", "fir_direct", "fir_direct_multi", "fir_ols_blocks",
           "parity_bound", "state_next", "pfb_channelize", "pfb_parity_bound",
           "pfb_state_next"]
