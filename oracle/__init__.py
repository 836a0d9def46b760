"""fp64 CPU oracle for varlen FlashAttention forward/backward and decode attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py, never by the product library.  It shares no code
with the HIP path.  Parity status of each function is recorded in the design
notes; every function here is pinned by CPU tests against closed forms,
library routines or finite differences, except the two conventions the pages
leave open (keep-mask bit order, band alignment when Lq != Lkv), which are
"parity unpinned" by the pages and only checked for self-consistency.
"""
from .attention import (INT_MAX_TOKENS, allowed, alibi_pse, keep_bits, forward, backward,
                        probabilities, pse_block, sequence_mode)
from .decode import cache_as_bsnd, decode

__all__ = ["INT_MAX_TOKENS", "allowed", "alibi_pse", "keep_bits", "forward", "backward", "probabilities",
           "pse_block", "sequence_mode", "cache_as_bsnd", "decode"]
