"""CPU oracle for the SAF hybrid attention layer: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import this
package. The HIP library never calls it and shares no code with it. Each function is
pinned by the CPU tests (closed forms, invariants, finite differences, brute force);
none of them is "parity unpinned". compact_fit holds the fit of Eq. (3) to a target
pattern (its own pins: tests/oracle_pins_fit.py).
"""
from .saf_oracle import (attn_bwd, attn_fwd, causal_mask, dynamic_probs, frozen_probs,  # noqa: F401
                         kl_score, kl_score_of, mean_attention, n_selected, rank_heads,
                         reconstruction_risk, select_heads, sharp_mean, var_score, variance_score)
