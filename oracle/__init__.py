"""CPU oracle (float64, NumPy) for the paged decode path.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.
"""
from .paged_attention import (attention_one, decode, gather_sequence, merge_states,
                              partial_state, widen, write_kv)

__all__ = ["attention_one", "decode", "gather_sequence", "merge_states", "partial_state",
           "widen", "write_kv"]
