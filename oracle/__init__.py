"""CPU oracle (float64, NumPy) for the paged decode path.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

paged_attention: slot write, decode attention, split/merge identities.
block_manager:   reference model of the block manager (free list, tables,
                 reference counts, copy-on-write, fork, swap), block copies,
                 waste measures.
"""
from .paged_attention import (attention_one, decode, gather_sequence, merge_states,
                              partial_state, widen, write_kv)

__all__ = ["attention_one", "decode", "gather_sequence", "merge_states", "partial_state",
           "widen", "write_kv"]
