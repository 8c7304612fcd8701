"""CPU oracle for the paged decode path.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python
binding) never calls it and never falls back to it.

It is a plain, slow, obviously correct implementation in float64 of what the
path computes, written from the pages:

* "PagedAttention and KV memory management", section "The kernel side":
  attention over paged KV reads the sequence's block table, then each
  physical block's K and V tiles, and produces the scores and the weighted
  values of ordinary attention over the sequence.  Paging changes where the
  tokens live, not the result, so the oracle gathers each sequence's logical
  K/V through its table and computes exact softmax attention.
* "How does vLLM PagedAttention manage Virtual Memory Pages ...", sections
  "Key Technical Innovations" (item 2, one block of e.g. 16 tokens taken at
  a time as generation proceeds) and "Example" (the new token goes into the
  sequence's current block): the slot write.

Readings where the pages are silent (shared with the HIP side only as a
written convention, never as code):
  * k_cache [NB, Hkv, bs, D]; slot = block*bs + offset.  v_cache is
    feature-major in sub-tiles of T tokens (T = 16 when 16 divides bs, else
    T = bs): v_cache [NB, Hkv, (bs/T)*D, T], and token o's feature d sits at
    [block, head, (o // T)*D + d, o % T].  With bs <= 16 that is plainly
    [NB, Hkv, D, bs].
  * Scores are scale * q.k over positions 0 .. L-1 (one query at the last
    position, so no causal mask is needed); no bias of any kind.
  * Query head h reads KV head h // (Hq // Hkv).
  * A negative slot means "write nothing"; L = 0 gives an all-zero output.
  * bf16 values are widened exactly: the 16 stored bits become the top half
    of an IEEE fp32 word.

This module imports NumPy only.
"""
from __future__ import annotations

import numpy as np


def widen(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Stored KV/q elements -> float64, exactly.

    bf16 is held as raw uint16 bits; placing them in the high half of a
    32-bit word yields the identical fp32 value, which widens exactly.
    """
    if kv_dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 data must be raw uint16 bits")
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(kv_dtype)


def _raw_view(x: np.ndarray) -> np.ndarray:
    """Integer view of the storage so copies move bits, never values."""
    if x.dtype == np.float32:
        return x.view(np.uint32)
    if x.dtype == np.uint16:
        return x
    raise TypeError(x.dtype)


def v_tile_tokens(block_size):
    """Tokens per feature-major V sub-tile (a layout convention, see above)."""
    return 16 if block_size % 16 == 0 else block_size


def _v_tiles(v_cache, block_size):
    """The V pool as [NB, Hkv, bs/T, D, T] (a view: only the axes are split)."""
    T = v_tile_tokens(block_size)
    NB, Hkv, R, cols = v_cache.shape
    if cols != T or R % (block_size // T):
        raise ValueError(f"v_cache shape {v_cache.shape} does not fit block_size {block_size}")
    return v_cache.reshape(NB, Hkv, block_size // T, R // (block_size // T), T)


def write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, block_size):
    """Slot write: new token t's K/V go to slot_mapping[t] of the pool.

    Returns new arrays (the inputs are left untouched).  slot = block *
    block_size + offset; a negative slot is skipped.  The copy is of the raw
    element bits, so any value, NaN payloads included, arrives unchanged.
    """
    k_out = k_cache.copy()
    v_out = v_cache.copy()
    kr, vr = _raw_view(k_out), _v_tiles(_raw_view(v_out), block_size)
    knr, vnr = _raw_view(np.ascontiguousarray(k_new)), _raw_view(np.ascontiguousarray(v_new))
    T = v_tile_tokens(block_size)
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        b, o = divmod(slot, block_size)
        kr[b, :, o, :] = knr[t]              # K tile keeps a token's features together
        vr[b, :, o // T, :, o % T] = vnr[t]  # V sub-tile keeps a feature's tokens together
    return k_out, v_out


def gather_sequence(k_cache, v_cache, table_row, L, block_size, kv_dtype):
    """Logical K and V of one sequence, read through its block table.

    Position p lives in physical block table_row[p // bs] at offset p % bs.
    Returns float64 arrays K [Hkv, L, D] and V [Hkv, L, D].
    """
    pos = np.arange(L)
    blocks = np.asarray(table_row)[pos // block_size].astype(np.int64)
    offs = pos % block_size
    T = v_tile_tokens(block_size)
    K = k_cache[blocks, :, offs, :]                                  # [L, Hkv, D]
    V = _v_tiles(v_cache, block_size)[blocks, :, offs // T, :, offs % T]  # [L, Hkv, D]
    K = widen(K, kv_dtype).transpose(1, 0, 2)
    V = widen(V, kv_dtype).transpose(1, 0, 2)
    return K, V


def attention_one(q_vec, K, V, scale):
    """softmax(scale * K q) V for one query vector; fp64, exact two-pass softmax."""
    x = scale * (K @ q_vec)
    x = x - x.max()
    p = np.exp(x)
    return (p @ V) / p.sum()


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, kv_dtype):
    """Single-query decode attention over the paged pool; returns float64 [S, Hq, D].

    scale is used at the exact value the GPU receives (an fp32 number),
    widened to float64.
    """
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    qd = widen(q, kv_dtype)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        if L == 0:
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], L, block_size, kv_dtype)
        for h in range(Hq):
            kv = h // G
            out[s, h] = attention_one(qd[s, h], K[kv], V[kv], sc)
    return out


# --------------------------------------------------------------------------
# Split-context form: partial softmax states over token ranges and their
# log-sum-exp merge.  The pages do not describe long-context splitting; the
# HIP path splits long sequences across workgroups and combines the pieces
# with this merge, so the identity "merge of the pieces == unsplit result"
# is checked on these float64 definitions.
# --------------------------------------------------------------------------

def partial_state(q_vec, K, V, scale, lo, hi):
    """(m, l, acc) of positions lo .. hi-1: max score, sum of exp(x - m), sum of exp(x - m) v."""
    x = scale * (K[lo:hi] @ q_vec)
    m = x.max()
    p = np.exp(x - m)
    return m, p.sum(), p @ V[lo:hi]


def merge_states(states):
    """Combine partial states in the given order: rescale each to the common max, then sum."""
    M = max(m for m, _, _ in states)
    lam = sum(l * np.exp(m - M) for m, l, _ in states)
    acc = sum(a * np.exp(m - M) for m, _, a in states)
    return acc / lam
