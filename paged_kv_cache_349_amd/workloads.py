"""Seeded synthetic inputs for the paged decode path.

This module builds inputs only: a physical block pool, per-sequence block
tables, context lengths, the query, the new token's K/V and the slot each new
token is written to.  It holds none of the attention arithmetic (no scores, no
softmax, no weighted sums); both the CPU oracle's tests and the HIP path's
tests and benchmark consume what it returns, so nothing here may import
either of them.

The pool plays the role of the block manager described on the pages: KV
memory is split into fixed-size blocks and each sequence reaches its blocks
through a block table ("PagedAttention and KV memory management", intro and
"The kernel side"; "Paged Attention: OS-Inspired Memory Management for KV
Caches", "Key terms in this lesson": Block, Block table).  Blocks are taken
from a seeded random permutation of the pool, so consecutive logical blocks
sit at unrelated physical addresses, as in the block-mapping diagram of
"How does vLLM PagedAttention manage Virtual Memory Pages ...", section
"Detail" (logical block 0 -> physical 42, logical block 1 -> physical 105).

Cache layout (a boundary decision, the same on both sides of every test):
  k_cache [num_blocks, num_kv_heads, block_size, head_dim]
  v_cache [num_blocks, num_kv_heads, (block_size / T) * head_dim, T]
with T = 16 when 16 divides block_size, else T = block_size (`v_pool_shape`).
For one (block, kv head) both tiles are contiguous spans of
block_size * head_dim elements.  K keeps a token's head_dim values together;
V keeps a feature's T token values together, in sub-tiles of T tokens
(token o, feature d at row (o // T) * head_dim + d, column o % T).

Element storage: fp32 values are held as np.float32; bf16 values are held as
their raw 16-bit patterns in np.uint16 (NumPy has no bf16 type).  fp32 draws
are rounded to bf16 once, to nearest-even, here; both sides then read the
same bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

# Bit patterns used to poison memory that a correct kernel never reads:
# partially filled block tails, free blocks, and the new token's slot before
# the write.  Several NaN payloads so that a copy that canonicalises NaNs is
# caught by the bitwise pool comparison.
_BF16_NANS = np.array([0x7FC0, 0x7FC1, 0xFFC3, 0x7F81], dtype=np.uint16)
_F32_NANS = np.array([0x7FC00000, 0x7FC00001, 0xFFC00003, 0x7F800011],
                     dtype=np.uint32)

SEED_BASE = 3490


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns raw bits.

    Inputs here are finite normal draws, so no NaN/Inf special-casing is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def element_bytes(kv_dtype: str) -> int:
    return 4 if kv_dtype == F32 else 2


def _storage_dtype(kv_dtype: str):
    return np.float32 if kv_dtype == F32 else np.uint16


def _draw(rng: np.random.Generator, shape, kv_dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if kv_dtype == F32:
        return x
    return f32_to_bf16_bits(x)


@dataclasses.dataclass
class Workload:
    """One decode step's inputs.  Arrays are host NumPy arrays.

    k_cache / v_cache hold the pool *before* the slot write: positions
    0 .. L-2 of every sequence are filled, the slot of position L-1 holds
    poison until pa_write_kv copies k_new / v_new into it.  context_lens
    counts the token written in this step.
    """
    name: str
    kv_dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray   # int32 [S]
    block_tables: np.ndarray   # int32 [S, max_blocks], padding -1
    k_cache: np.ndarray        # [NB, Hkv, bs, D]
    v_cache: np.ndarray        # v_pool_shape(NB, Hkv, D, bs)
    q: np.ndarray              # [S, Hq, D]
    k_new: np.ndarray          # [S, Hkv, D]
    v_new: np.ndarray          # [S, Hkv, D]
    slot_mapping: np.ndarray   # int32 [S]; -1 = nothing to write
    scale: np.float32
    poison: str = "nan"
    # (physical block id, owner count) for blocks shared by several tables.
    shared_blocks: int = 0

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group_size(self) -> int:
        return self.num_heads // self.num_kv_heads

    def blocks_per_seq(self) -> np.ndarray:
        return (self.context_lens.astype(np.int64) + self.block_size - 1) // self.block_size

    def kv_bytes_logical(self) -> int:
        """Bytes of K and V that attention over every sequence reads (live tokens only)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * \
            self.head_dim * element_bytes(self.kv_dtype) * 2

    def kv_bytes_unique(self) -> int:
        """Bytes of K and V in distinct live positions (shared blocks counted once)."""
        seen = {}
        for s in range(self.num_seqs):
            L = int(self.context_lens[s])
            for j in range((L + self.block_size - 1) // self.block_size):
                b = int(self.block_tables[s, j])
                live = min(self.block_size, L - j * self.block_size)
                seen[b] = max(seen.get(b, 0), live)
        tokens = sum(seen.values())
        return tokens * self.num_kv_heads * self.head_dim * element_bytes(self.kv_dtype) * 2

    def small_bytes(self) -> int:
        """q, out (fp32) and live block-table entries per decode step."""
        e = element_bytes(self.kv_dtype)
        q = self.num_seqs * self.num_heads * self.head_dim * e
        out = self.num_seqs * self.num_heads * self.head_dim * 4
        tab = int(self.blocks_per_seq().sum()) * 4 + self.num_seqs * 4
        return q + out + tab

    def prefix_groups(self):
        """(group_starts [G+1], prefix_blocks [G]) of runs of consecutive
        sequences whose tables start with the same block, and the number of
        leading whole blocks every member of the run shares."""
        return shared_prefix_groups(self.block_tables, self.context_lens, self.block_size)

    def write_bytes(self) -> int:
        """Bytes one slot write reads plus writes (K and V of every new token)."""
        n = int((self.slot_mapping >= 0).sum())
        return 2 * 2 * n * self.num_kv_heads * self.head_dim * element_bytes(self.kv_dtype)


def shared_prefix_groups(tables: np.ndarray, lens: np.ndarray, block_size: int):
    """Runs of consecutive sequences that share leading blocks, for the
    shared-prefix decode: (group_starts [G+1], prefix_blocks [G]) int32.
    A run is a maximal set of consecutive sequences whose first table entry
    is the same block; its prefix is the common leading part of their tables,
    cut to the whole blocks inside every member's context."""
    S = len(lens)
    starts, pref = [0], []
    s = 0
    while s < S:
        e = s + 1
        nb0 = int(lens[s]) // block_size
        while e < S and nb0 > 0 and int(lens[e]) // block_size > 0 and \
                tables[e, 0] == tables[s, 0]:
            e += 1
        p = min(int(lens[i]) // block_size for i in range(s, e))
        for i in range(s + 1, e):
            same = tables[i, :p] == tables[s, :p]
            p = int(np.argmin(same)) if not same.all() else p
        pref.append(p if e - s > 1 else 0)
        starts.append(e)
        s = e
    return np.array(starts, np.int32), np.array(pref, np.int32)


def new_token_slot(table_row: np.ndarray, L: int, block_size: int) -> int:
    """Slot of the token at 0-indexed position L-1: physical block * block_size + offset.

    The block for a position is the table entry of its logical block number;
    a fresh block is opened whenever the 1-indexed length reaches
    1, bs+1, 2*bs+1, ... (the allocation trigger of the PagedKVCacheManager
    sketch in "How does vLLM PagedAttention ...", section "Example", read
    with the length counted after the append).
    """
    if L <= 0:
        return -1
    pos = L - 1
    return int(table_row[pos // block_size]) * block_size + pos % block_size


def v_pool_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int):
    """Shape of the V pool: feature-major sub-tiles of T tokens (layout above)."""
    T = 16 if block_size % 16 == 0 else block_size
    return (num_blocks, num_kv_heads, (block_size // T) * head_dim, T)


def _poison_fill(rng: np.random.Generator, k_cache, v_cache, live_mask, kv_dtype, poison):
    """Overwrite every (block, offset) slot that is not live with poison.

    live_mask: bool [NB, bs] -- True where a cached token lives.  For
    poison == "finite" the pool keeps its N(0,1) draws everywhere.
    """
    if poison == "finite":
        return
    if poison != "nan":
        raise ValueError(f"unknown poison {poison!r}")
    dead_b, dead_o = np.nonzero(~live_mask)
    if dead_b.size == 0:
        return
    nans = _BF16_NANS if kv_dtype == BF16 else _F32_NANS
    kview = k_cache if kv_dtype == BF16 else k_cache.view(np.uint32)
    vview = v_cache if kv_dtype == BF16 else v_cache.view(np.uint32)
    pick = nans[np.arange(dead_b.size) % nans.size]
    # K: [NB, Hkv, bs, D] -> slot (b, :, o, :);  V sub-tiles -> (b, :, o // T, :, o % T)
    NB, Hkv, R, T = vview.shape
    bs = kview.shape[2]
    vtiles = vview.reshape(NB, Hkv, bs // T, R // (bs // T), T)
    kview[dead_b, :, dead_o, :] = pick[:, None, None]
    vtiles[dead_b, :, dead_o // T, :, dead_o % T] = pick[:, None, None]


def build_workload(name: str, rng: np.random.Generator, *, kv_dtype: str, context_lens,
                   num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                   num_blocks: Optional[int] = None, pool_factor: float = 1.25,
                   shared_prefix_groups: Optional[List[List[int]]] = None,
                   shared_prefix_blocks: int = 0, poison: str = "nan",
                   scale: Optional[float] = None) -> Workload:
    """Assemble a paged workload from already drawn context lengths.

    Draw order after the lengths: physical permutation, pool K, pool V, q,
    k_new, v_new.  Logical blocks take perm[0], perm[1], ... in allocation
    order: shared prompt blocks first (group-major), then each sequence's own
    blocks (sequence-major, logical-block-minor).
    """
    lens = np.asarray(context_lens, dtype=np.int64)
    S = int(lens.size)
    bs = block_size
    nblk = (lens + bs - 1) // bs
    groups = shared_prefix_groups or []
    owner = {}
    for gi, members in enumerate(groups):
        for s in members:
            owner[s] = gi
    shared_total = len(groups) * shared_prefix_blocks
    needed = shared_total + int(sum(int(nblk[s]) - (shared_prefix_blocks if s in owner else 0)
                                    for s in range(S)))
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * needed))
    if num_blocks < needed:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {needed}")
    max_blocks = max(1, int(nblk.max()) if S else 1)

    perm = rng.permutation(num_blocks).astype(np.int32)
    cursor = 0
    group_blocks = []
    for _ in groups:
        group_blocks.append(perm[cursor:cursor + shared_prefix_blocks])
        cursor += shared_prefix_blocks
    tables = np.full((S, max_blocks), -1, dtype=np.int32)
    for s in range(S):
        j0 = 0
        if s in owner:
            if lens[s] <= shared_prefix_blocks * bs:
                raise ValueError("a sharing sequence must extend past the shared prompt")
            tables[s, :shared_prefix_blocks] = group_blocks[owner[s]]
            j0 = shared_prefix_blocks
        n_own = int(nblk[s]) - j0
        tables[s, j0:j0 + n_own] = perm[cursor:cursor + n_own]
        cursor += n_own

    Hkv, D = num_kv_heads, head_dim
    k_cache = _draw(rng, (num_blocks, Hkv, bs, D), kv_dtype)
    v_cache = _draw(rng, v_pool_shape(num_blocks, Hkv, D, bs), kv_dtype)
    q = _draw(rng, (S, num_heads, D), kv_dtype)
    k_new = _draw(rng, (S, Hkv, D), kv_dtype)
    v_new = _draw(rng, (S, Hkv, D), kv_dtype)

    # Live slots: positions 0 .. L-2 (the cached prefix).  Position L-1 is
    # the new token's slot; it stays poisoned until the write.
    live = np.zeros((num_blocks, bs), dtype=bool)
    slots = np.full(S, -1, dtype=np.int32)
    for s in range(S):
        L = int(lens[s])
        if L <= 0:
            continue
        pos = np.arange(L - 1)
        live[tables[s, pos // bs], pos % bs] = True
        slots[s] = new_token_slot(tables[s], L, bs)
    _poison_fill(rng, k_cache, v_cache, live, kv_dtype, poison)

    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Workload(name=name, kv_dtype=kv_dtype, num_seqs=S, num_heads=num_heads,
                    num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=num_blocks,
                    context_lens=lens.astype(np.int32), block_tables=tables,
                    k_cache=k_cache, v_cache=v_cache, q=q, k_new=k_new, v_new=v_new,
                    slot_mapping=slots, scale=np.float32(scale), poison=poison,
                    shared_blocks=shared_total)


# --------------------------------------------------------------------------
# The five decode workloads.
# --------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny-fp32",
    2: "gqa-bf16",
    3: "skewed-long-bf16",
    4: "shared-prefix-bf16",
    5: "large-batch-gqa-bf16",
}


# Largest context each workload's recipe allows: the reservation a server
# that sizes every request's KV for its maximum length would make.
MAX_CONTEXT = {1: 300, 2: 4096, 3: 32768, 4: 2048 + 512 + 1, 5: 8192}


def config_lengths(i: int, rng: np.random.Generator, *, long_last: bool = False,
                   num_seqs: Optional[int] = None) -> np.ndarray:
    """Context lengths of workload ``i``: the first draws of its recipe."""
    if i == 1:
        return np.array([1, 17, 100, 300])
    if i == 2:
        lens = rng.integers(128, 4096, size=32, endpoint=True)
    elif i == 3:
        lens = np.concatenate([[32768], rng.integers(256, 2048, size=7, endpoint=True)])
        if long_last:
            lens = np.concatenate([lens[1:], lens[:1]])
    elif i == 4:
        tails = rng.integers(0, 512, size=CFG4_GROUPS * CFG4_SAMPLES, endpoint=True)
        return CFG4_PROMPT + tails + 1
    elif i == 5:
        lens = np.clip(np.rint(rng.lognormal(6.9, 0.6, size=256)), 16, 8192).astype(np.int64)
    else:
        raise ValueError(f"no workload {i}")
    return lens[:num_seqs] if num_seqs else lens


CFG4_GROUPS, CFG4_SAMPLES, CFG4_PROMPT = 16, 8, 2048


def make_config(i: int, *, seed: Optional[int] = None, poison: str = "nan",
                block_size: Optional[int] = None, long_last: bool = False,
                num_seqs: Optional[int] = None) -> Workload:
    """Build decode workload ``i`` (1..5) from its seeded recipe.

    block_size overrides the default 16 (workload 5 is also run at 32);
    long_last moves workload 3's long sequence to the end; num_seqs trims
    workloads 2, 3 and 5 to their first sequences (same draws) for quick tests.
    """
    rng = np.random.default_rng(SEED_BASE + i if seed is None else seed)
    lens = config_lengths(i, rng, long_last=long_last, num_seqs=num_seqs)
    if i == 1:
        return build_workload(CONFIG_NAMES[1], rng, kv_dtype=F32, context_lens=lens,
                              num_heads=4, num_kv_heads=4, head_dim=64,
                              block_size=block_size or 16, num_blocks=48, poison=poison,
                              scale=0.125)
    if i == 2:
        return build_workload(CONFIG_NAMES[2], rng, kv_dtype=BF16, context_lens=lens,
                              num_heads=32, num_kv_heads=8, head_dim=128,
                              block_size=block_size or 16, poison=poison)
    if i == 3:
        return build_workload(CONFIG_NAMES[3] + ("-longlast" if long_last else ""), rng,
                              kv_dtype=BF16, context_lens=lens, num_heads=32,
                              num_kv_heads=8, head_dim=128, block_size=block_size or 16,
                              poison=poison)
    if i == 4:
        bs = block_size or 16
        groups = [list(range(g * CFG4_SAMPLES, (g + 1) * CFG4_SAMPLES)) for g in range(CFG4_GROUPS)]
        return build_workload(CONFIG_NAMES[4], rng, kv_dtype=BF16, context_lens=lens,
                              num_heads=32, num_kv_heads=8, head_dim=128, block_size=bs,
                              shared_prefix_groups=groups, shared_prefix_blocks=CFG4_PROMPT // bs,
                              poison=poison)
    bs = block_size or 16
    nblk = int(((lens + bs - 1) // bs).sum())
    return build_workload(CONFIG_NAMES[5] + f"-bs{bs}", rng, kv_dtype=BF16,
                          context_lens=lens, num_heads=64, num_kv_heads=8, head_dim=128,
                          block_size=bs, num_blocks=int(math.ceil(nblk / 0.97)),
                          poison=poison)


# --------------------------------------------------------------------------
# Input transforms used by invariance tests and the contiguous comparison run.
# --------------------------------------------------------------------------

def _slot_arrays(w: Workload):
    """Arrays of (block, offset) pairs per sequence, positions 0 .. L-1."""
    out = []
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        pos = np.arange(L)
        out.append((w.block_tables[s, pos // w.block_size], pos % w.block_size))
    return out


def permute_pool(w: Workload, perm: np.ndarray) -> Workload:
    """Move physical block b to perm[b] and rewrite tables and slots to match.

    The logical content seen by every sequence is unchanged.
    """
    perm = np.asarray(perm, dtype=np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    k = w.k_cache[inv]
    v = w.v_cache[inv]
    tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    slots = w.slot_mapping.astype(np.int64)
    live = slots >= 0
    sb, so = np.divmod(np.where(live, slots, 0), w.block_size)
    slots = np.where(live, perm[sb] * w.block_size + so, -1).astype(np.int32)
    return dataclasses.replace(w, name=w.name + "-perm", k_cache=k, v_cache=v,
                               block_tables=tables, slot_mapping=slots)


def to_contiguous(w: Workload) -> Workload:
    """Pack each sequence's blocks in logical order at ids base_s + j.

    base_s is the running sum of earlier sequences' block counts: the
    layout a per-request contiguous reservation would give, expressed in the
    same pool format.  Shared blocks are copied once per sequence, so a
    sequence never reads another's memory.  Free space after the packed
    blocks keeps poison.
    """
    nblk = w.blocks_per_seq()
    total = int(nblk.sum())
    nb = max(total, 1)
    k = np.empty((nb,) + w.k_cache.shape[1:], dtype=w.k_cache.dtype)
    v = np.empty((nb,) + w.v_cache.shape[1:], dtype=w.v_cache.dtype)
    tables = np.full_like(w.block_tables, -1)
    slots = np.full_like(w.slot_mapping, -1)
    base = 0
    for s in range(w.num_seqs):
        n = int(nblk[s])
        ids = w.block_tables[s, :n]
        k[base:base + n] = w.k_cache[ids]
        v[base:base + n] = w.v_cache[ids]
        tables[s, :n] = np.arange(base, base + n, dtype=np.int32)
        if w.slot_mapping[s] >= 0:
            b, o = divmod(int(w.slot_mapping[s]), w.block_size)
            j = int(np.nonzero(ids == b)[0][-1])
            slots[s] = (base + j) * w.block_size + o
        base += n
    return dataclasses.replace(w, name=w.name + "-contig", num_blocks=nb, k_cache=k, v_cache=v,
                               block_tables=tables, slot_mapping=slots, shared_blocks=0)


def pack_logical(logical_k: List[np.ndarray], logical_v: List[np.ndarray], tables: np.ndarray,
                 num_blocks: int, block_size: int, fill) -> tuple:
    """Place per-sequence logical K/V ([Hkv, L, D] each) into a fresh pool.

    Used by tests that start from logical tensors and need the paged form.
    Every unused slot receives ``fill`` (a scalar in the storage dtype).
    """
    Hkv, _, D = logical_k[0].shape
    dt = logical_k[0].dtype
    k = np.full((num_blocks, Hkv, block_size, D), fill, dtype=dt)
    v = np.full(v_pool_shape(num_blocks, Hkv, D, block_size), fill, dtype=dt)
    T = v.shape[3]
    for s, (ks, vs) in enumerate(zip(logical_k, logical_v)):
        L = ks.shape[1]
        for p in range(L):
            b = int(tables[s, p // block_size])
            o = p % block_size
            k[b, :, o, :] = ks[:, p, :]
            row = (o // T) * D
            v[b, :, row:row + D, o % T] = vs[:, p, :]
    return k, v
