"""Reference model of the KV block manager, and block copies.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product (libpa.so: its C++ block manager and its HIP
block-copy kernel) never calls it.

What it models, from the pages:

* "How does vLLM PagedAttention manage Virtual Memory Pages ...", section
  "Key Technical Innovations": item 1, each sequence has a table from its
  logical blocks to physical blocks anywhere in the pool; item 2, one block
  (e.g. 16 tokens) is taken at a time as generation proceeds; item 3, parallel
  samples share the physical blocks of an identical prompt, copy-on-write.
  Section "Example": the free list is taken from its front, and a block is
  opened when the length after the append is 1 more than a multiple of the
  block size (position p = length - 1 with p % block_size == 0).
* "Paged Attention: OS-Inspired Memory Management for KV Caches", section
  "Key terms in this lesson": a shared block carries a reference count (the
  number of sequences pointing at it); copy-on-write shares a block until
  someone writes to it and then gives that writer a private copy; internal
  fragmentation is memory reserved for a request that it never uses.
* "PagedAttention and KV memory management", "Key takeaways": sequences are
  preempted by swapping (or recomputing); paging makes that finer grained.

Readings where the pages are silent (the C++ manager follows the same written
rules, it shares no code with this model):
  * Freed blocks go to the back of the free list, in table order; swapped-out
    sequences' blocks are released the same way.  With the front-of-list
    allocation of the pages' sketch this makes every block id deterministic.
  * Copy-on-write happens on append: a sequence that writes a new token into a
    last block whose reference count is above 1 first takes a fresh block,
    and the old block's content must be copied into it (the returned pair);
    the old block loses one reference.  A block that has become private (count
    1) is written in place.
  * Fork gives the child the parent's whole table and length; every block gains
    one reference.
  * Swap moves the listed sequences between the device pool and a host pool;
    a block shared by several listed sequences is copied once and its
    reference count moves with it.  A block shared with a sequence that stays
    behind is copied, and the one left behind keeps its other references.
  * Every operation is all-or-nothing: it checks capacity before changing
    anything.
"""
from __future__ import annotations

import numpy as np

DEVICE = 0
HOST = 1


class BlockManagerError(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_device_blocks, num_host_blocks, block_size, max_blocks_per_seq,
                 device_free_order=None):
        self.bs = int(block_size)
        self.max_blocks = int(max_blocks_per_seq)
        order = list(range(num_device_blocks)) if device_free_order is None else \
            [int(b) for b in device_free_order]
        if sorted(order) != list(range(num_device_blocks)):
            raise BlockManagerError("device_free_order must be a permutation of the pool")
        self.free = [order, list(range(num_host_blocks))]
        self.ref = [[0] * num_device_blocks, [0] * num_host_blocks]
        self.seqs = {}          # seq_id -> {"table": [...], "len": L, "where": DEVICE|HOST}

    # -- helpers ---------------------------------------------------------
    def _seq(self, sid):
        if sid not in self.seqs:
            raise BlockManagerError(f"unknown sequence {sid}")
        return self.seqs[sid]

    def _take(self, where):
        b = self.free[where].pop(0)
        self.ref[where][b] = 1
        return b

    def _release(self, where, b):
        self.ref[where][b] -= 1
        if self.ref[where][b] == 0:
            self.free[where].append(b)

    def blocks_for(self, n_tokens):
        return -(-n_tokens // self.bs)

    # -- operations ------------------------------------------------------
    def add(self, sid, num_tokens):
        """New sequence holding num_tokens prompt tokens; returns their slots."""
        if sid in self.seqs:
            raise BlockManagerError(f"sequence {sid} exists")
        nb = self.blocks_for(num_tokens)
        if num_tokens < 0 or nb > self.max_blocks or nb > len(self.free[DEVICE]):
            raise BlockManagerError("no room")
        table = [self._take(DEVICE) for _ in range(nb)]
        self.seqs[sid] = {"table": table, "len": int(num_tokens), "where": DEVICE}
        return [table[p // self.bs] * self.bs + p % self.bs for p in range(num_tokens)]

    def append(self, sid):
        """One new token; returns (slot, cow_src, cow_dst), -1 for no copy."""
        s = self._seq(sid)
        if s["where"] != DEVICE:
            raise BlockManagerError("sequence is swapped out")
        p = s["len"]
        j, o = divmod(p, self.bs)
        src = dst = -1
        if o == 0:
            if j >= self.max_blocks or not self.free[DEVICE]:
                raise BlockManagerError("no room")
            s["table"].append(self._take(DEVICE))
        else:
            last = s["table"][j]
            if self.ref[DEVICE][last] > 1:
                if not self.free[DEVICE]:
                    raise BlockManagerError("no room")
                new = self._take(DEVICE)
                self.ref[DEVICE][last] -= 1
                s["table"][j] = new
                src, dst = last, new
        s["len"] = p + 1
        return s["table"][j] * self.bs + o, src, dst

    def fork(self, parent, child):
        s = self._seq(parent)
        if child in self.seqs:
            raise BlockManagerError(f"sequence {child} exists")
        for b in s["table"]:
            self.ref[s["where"]][b] += 1
        self.seqs[child] = {"table": list(s["table"]), "len": s["len"], "where": s["where"]}

    def free_seq(self, sid):
        s = self._seq(sid)
        for b in s["table"]:
            self._release(s["where"], b)
        del self.seqs[sid]

    def _swap(self, sids, frm, to):
        for sid in sids:
            if self._seq(sid)["where"] != frm:
                raise BlockManagerError(f"sequence {sid} is not in the source pool")
        if len(set(sids)) != len(sids):
            raise BlockManagerError("duplicate sequence")
        distinct = []
        for sid in sids:
            for b in self.seqs[sid]["table"]:
                if b not in distinct:
                    distinct.append(b)
        if len(distinct) > len(self.free[to]):
            raise BlockManagerError("no room")
        mapping = {}
        pairs = []
        for sid in sids:
            s = self.seqs[sid]
            for j, b in enumerate(s["table"]):
                if b not in mapping:
                    mapping[b] = self._take(to)
                    pairs.append((b, mapping[b]))
                else:
                    self.ref[to][mapping[b]] += 1
                s["table"][j] = mapping[b]
            s["where"] = to
        # Release the source blocks after all mappings are made, in the order
        # of first appearance: one reference per listed holder moves, the
        # block keeps the rest (holders that stay behind).
        for b, c in pairs:
            for _ in range(self.ref[to][c]):
                self._release(frm, b)
        return pairs

    def swap_out(self, sids):
        """Move the listed sequences to the host pool; returns (device, host) block pairs."""
        return self._swap(list(sids), DEVICE, HOST)

    def swap_in(self, sids):
        """Move the listed sequences back to the device pool; returns (host, device) pairs."""
        return self._swap(list(sids), HOST, DEVICE)

    # -- queries ---------------------------------------------------------
    def tables(self, sids):
        """Device block tables [n, max_blocks] (padding -1) and lengths [n]."""
        t = np.full((len(sids), self.max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(sids), dtype=np.int32)
        for i, sid in enumerate(sids):
            s = self._seq(sid)
            if s["where"] != DEVICE:
                raise BlockManagerError("sequence is swapped out")
            t[i, :len(s["table"])] = s["table"]
            lens[i] = s["len"]
        return t, lens

    def num_free(self, where=DEVICE):
        return len(self.free[where])


# ----------------------------------------------------------------------
# Block copies.  A block is all of its KV heads' K tiles and V tiles; the
# copy moves raw element bits.  Pairs with an id outside the pools are
# skipped.  Destinations must be distinct and must not be sources of the
# same call (then every order of the copies gives the same result).
# ----------------------------------------------------------------------

def _raw(x):
    return x.view(np.uint32) if x.dtype == np.float32 else x


def copy_blocks(k_cache, v_cache, src, dst):
    """Copy-on-write copies inside one pool; returns new (k_cache, v_cache)."""
    return swap_blocks(k_cache, v_cache, k_cache, v_cache, src, dst)


def swap_blocks(dst_k, dst_v, src_k, src_v, src, dst):
    """Block dst[i] of the destination pool := block src[i] of the source pool."""
    out_k, out_v = dst_k.copy(), dst_v.copy()
    rk, rv = _raw(out_k), _raw(out_v)
    sk, sv = _raw(src_k), _raw(src_v)
    for a, b in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        if not (0 <= a < sk.shape[0] and 0 <= b < rk.shape[0]):
            continue
        rk[b] = sk[a]
        rv[b] = sv[a]
    return out_k, out_v


# ----------------------------------------------------------------------
# Waste accounting: internal fragmentation, the share of reserved KV slots
# that hold no token ("Paged Attention: OS-Inspired ...", "Key terms").
# ----------------------------------------------------------------------

def waste_contiguous(context_lens, max_len):
    """Each sequence reserves max_len slots up front."""
    L = np.asarray(context_lens, dtype=np.int64)
    return 1.0 - L.sum() / (len(L) * int(max_len))


def waste_paged(context_lens, block_size, shared_tokens=0, shared_blocks=0):
    """Each sequence holds ceil(L / bs) blocks; shared prefix blocks are held once.

    shared_tokens / shared_blocks: tokens and blocks held by prefixes that
    several sequences share, to be counted once (pass them as the amount to
    subtract from the per-sequence sums).
    """
    L = np.asarray(context_lens, dtype=np.int64)
    blocks = (-(-L // int(block_size))).sum() - shared_blocks
    tokens = L.sum() - shared_tokens
    return 1.0 - tokens / (blocks * int(block_size))
