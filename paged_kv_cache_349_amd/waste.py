"""KV memory waste of the decode workloads: contiguous reservation vs paging.

    python -m paged_kv_cache_349_amd.waste [--block-size 16 32]

A server that reserves each request's KV for the longest context it allows
leaves the unused part of every reservation empty ("PagedAttention and KV
memory management", intro and "Key takeaways"; "How does vLLM PagedAttention
manage Virtual Memory Pages ...", section "Detail", the contiguous-allocation
diagram).  With paging, each sequence holds ceil(L / block_size) blocks and
parallel samples hold their common prompt once ("Key Technical Innovations",
item 3).  Waste = the share of reserved (or allocated) KV slots that hold no
token, i.e. internal fragmentation ("Paged Attention: OS-Inspired Memory
Management for KV Caches", "Key terms in this lesson").

The paged numbers come from the C++ block manager holding each workload's
sequences: prompts added, parallel samples forked from their group's prompt
and grown token by token with copy-on-write, exactly as a server would.
The manager's host cost per decode step (one batched append for every
sequence plus the block tables for the decode call) is timed as well.
"""
from __future__ import annotations

import argparse
import json
import statistics
import time

import numpy as np

from . import workloads as wl
from .block_manager import BlockManager


def _populate(i: int, block_size: int, spare: int = 64):
    rng = np.random.default_rng(wl.SEED_BASE + i)
    lens = wl.config_lengths(i, rng)
    blocks = int(((lens + block_size - 1) // block_size).sum())
    m = BlockManager(blocks + spare, 0, block_size,
                     int((wl.MAX_CONTEXT[i] + spare) // block_size + 2))
    if i == 4:
        n = wl.CFG4_SAMPLES
        for g in range(wl.CFG4_GROUPS):
            base = g * n
            m.add(base, wl.CFG4_PROMPT)
            for c in range(1, n):
                m.fork(base, base + c)
        # grow every sample to its length, one batched append per step
        remaining = lens - wl.CFG4_PROMPT
        ids = np.arange(len(lens))
        while remaining.max() > 0:
            live = ids[remaining > 0]
            m.append_batch(live)
            remaining[live] -= 1
    else:
        for s, L in enumerate(lens):
            m.add(s, int(L))
    return m, lens


def waste(i: int, block_size: int = 16) -> dict:
    m, lens = _populate(i, block_size)
    st = m.stats()
    S = len(lens)
    reserved = S * wl.MAX_CONTEXT[i]
    paged_slots = st["device_blocks_used"] * block_size
    return {
        "workload": i,
        "block_size": block_size,
        "num_seqs": S,
        "max_context": int(wl.MAX_CONTEXT[i]),
        "tokens_logical": int(lens.sum()),
        "tokens_stored": st["device_tokens_stored"],
        "contiguous_slots": int(reserved),
        "contiguous_waste": 1.0 - lens.sum() / reserved,
        "paged_slots": int(paged_slots),
        "paged_waste": st["device_internal_waste"],
        "shared_blocks": st["device_blocks_shared"],
        "memory_ratio": reserved / paged_slots,
    }


def time_step(i: int = 5, block_size: int = 16, steps: int = 200) -> float:
    """Median host microseconds of one decode step's manager work."""
    rng = np.random.default_rng(wl.SEED_BASE + i)
    S = len(wl.config_lengths(i, rng))
    # room for every sequence to grow by `steps` tokens
    m, lens = _populate(i, block_size, spare=S * (steps // block_size + 1))
    ids = np.arange(len(lens), dtype=np.int64)
    stride = int((lens.max() + steps + block_size - 1) // block_size)   # the batch's table width
    # outputs go to buffers reused every step, as a server's staging buffers would be
    step_out = tuple(np.empty(len(ids), np.int32) for _ in range(3))
    table_out = (np.empty((len(ids), stride), np.int32), np.empty(len(ids), np.int32))
    t = []
    for _ in range(steps):
        t0 = time.perf_counter()
        m.append_batch(ids, out=step_out)
        m.tables(ids, stride=stride, out=table_out)
        t.append(time.perf_counter() - t0)
    return statistics.median(t) * 1e6


def main():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--block-size", type=int, nargs="+", default=[16, 32])
    args = p.parse_args()
    for bs in args.block_size:
        for i in (1, 2, 3, 4, 5):
            print(json.dumps({k: (round(v, 6) if isinstance(v, float) else v)
                              for k, v in waste(i, bs).items()}))
    print(json.dumps({"manager_us_per_step": round(time_step(5, 16), 2), "workload": 5,
                      "block_size": 16}))


if __name__ == "__main__":
    main()
