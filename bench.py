"""Benchmark of the paged decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--block-size 16|32]

One step = the slot write (the new token of every sequence goes into its
slot) + decode (single-query attention of every sequence over the paged
pool), on one HIP stream, issued as one pa_decode_step call (also timed as
pa_write_kv + pa_decode), over the large-batch GQA workload:
256 sequences, context lengths lognormal(6.9, 0.6) clipped to [16, 8192],
64 query heads / 8 KV heads, head_dim 128, block size 16, bf16 K/V/q, fp32
output, a shuffled pool with 3% free blocks.  Inputs are seeded synthetic
draws, resident in HBM before the timed region.

Printed: one JSON line on stdout.  Progress goes to stderr.

  value        KV bytes read per step / wall time per step (GB/s): K
               steps back to back between two device synchronisations, with
               no events on the stream (a second loop of K steps records the
               per-call and per-kernel breakdown).
  roofline     the attention kernel alone (decode_mfma_bf16, without the
               planner and the partition merge): algorithmic bytes per launch
               (live K/V tokens + q + out + live block-table entries) / its
               mean duration from HIP events that the library records on the
               launch stream right around that kernel, against the 8 TB/s HBM
               peak.  `call_frac` is the same bytes over the whole pa_decode
               call (three kernels and the gaps between them).  `traffic` is
               the HBM bytes per launch that the FETCH_SIZE / WRITE_SIZE
               counters measured, scaled by a plain-copy calibration, read
               from profiles/ and reported only while the kernel source is
               unchanged since it was measured.
  cpu_baseline the float64 CPU oracle (one thread) on the whole step.

The contiguous comparison runs the same decode kernel over the same tokens
packed sequence by sequence in logical order (identity-like tables):
paged_overhead_vs_contig compares whole pa_decode calls, paged and packed
alternating and timed alike; paged_overhead_vs_contig_kernel compares the
attention kernel alone.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV GB/s (% of HBM peak) and seq-steps/s at 1 GPU"
HBM_PEAK_GBPS = 8000.0
DECODE_SOURCES = ["paged_kv_cache_349_amd/csrc/pa_decode.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_large_batch_gqa.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per decode launch from the committed counter summary, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def bench_ceilings(w, d, dev, stream, kern_mean_us):
    """Empirical read ceilings on this GPU, for the roofline's context:
    a contiguous read of the whole K and V pools, and a read of exactly the
    decode's live K/V tiles through the block tables (sequence, block, head
    order), both with no arithmetic."""
    import numpy as np
    import torch

    import paged_kv_cache_349_amd as pa

    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    nb = w.blocks_per_seq()
    ids = np.concatenate([w.block_tables[s, :nb[s]] for s in range(w.num_seqs)]).astype(np.int64)
    tiles_np = (ids[:, None] * w.num_kv_heads + np.arange(w.num_kv_heads)[None, :]).reshape(-1)
    tiles = torch.from_numpy(tiles_np.astype(np.int32)).to(dev)
    tile_bytes = w.block_size * w.head_dim * 2
    tile_total = 2 * tiles.numel() * tile_bytes

    def timed(fn, iters=20):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return statistics.mean(a.elapsed_time(b) * 1e3 for a, b in ev)

    t_pool = timed(lambda: (pa.probe_read(d.k_cache, sink), pa.probe_read(d.v_cache, sink)))
    pool_bytes = 2 * d.k_cache.numel() * d.k_cache.element_size()
    t_tiles = timed(lambda: pa.probe_read_tiles(d.k_cache, d.v_cache, tiles, sink))
    stream_gbps = pool_bytes / (t_pool * 1e-6) / 1e9
    tiles_gbps = tile_total / (t_tiles * 1e-6) / 1e9
    kernel_gbps = (w.kv_bytes_unique() + w.small_bytes()) / (kern_mean_us * 1e-6) / 1e9
    log(f"ceilings: contiguous read {stream_gbps:.0f} GB/s, paged tile read {tiles_gbps:.0f} GB/s")
    return {
        "contiguous_read_gbps": round(stream_gbps, 1), "contiguous_read_bytes": pool_bytes,
        "paged_tile_read_gbps": round(tiles_gbps, 1), "paged_tile_read_bytes": tile_total,
        "paged_tile_read_us": round(t_tiles, 2),
        "decode_kernel_vs_paged_tile_read": round(kernel_gbps / tiles_gbps, 4),
    }


def copy_calibration(dev):
    """One plain 1 GiB device-to-device copy: a known byte count for scaling the
    FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 --pmc run of the same job."""
    import torch

    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    log("copy calibration: one 1 GiB device copy done")


def bench_shared_prefix(args, dev, stream):
    """Parallel sampling: 16 prompts of 2048 tokens, 8 samples each with private
    tails of 1..513 tokens (bf16, 32/8 heads, D 128, bs 16).  pa_decode reads
    every sample's prompt blocks; pa_decode_shared_prefix reads each once.
    Roofline: distinct live K/V bytes + q + out + table per call / call time.
    """
    import numpy as np
    import torch

    import paged_kv_cache_349_amd as pa
    from paged_kv_cache_349_amd import workloads as wl
    from paged_kv_cache_349_amd.device_io import upload

    w = wl.make_config(4)
    d = upload(w, dev)
    pa.write_kv(d.k_cache, d.v_cache, d.k_new, d.v_new, d.slot_mapping)
    gs, pbl = w.prefix_groups()
    gs_d, pb_d = torch.from_numpy(gs).to(dev), torch.from_numpy(pbl).to(dev)
    out_p = torch.empty_like(d.out)

    def plain():
        pa.decode(d.out, d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                  float(w.scale), w.block_size)

    def shared():
        pa.decode_shared_prefix(out_p, d.q, d.k_cache, d.v_cache, d.block_tables,
                                d.context_lens, gs_d, pb_d, float(w.scale), w.block_size)

    def timed(fn, iters=50):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return statistics.mean(a.elapsed_time(b) * 1e3 for a, b in ev)

    t_plain, t_shared = timed(plain), timed(shared)
    uniq = w.kv_bytes_unique() + w.small_bytes()
    diff = float((out_p - d.out).abs().max())
    log(f"shared-prefix workload: pa_decode {t_plain:.1f} us, pa_decode_shared_prefix "
        f"{t_shared:.1f} us ({t_plain / t_shared:.2f}x)")
    return {
        "workload": w.name, "num_seqs": w.num_seqs, "groups": int(len(pbl)),
        "prefix_tokens": int(pbl.max()) * w.block_size,
        "kv_bytes_logical": w.kv_bytes_logical(), "kv_bytes_unique": w.kv_bytes_unique(),
        "decode_us": round(t_plain, 2), "shared_prefix_us": round(t_shared, 2),
        "speedup": round(t_plain / t_shared, 3),
        "logical_gbps": round(w.kv_bytes_logical() / (t_shared * 1e-6) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(uniq / (t_shared * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(uniq / (t_shared * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "algorithmic_bytes_per_call": uniq, "scope": "whole call"},
        "max_abs_diff_vs_decode": float(f"{diff:.3e}"),
    }


def bench_block_size_32(args, dev, stream):
    """The large-batch workload's block-size-32 variant (same lengths, own pool):
    whole steps through pa_decode_step timed back to back, then the attention
    kernel alone by the library's events."""
    import torch

    import paged_kv_cache_349_amd as pa
    from paged_kv_cache_349_amd import workloads as wl
    from paged_kv_cache_349_amd.device_io import upload

    w = wl.make_config(5, block_size=32, seed=args.seed)
    d = upload(w, dev)

    def step():
        pa.decode_step(d.k_cache, d.v_cache, d.k_new, d.v_new, d.slot_mapping, d.out, d.q,
                       d.block_tables, d.context_lens, float(w.scale), w.block_size)

    K = max(20, min(args.steps, 100))
    for _ in range(5):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / K
    pa.kernel_timing_begin(K)
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    kern_ms, kern_n = pa.kernel_timing_end()
    kern_us = kern_ms * 1e3 / kern_n
    alg = w.kv_bytes_unique() + w.small_bytes()
    log(f"block size 32: {us:.1f} us/step, attention kernel {kern_us:.1f} us")
    del d
    return {
        "workload": w.name, "block_size": 32, "num_blocks": w.num_blocks, "steps": K,
        "us_per_step": round(us, 2),
        "kv_gbps_step": round(w.kv_bytes_logical() / (us * 1e-6) / 1e9, 2),
        "kernel_us_mean": round(kern_us, 2),
        "kernel_frac": round(alg / (kern_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_launch": alg,
    }


def bench_configs(args, dev, stream, which):
    """The other workloads (gqa, skewed long context, parallel sampling), cold.

    Their K/V (166-285 MB) is about the size of the 256 MB last-level cache,
    so every timed launch follows a read of 1 GiB that evicts it (outside the
    event pair; a read leaves no dirty lines for the decode to write back).
    Per workload:
      step_us_warm     pa_decode_step (the parallel-sampling workload: write +
                       pa_decode_shared_prefix) back to back, warm
      call_us_cold     one decode call (planner, attention kernel, merge)
      kernel_us_cold   the attention kernel alone (the library's events)
      *_frac           algorithmic bytes (distinct live K/V + q + out + table)
                       / time / 8 TB/s
      contig_*         the same calls over the tokens packed sequence by
                       sequence (identity-like tables), cold, alternating
      max_abs_err      output of the timed call against the float64 oracle
    """
    import numpy as np
    import torch

    import oracle
    import paged_kv_cache_349_amd as pa
    from paged_kv_cache_349_amd import workloads as wl
    from paged_kv_cache_349_amd.device_io import upload

    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    n_cold = max(5, args.config_iters)
    res = {}
    for cfg in which:
        w = wl.make_config(cfg)
        d = upload(w, dev)
        pa.write_kv(d.k_cache, d.v_cache, d.k_new, d.v_new, d.slot_mapping)
        prefix = cfg == 4
        if prefix:
            gs, pbl = w.prefix_groups()
            gsd, pbd = torch.from_numpy(gs).to(dev), torch.from_numpy(pbl).to(dev)

        def call(dd=d, ww=w, shared=prefix):
            if shared:
                pa.decode_shared_prefix(dd.out, dd.q, dd.k_cache, dd.v_cache, dd.block_tables,
                                        dd.context_lens, gsd, pbd, float(ww.scale), ww.block_size)
            else:
                pa.decode(dd.out, dd.q, dd.k_cache, dd.v_cache, dd.block_tables,
                          dd.context_lens, float(ww.scale), ww.block_size)

        def step():
            if prefix:
                pa.write_kv(d.k_cache, d.v_cache, d.k_new, d.v_new, d.slot_mapping)
                call()
            else:
                pa.decode_step(d.k_cache, d.v_cache, d.k_new, d.v_new, d.slot_mapping, d.out,
                               d.q, d.block_tables, d.context_lens, float(w.scale), w.block_size)

        def cold_calls(fn, n):
            ts = []
            for _ in range(n):
                flush.sum()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            return ts

        def cold_kernel(fn, n):
            pa.kernel_timing_begin(n)
            for _ in range(n):
                flush.sum()
                fn()
            torch.cuda.synchronize()
            ms, k = pa.kernel_timing_end()
            return ms * 1e3 / k

        def warm_kernel(fn, n):
            pa.kernel_timing_begin(n)
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            ms, k = pa.kernel_timing_end()
            return ms * 1e3 / k

        for _ in range(5):
            step()
        torch.cuda.synchronize()
        K = max(20, min(args.steps, 200))
        t0 = time.perf_counter()
        for _ in range(K):
            step()
        torch.cuda.synchronize()
        step_us = (time.perf_counter() - t0) * 1e6 / K
        kern_warm = warm_kernel(call, K)
        calls = cold_calls(call, n_cold)
        kern_cold = cold_kernel(call, n_cold)
        out = d.out.cpu().numpy()
        k_ref, v_ref = oracle.write_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping,
                                       w.block_size)
        ref = oracle.decode(w.q, k_ref, v_ref, w.block_tables, w.context_lens, w.scale,
                            w.block_size, w.kv_dtype)
        err = float(np.abs(out - ref).max())
        alg = w.kv_bytes_unique() + w.small_bytes()
        frac = lambda us: round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        call_cold = statistics.median(calls)
        rec = {
            "num_seqs": w.num_seqs, "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size,
            "context_tokens": int(w.context_lens.sum()), "max_context": int(w.context_lens.max()),
            "call": "pa_decode_shared_prefix" if prefix else "pa_decode",
            "algorithmic_bytes": alg, "kv_bytes_logical": w.kv_bytes_logical(),
            "step_us_warm": round(step_us, 2),
            "call_us_cold": round(call_cold, 2),
            "call_us_cold_p90": round(float(np.percentile(calls, 90)), 2),
            "kernel_us_cold": round(kern_cold, 2), "kernel_us_warm": round(kern_warm, 2),
            "kernel_frac_cold": frac(kern_cold), "call_frac_cold": frac(call_cold),
            "kernel_frac_warm": frac(kern_warm), "step_frac_warm": frac(step_us),
            "seq_steps_per_s": round(w.num_seqs / (step_us * 1e-6), 1),
            "max_abs_err": float(f"{err:.3e}"),
        }
        if prefix:
            plain = lambda: call(shared=False)
            rec["plain_decode_call_us_cold"] = round(statistics.median(cold_calls(plain, n_cold)), 2)
            rec["plain_decode_kernel_us_cold"] = round(cold_kernel(plain, n_cold), 2)
        if not args.no_contig:
            wc = wl.to_contiguous(w)
            dc = upload(wc, dev)
            pa.write_kv(dc.k_cache, dc.v_cache, dc.k_new, dc.v_new, dc.slot_mapping)
            pc, cc = [], []
            for _ in range(n_cold):
                pc += cold_calls(lambda: call(shared=False), 1)
                cc += cold_calls(lambda: call(dc, wc, False), 1)
            rec["contig_call_us_cold"] = round(statistics.median(cc), 2)
            rec["paged_call_us_cold"] = round(statistics.median(pc), 2)
            rec["paged_overhead_vs_contig"] = round(statistics.median(pc) / statistics.median(cc) - 1, 4)
            kp = cold_kernel(lambda: call(shared=False), n_cold)
            kc = cold_kernel(lambda: call(dc, wc, False), n_cold)
            rec["paged_overhead_vs_contig_kernel"] = round(kp / kc - 1, 4)
            if prefix:
                rec["contig_note"] = ("packed run gives every sample its own copy of the prompt "
                                      "(plain pa_decode on both sides): context only")
            del dc
        log(f"{w.name}: step {step_us:.1f} us warm; call {call_cold:.1f} us cold "
            f"({rec['call_frac_cold']:.3f}); kernel {kern_cold:.1f} us cold "
            f"({rec['kernel_frac_cold']:.3f}), {kern_warm:.1f} us warm; err {err:.2e}"
            + (f"; paged vs packed {rec['paged_overhead_vs_contig']:+.2%} per call, "
               f"{rec['paged_overhead_vs_contig_kernel']:+.2%} per kernel"
               if "paged_overhead_vs_contig" in rec else ""))
        res[w.name] = rec
        del d
    del flush
    return res


PCIE_GEN5_X16_GBPS = 63.0   # 32 GT/s x 16 lanes, 128b/130b coding, per direction


def bench_blocks(args, w, d, dev, stream):
    """Block manager, copy-on-write copies and swap on the same workload.

    Runs last: the copies overwrite blocks of the decode pool.
      kv_waste        contiguous max-context reservation vs the manager's paged
                      allocation of this workload's sequences
      manager_us      host time of the manager's work for one decode step
                      (one batched append for all sequences + their tables)
      copy            pa_copy_blocks of 4096 random block pairs (32 KB per K or
                      V span): bytes read + written per launch / mean duration
      swap_out/in     pa_swap_blocks of 2048 blocks to / from a pinned host
                      pool, against one contiguous copy of the same bytes
                      (torch / HIP DMA) and the host link's nominal rate
    """
    import numpy as np
    import torch

    import paged_kv_cache_349_amd as pa
    from paged_kv_cache_349_amd import waste

    out = {}
    cfg = args.config
    wr = waste.waste(cfg, w.block_size)
    out["kv_waste"] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in wr.items()}
    out["manager_us_per_step"] = round(waste.time_step(cfg, w.block_size), 2)

    rng = np.random.default_rng(1)
    NB = w.num_blocks
    span = w.num_kv_heads * w.block_size * w.head_dim * 2
    n = min(4096, NB // 2)
    ids = rng.permutation(NB)[:2 * n].astype(np.int32)
    src = torch.from_numpy(ids[:n]).to(dev)
    dst = torch.from_numpy(ids[n:]).to(dev)

    def timed(fn, iters=20):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return statistics.mean(a.elapsed_time(b) * 1e3 for a, b in ev)

    us = timed(lambda: pa.copy_blocks(d.k_cache, d.v_cache, src, dst))
    moved = 2 * n * span * 2
    out["copy"] = {"pairs": n, "bytes_per_launch": moved, "us_mean": round(us, 2),
                   "achieved_gbps": round(moved / (us * 1e-6) / 1e9, 1),
                   "peak_gbps": HBM_PEAK_GBPS}
    log(f"copy_blocks: {n} pairs, {us:.1f} us, {moved / (us * 1e-6) / 1e9:.0f} GB/s")

    ns = min(2048, NB)
    hk = torch.empty((ns,) + tuple(d.k_cache.shape[1:]), dtype=d.k_cache.dtype, pin_memory=True)
    hv = torch.empty((ns,) + tuple(d.v_cache.shape[1:]), dtype=d.v_cache.dtype, pin_memory=True)
    dev_ids = torch.from_numpy(rng.permutation(NB)[:ns].astype(np.int32)).to(dev)
    host_ids = torch.from_numpy(rng.permutation(ns).astype(np.int32)).to(dev)
    t_out = timed(lambda: pa.swap_blocks(hk, hv, d.k_cache, d.v_cache, dev_ids, host_ids), 5)
    t_in = timed(lambda: pa.swap_blocks(d.k_cache, d.v_cache, hk, hv, host_ids, dev_ids), 5)
    sb = 2 * ns * span
    flat_d = torch.empty(sb, dtype=torch.uint8, device=dev)
    flat_h = torch.empty(sb, dtype=torch.uint8, pin_memory=True)
    t_d2h = timed(lambda: flat_h.copy_(flat_d, non_blocking=True), 5)
    t_h2d = timed(lambda: flat_d.copy_(flat_h, non_blocking=True), 5)
    gb = lambda t: round(sb / (t * 1e-6) / 1e9, 2)
    out["swap"] = {"blocks": ns, "bytes": sb, "out_us": round(t_out, 1), "in_us": round(t_in, 1),
                   "out_gbps": gb(t_out), "in_gbps": gb(t_in),
                   "contiguous_copy_gbps": {"d2h": gb(t_d2h), "h2d": gb(t_h2d)},
                   "link_peak_gbps": PCIE_GEN5_X16_GBPS}
    log(f"swap_blocks: {ns} blocks, out {gb(t_out)} GB/s, in {gb(t_in)} GB/s "
        f"(contiguous copy d2h {gb(t_d2h)}, h2d {gb(t_h2d)})")
    return out


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--block-size", type=int, default=16, choices=(16, 32))
    p.add_argument("--config", type=int, default=5, choices=(2, 3, 4, 5),
                   help="workload to time (5, the large-batch GQA decode, is the headline; "
                        "the others are for diagnosis)")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--partition-tokens", type=int, default=0,
                   help="tokens per decode work item (0 = the library's choice)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-contig", action="store_true")
    p.add_argument("--cold-iters", type=int, default=20,
                   help="decode launches timed after flushing the caches (0 = skip)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain 1 GiB device copy (counter calibration)")
    p.add_argument("--no-blocks", action="store_true",
                   help="skip the block-manager, copy-on-write and swap measurements")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the streaming-read and paged-tile-read probes")
    p.add_argument("--no-bs32", action="store_true",
                   help="skip the block-size-32 variant of the large-batch workload")
    p.add_argument("--no-shared-prefix", action="store_true",
                   help="skip the shared-prefix decode measurement (parallel-sampling workload)")
    p.add_argument("--configs", default="2,3,4",
                   help="comma-separated other workloads measured cold in the `configs` record "
                        "('none' = no record)")
    p.add_argument("--config-iters", type=int, default=20,
                   help="cold launches per measurement in the `configs` record")
    p.add_argument("--configs-only", action="store_true",
                   help="run only the `configs` record (for profiling its cold launches)")
    p.add_argument("--shared-prefix", action="store_true",
                   help="time pa_decode_shared_prefix instead of pa_decode in the main loop "
                        "(groups of consecutive sequences with common leading blocks)")
    return p.parse_args()


def main() -> int:
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the paged decode step runs and is timed on a single MI355X.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_cache_349_amd as pa
    from paged_kv_cache_349_amd import workloads as wl
    from paged_kv_cache_349_amd.device_io import upload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    pa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    which = [] if args.configs.strip().lower() in ("", "none") else \
        [int(c) for c in args.configs.split(",") if c.strip()]
    if args.configs_only:
        res = bench_configs(args, dev, torch.cuda.current_stream(dev), which)
        if args.copy_calibration:
            copy_calibration(dev)
        print(json.dumps({"configs": res}), flush=True)
        return 0

    t = time.perf_counter()
    w = wl.make_config(args.config, block_size=args.block_size, seed=args.seed)
    log(f"workload {w.name}: S={w.num_seqs} NB={w.num_blocks} max_blocks={w.max_blocks} "
        f"tokens={int(w.context_lens.sum())} ({time.perf_counter() - t:.1f} s)")
    d = upload(w, dev)
    stream = torch.cuda.current_stream(dev)

    def write():
        pa.write_kv(d.k_cache, d.v_cache, d.k_new, d.v_new, d.slot_mapping)

    if args.shared_prefix:
        gs, pbl = w.prefix_groups()
        groups = (torch.from_numpy(gs).to(dev), torch.from_numpy(pbl).to(dev))

    def decode(dd=d, ww=w):
        if args.shared_prefix and dd is d:
            pa.decode_shared_prefix(dd.out, dd.q, dd.k_cache, dd.v_cache, dd.block_tables,
                                    dd.context_lens, groups[0], groups[1], float(ww.scale),
                                    ww.block_size, partition_tokens=args.partition_tokens)
            return
        pa.decode(dd.out, dd.q, dd.k_cache, dd.v_cache, dd.block_tables, dd.context_lens,
                  float(ww.scale), ww.block_size, partition_tokens=args.partition_tokens)

    for _ in range(args.warmup):
        write()
        decode()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    def step():
        pa.decode_step(d.k_cache, d.v_cache, d.k_new, d.v_new, d.slot_mapping, d.out, d.q,
                       d.block_tables, d.context_lens, float(w.scale), w.block_size)

    fused = not args.shared_prefix and args.partition_tokens == 0
    for _ in range(args.warmup if fused else 0):
        step()

    def timed_loop(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    K = args.steps
    # Throughput: K steps back to back, nothing else on the stream, one
    # synchronisation on each side.  A step is pa_decode_step (the write and
    # the decode, the write sharing the planner's launch); the same steps as
    # two calls (pa_write_kv, pa_decode) are timed the same way.
    wall_sep = timed_loop(lambda: (write(), decode()))
    wall = timed_loop(step) if fused else wall_sep
    log(f"timed {K} steps: {wall * 1e6 / K:.1f} us/step"
        + (f" (as two calls: {wall_sep * 1e6 / K:.1f} us/step)" if fused else ""))

    # Breakdown: the same K steps again with HIP events around each call and
    # the library's events around the attention kernel.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    pa.kernel_timing_begin(K)
    for i in range(K):
        ev[i][0].record(stream)
        write()
        ev[i][1].record(stream)
        decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    kern_ms, kern_n = pa.kernel_timing_end()
    kern_mean = kern_ms * 1e3 / kern_n
    write_us = [ev[i][0].elapsed_time(ev[i][1]) * 1e3 for i in range(K)]
    decode_us = [ev[i][1].elapsed_time(ev[i][2]) * 1e3 for i in range(K)]
    log(f"breakdown: decode call mean {statistics.mean(decode_us):.1f} us, attention kernel "
        f"mean {kern_mean:.1f} us, write mean {statistics.mean(write_us):.1f} us")

    out_gpu = d.out.cpu().numpy().astype(np.float64)

    kv_bytes = w.kv_bytes_logical()
    # Algorithmic minimum: distinct live K/V positions (blocks shared by
    # several sequences counted once) + q + out + live table entries.
    alg_bytes = w.kv_bytes_unique() + w.small_bytes()
    ms_per_step = wall * 1e3 / K
    dec_mean = statistics.mean(decode_us)
    dec_med = statistics.median(decode_us)
    qs = np.percentile(decode_us, [10, 90])

    result = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "num_seqs": w.num_seqs, "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "num_blocks": w.num_blocks,
            "context_tokens": int(w.context_lens.sum()), "max_context": int(w.context_lens.max()),
            "partition_tokens": args.partition_tokens or "adaptive",
            "seed": args.seed if args.seed is not None else wl.SEED_BASE + args.config,
        },
        "seq_steps_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "step_call": "pa_decode_step" if fused else "pa_write_kv + pa_decode",
        "ms_per_step_two_calls": round(wall_sep * 1e3 / K, 5),
        "pct_hbm_peak_step": round(100 * (alg_bytes + w.write_bytes()) / (ms_per_step * 1e-3) /
                                   (HBM_PEAK_GBPS * 1e9), 2),
        "decode_us": {"mean": round(dec_mean, 2), "median": round(dec_med, 2),
                      "p10": round(float(qs[0]), 2), "p90": round(float(qs[1]), 2)},
        "write_us_mean": round(statistics.mean(write_us), 2),
        "kv_gbps_decode": round(kv_bytes / (dec_med * 1e-6) / 1e9, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(alg_bytes / (kern_mean * 1e-6) / 1e9, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(alg_bytes / (kern_mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(w.name),
            "kernel": "decode_mfma_bf16",
            "kernel_us_mean": round(kern_mean, 2),
            "kernel_launches_timed": kern_n,
            "algorithmic_bytes_per_launch": alg_bytes,
            "call_frac": round(alg_bytes / (dec_mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        },
    }

    # Decode alone with the caches flushed before each launch by reading
    # 1 GiB outside the event pair (a read leaves no dirty lines behind for the
    # decode to write back): the 256 MB last-level cache holds a fifth of this
    # workload's KV, so warm and cold should be close.
    if args.cold_iters > 0:
        flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        cold = []
        for _ in range(args.cold_iters):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            decode()
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b) * 1e3)
        del flush
        result["decode_us_cold_median"] = round(statistics.median(cold), 2)
        result["decode_us_cold_p10_p90"] = [round(float(x), 2) for x in np.percentile(cold, [10, 90])]
        log(f"cold decode median {statistics.median(cold):.1f} us")

    if not args.no_contig:
        # The same kernels over the same tokens packed sequence by sequence
        # (identity-like tables).  Calls: paged and packed alternate, each
        # between two events and with nothing else recorded inside, so both
        # are timed the same way; kernels: the library's events around the
        # attention kernel, a loop of each.
        wc = wl.to_contiguous(w)
        dc = upload(wc, dev)
        pa.write_kv(dc.k_cache, dc.v_cache, dc.k_new, dc.v_new, dc.slot_mapping)
        for _ in range(args.warmup):
            decode(dc, wc)
            decode()
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        for i in range(K):
            evc[i][0].record(stream)
            decode()
            evc[i][1].record(stream)
            decode(dc, wc)
            evc[i][2].record(stream)
        torch.cuda.synchronize()
        paged_us = statistics.mean(evc[i][0].elapsed_time(evc[i][1]) * 1e3 for i in range(K))
        contig_us = statistics.mean(evc[i][1].elapsed_time(evc[i][2]) * 1e3 for i in range(K))
        pa.kernel_timing_begin(K)
        for i in range(K):
            decode(dc, wc)
        torch.cuda.synchronize()
        ck_ms, ck_n = pa.kernel_timing_end()
        contig_kern = ck_ms * 1e3 / ck_n
        out_c = dc.out.cpu().numpy()
        # The packed pool once more without per-block table reads (block j of
        # sequence s = its first table entry + j): splits the paged cost into
        # the table reads and the scatter of blocks over the pool.
        def decode_packed():
            pa.decode(dc.out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                      float(wc.scale), wc.block_size, partition_tokens=args.partition_tokens,
                      packed_pool=True)
        packed_kern = None
        if not args.shared_prefix and wc.kv_dtype == "bf16":
            for _ in range(args.warmup):
                decode_packed()
            pa.kernel_timing_begin(K)
            for i in range(K):
                decode_packed()
            torch.cuda.synchronize()
            pk_ms, pk_n = pa.kernel_timing_end()
            packed_kern = pk_ms * 1e3 / pk_n
        decode()
        torch.cuda.synchronize()
        result["paged_decode_us_mean"] = round(paged_us, 2)
        result["contig_decode_us_mean"] = round(contig_us, 2)
        result["paged_overhead_vs_contig"] = round(paged_us / contig_us - 1.0, 4)
        result["contig_kernel_us_mean"] = round(contig_kern, 2)
        result["paged_overhead_vs_contig_kernel"] = round(kern_mean / contig_kern - 1.0, 4)
        result["contig_output_bitwise_equal"] = bool(
            np.array_equal(out_c.view(np.uint32), d.out.cpu().numpy().view(np.uint32)))
        if packed_kern is not None:
            result["packed_no_table_kernel_us_mean"] = round(packed_kern, 2)
            result["paged_cost_split_kernel"] = {
                "table_reads": round(contig_kern / packed_kern - 1.0, 4),
                "block_scatter": round(kern_mean / contig_kern - 1.0, 4),
            }
            log(f"attention kernel on the packed pool without per-block table reads "
                f"{packed_kern:.1f} us: table reads {contig_kern / packed_kern - 1:.2%}, "
                f"scatter {kern_mean / contig_kern - 1:.2%}")
        log(f"decode call paged {paged_us:.1f} us, contiguous {contig_us:.1f} us "
            f"(overhead {paged_us / contig_us - 1:.2%}); attention kernel paged {kern_mean:.1f} us, "
            f"contiguous {contig_kern:.1f} us (overhead {kern_mean / contig_kern - 1:.2%})")
        del dc

    if args.copy_calibration:
        copy_calibration(dev)

    if not args.no_ceilings:
        result["ceilings"] = bench_ceilings(w, d, dev, stream, kern_mean)

    if not args.no_bs32 and args.config == 5 and args.block_size == 16 \
            and not args.shared_prefix:
        result["block_size_32"] = bench_block_size_32(args, dev, stream)

    if not args.no_shared_prefix and args.config == 5:
        result["shared_prefix"] = bench_shared_prefix(args, dev, stream)

    if which and args.config == 5 and not args.shared_prefix:
        result["configs"] = bench_configs(args, dev, stream, which)

    if not args.no_blocks:
        result["blocks"] = bench_blocks(args, w, d, dev, stream)

    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        import oracle
        # Whole oracle steps, at least 3 and until about 10 s of CPU work.
        reps = []
        with threadpool_limits(1):
            r = 0
            while r < 3 or (sum(reps) < 10.0 and r < 50):
                r += 1
                t = time.perf_counter()
                kr, vr = oracle.write_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping,
                                         w.block_size)
                ref = oracle.decode(w.q, kr, vr, w.block_tables, w.context_lens, w.scale,
                                    w.block_size, w.kv_dtype)
                reps.append(time.perf_counter() - t)
                log(f"oracle step {r}: {reps[-1]:.2f} s")
        tcpu = statistics.median(reps)
        result["cpu_baseline"] = {
            "value": round(kv_bytes / tcpu / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"the whole step (write + decode of all {w.num_seqs} sequences, "
                      f"{int(w.context_lens.sum())} context tokens), median of {len(reps)} "
                      f"steps ({sum(reps):.1f} s of CPU work), NumPy BLAS "
                      f"limited to 1 thread; host has {len(os.sched_getaffinity(0))} usable cores",
            "seq_steps_per_s": round(w.num_seqs / tcpu, 2),
        }
        err = float(np.abs(out_gpu - ref).max())
        result["max_abs_err_vs_oracle"] = float(f"{err:.3e}")
        log(f"max-abs err vs oracle {err:.3e}")

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
