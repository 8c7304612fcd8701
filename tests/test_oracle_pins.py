"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each check is written as a function of the decode / write implementation
so that the same checks can be run against deliberately broken copies of
the oracle (planted mistakes, at the end of this file) and shown to fail.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_349_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_mapping_example.txt")


# ---------------------------------------------------------------------------
# helpers: random logical sequences placed in a pool through a table
# ---------------------------------------------------------------------------

def _random_paged(rng, lens, Hq, Hkv, D, bs, dtype="f32", extra_blocks=3, shuffle=True):
    """Logical K/V per sequence plus a paged pool holding them (tables random)."""
    nblk = [(L + bs - 1) // bs for L in lens]
    NB = sum(nblk) + extra_blocks
    ids = rng.permutation(NB) if shuffle else np.arange(NB)
    tables = np.full((len(lens), max(max(nblk), 1)), -1, dtype=np.int32)
    c = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = ids[c:c + n]
        c += n
    if dtype == "f32":
        lk = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
        lv = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
        q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
        fill = np.float32(np.nan)
    else:
        lk = [wl.f32_to_bf16_bits(rng.standard_normal((Hkv, L, D))) for L in lens]
        lv = [wl.f32_to_bf16_bits(rng.standard_normal((Hkv, L, D))) for L in lens]
        q = wl.f32_to_bf16_bits(rng.standard_normal((len(lens), Hq, D)))
        fill = np.uint16(0x7FC0)
    kc, vc = wl.pack_logical(lk, lv, tables, NB, bs, fill)
    return lk, lv, q, kc, vc, tables, np.array(lens, dtype=np.int32)


def _sdpa(qs, K, V, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU, one query per head.

    qs [H, D], K/V [H, L, D] (float64) -> [H, D]
    """
    qt = torch.from_numpy(np.ascontiguousarray(qs))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V))[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0, :].numpy()


def _torch_bf16_to_f64(bits):
    """bf16 bit patterns -> float64 through torch's own bfloat16 type (not the oracle's code)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _bf16_from_fields(bits):
    """Value of one bf16 pattern from the format's definition, as an mpmath number:
    1 sign bit, 8 exponent bits (bias 127), 7 fraction bits; exponent 0 holds
    zero and the subnormals (fraction * 2^-133), exponent 255 infinities and NaNs."""
    import mpmath
    bits = int(bits)
    sign = -1 if bits >> 15 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return mpmath.nan if f else sign * mpmath.inf
    if e == 0:
        return sign * mpmath.mpf(f) * mpmath.mpf(2) ** -133
    return sign * (1 + mpmath.mpf(f) / 128) * mpmath.mpf(2) ** (e - 127)


# ---------------------------------------------------------------------------
# pin functions (each returns the max deviation or raises AssertionError)
# ---------------------------------------------------------------------------

def pin_library_routine(decode, seed=0):
    """P1 + P8: paged oracle == torch SDPA (fp64) on the logical tensors.

    Covers MHA (G=1) and GQA (G=4) with the KV heads expanded per query head,
    shuffled tables, block sizes 1, 4, 16, 32 and 48 (V in 16-token sub-tiles
    for the last two) and ragged lengths.
    """
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (Hq, Hkv, D, bs, lens) in [(4, 4, 16, 16, [1, 17, 40, 5]),
                                   (8, 2, 8, 4, [3, 9, 30]),
                                   (6, 3, 4, 1, [7, 2]),
                                   (4, 1, 32, 16, [64, 33]),
                                   (4, 2, 8, 32, [70, 33, 1]),
                                   (2, 1, 4, 48, [100, 47])]:
        lk, lv, q, kc, vc, tables, L = _random_paged(rng, lens, Hq, Hkv, D, bs)
        sc = np.float32(1.0 / math.sqrt(D))
        out = decode(q, kc, vc, tables, L, sc, bs, "f32")
        G = Hq // Hkv
        for s in range(len(lens)):
            K = np.repeat(lk[s].astype(np.float64), G, axis=0)   # expanded per query head
            V = np.repeat(lv[s].astype(np.float64), G, axis=0)
            ref = _sdpa(q[s].astype(np.float64), K, V, float(sc))
            worst = max(worst, float(np.abs(out[s] - ref).max()))
    assert worst < 1e-12, worst
    return worst


def pin_library_routine_bf16(decode, seed=10):
    """P1 + P8 on bf16 KV: the oracle's bf16 path == torch SDPA (fp64) on values
    widened by torch's bfloat16 type.

    Block sizes 4, 16, 32 and 48 (two and three 16-token V sub-tiles for the
    last two), GQA by head expansion, ragged lengths, shuffled tables.
    """
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (Hq, Hkv, D, bs, lens) in [(4, 4, 16, 16, [1, 17, 40]),
                                   (8, 2, 8, 4, [3, 9, 30]),
                                   (8, 1, 32, 32, [70, 33, 1]),
                                   (4, 2, 8, 48, [100, 47, 49])]:
        lk, lv, q, kc, vc, tables, L = _random_paged(rng, lens, Hq, Hkv, D, bs, dtype="bf16")
        sc = np.float32(1.0 / math.sqrt(D))
        out = decode(q, kc, vc, tables, L, sc, bs, "bf16")
        G = Hq // Hkv
        for s in range(len(lens)):
            K = np.repeat(_torch_bf16_to_f64(lk[s]), G, axis=0)
            V = np.repeat(_torch_bf16_to_f64(lv[s]), G, axis=0)
            ref = _sdpa(_torch_bf16_to_f64(q[s]), K, V, float(sc))
            worst = max(worst, float(np.abs(out[s] - ref).max()))
    assert worst < 1e-12, worst
    return worst


def pin_brute_force_bf16(decode, cases=12, seed=11):
    """P7 on bf16 KV: 50-digit scalar loops over values decoded from the bf16
    format's fields (sign, exponent, fraction), at block sizes 16 and 32."""
    import mpmath
    mpmath.mp.dps = 50
    rng = np.random.default_rng(seed)
    worst = 0.0
    for c in range(cases):
        bs = [16, 32][c % 2]
        Hkv = 1 + c % 2
        G = 1 + (c // 2) % 3
        D = 1 + int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(1, 70, size=1 + c % 2)]
        lk, lv, q, kc, vc, tables, L = _random_paged(rng, lens, Hkv * G, Hkv, D, bs, dtype="bf16")
        sc = np.float32(rng.uniform(0.1, 1.0))
        out = decode(q, kc, vc, tables, L, sc, bs, "bf16")
        scm = mpmath.mpf(float(sc))
        for s, Ls in enumerate(lens):
            for h in range(Hkv * G):
                kv = h // G
                qv = [_bf16_from_fields(q[s, h, d]) for d in range(D)]
                x = [scm * mpmath.fsum(qv[d] * _bf16_from_fields(lk[s][kv, t, d]) for d in range(D))
                     for t in range(Ls)]
                mx = max(x)
                w = [mpmath.exp(xi - mx) for xi in x]
                den = mpmath.fsum(w)
                for d in range(D):
                    num = mpmath.fsum(w[t] * _bf16_from_fields(lv[s][kv, t, d]) for t in range(Ls))
                    worst = max(worst, abs(float(num / den) - out[s, h, d]))
    assert worst < 1e-13, worst
    return worst


def pin_widen_bf16(widen):
    """The oracle's bf16 widening: every one of the 65536 bit patterns against
    torch's bfloat16 -> float64 conversion (NaNs as NaNs), and a table of
    patterns against the format's definition (zeros, subnormals, the smallest
    and largest normals, infinities)."""
    import mpmath
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):      # signalling NaN patterns
        got = widen(bits, "bf16")
    ref = _torch_bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    table = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x4049, 0x3E00,
             0x7F7F, 0xFF7F, 0x7F80, 0xFF80]
    for b in table:
        v = widen(np.array([b], np.uint16), "bf16")[0]
        assert mpmath.mpf(float(v)) == _bf16_from_fields(b), hex(b)
        assert math.copysign(1.0, float(v)) == (-1.0 if b >> 15 else 1.0), hex(b)


def pin_brute_force(decode, cases=20, seed=1):
    """P7: 50-digit scalar loops (mpmath) on tiny random paged cases."""
    import mpmath
    mpmath.mp.dps = 50
    rng = np.random.default_rng(seed)
    worst = 0.0
    for c in range(cases):
        bs = [1, 2, 4, 16, 32][c % 5]
        Hkv = 1 + c % 2
        G = 1 + (c // 2) % 3
        D = 1 + int(rng.integers(1, 8))
        lens = [int(x) for x in rng.integers(1, 40, size=1 + c % 3)]
        lk, lv, q, kc, vc, tables, L = _random_paged(rng, lens, Hkv * G, Hkv, D, bs)
        sc = np.float32(rng.uniform(0.1, 1.0))
        out = decode(q, kc, vc, tables, L, sc, bs, "f32")
        scm = mpmath.mpf(float(sc))
        for s, Ls in enumerate(lens):
            for h in range(Hkv * G):
                kv = h // G
                x = [scm * mpmath.fsum(mpmath.mpf(float(q[s, h, d])) * mpmath.mpf(float(lk[s][kv, t, d]))
                                       for d in range(D)) for t in range(Ls)]
                mx = max(x)
                w = [mpmath.exp(xi - mx) for xi in x]
                den = mpmath.fsum(w)
                for d in range(D):
                    num = mpmath.fsum(w[t] * mpmath.mpf(float(lv[s][kv, t, d])) for t in range(Ls))
                    worst = max(worst, abs(float(num / den) - out[s, h, d]))
    assert worst < 1e-13, worst
    return worst


def pin_shuffle_invariance(decode, seed=2):
    """P2: moving physical blocks and rewriting the tables gives bitwise-identical output."""
    w = wl.make_config(1, seed=seed)
    k, v = oracle.write_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping, w.block_size)
    base = decode(w.q, k, v, w.block_tables, w.context_lens, w.scale, w.block_size, w.kv_dtype)
    rng = np.random.default_rng(seed + 100)
    w2 = wl.permute_pool(w, rng.permutation(w.num_blocks))
    k2, v2 = oracle.write_kv(w2.k_cache, w2.v_cache, w2.k_new, w2.v_new, w2.slot_mapping,
                             w2.block_size)
    out2 = decode(w2.q, k2, v2, w2.block_tables, w2.context_lens, w2.scale, w2.block_size,
                  w2.kv_dtype)
    assert np.array_equal(base.view(np.uint64), out2.view(np.uint64))


def pin_closed_forms(decode, seed=3):
    """P4, P5, P6: L=1 returns V[0] exactly; q=0 returns the mean of V; constant V returns it."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 4, 2, 8, 4
    lk, lv, q, kc, vc, tables, L = _random_paged(rng, [1, 13, 29], Hq, Hkv, D, bs)
    sc = np.float32(0.5)
    out = decode(q, kc, vc, tables, L, sc, bs, "f32")
    G = Hq // Hkv
    for h in range(Hq):                       # P4: softmax of one score is exactly 1
        assert np.array_equal(out[0, h], lv[0][h // G, 0].astype(np.float64))
    qz = np.zeros_like(q)
    outz = decode(qz, kc, vc, tables, L, sc, bs, "f32")
    for s in (1, 2):                          # P5: uniform weights
        for h in range(Hq):
            ref = np.mean(lv[s][h // G].astype(np.float64), axis=0)
            assert np.abs(outz[s, h] - ref).max() < 1e-14
    lvc = [np.broadcast_to(rng.standard_normal((Hkv, 1, D)).astype(np.float32), x.shape).copy()
           for x in lv]
    kc2, vc2 = wl.pack_logical(lk, lvc, tables, kc.shape[0], bs, np.float32(np.nan))
    outc = decode(q, kc2, vc2, tables, L, sc, bs, "f32")
    for s in range(3):                        # P6: convex combination of equal rows
        for h in range(Hq):
            assert np.abs(outc[s, h] - lvc[s][h // G, 0]).max() < 1e-14


def pin_shared_blocks(decode, seed=4):
    """P3: sequences on the same physical blocks with equal q and L agree bitwise,
    and so do sequences on separate physical copies of the same content."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 4, 2, 16, 4
    lk, lv, q, kc, vc, tables, L = _random_paged(rng, [22], Hq, Hkv, D, bs, dtype="bf16",
                                                 extra_blocks=10)
    n = (22 + bs - 1) // bs
    # three sequences: two share seq 0's blocks, the third reads copies of them
    free = [b for b in range(kc.shape[0]) if b not in set(tables[0, :n].tolist())]
    copy_ids = np.array(free[:n], dtype=np.int32)
    kc[copy_ids] = kc[tables[0, :n]]
    vc[copy_ids] = vc[tables[0, :n]]
    t3 = np.stack([tables[0], tables[0], copy_ids])
    q3 = np.stack([q[0], q[0], q[0]])
    out = decode(q3, kc, vc, t3, np.array([22, 22, 22], np.int32), np.float32(0.25), bs, "bf16")
    assert np.array_equal(out[0].view(np.uint64), out[1].view(np.uint64))
    assert np.array_equal(out[0].view(np.uint64), out[2].view(np.uint64))


def pin_split_merge(seed=5):
    """P9: merging partial states of arbitrary cuts equals the unsplit result."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for _ in range(10):
        L = int(rng.integers(2, 300))
        D = 8
        K = rng.standard_normal((L, D)) * 3
        V = rng.standard_normal((L, D))
        qv = rng.standard_normal(D)
        full = oracle.attention_one(qv, K, V, 0.7)
        cuts = sorted(set(rng.integers(1, L, size=int(rng.integers(1, 6))).tolist()))
        edges = [0] + cuts + [L]
        states = [oracle.partial_state(qv, K, V, 0.7, a, b) for a, b in zip(edges, edges[1:])]
        worst = max(worst, float(np.abs(oracle.merge_states(states) - full).max()))
    assert worst < 1e-13, worst
    return worst


def pin_write_readback(write_kv, seed=6):
    """P10: each new token's bits land in its slot; every other element of the
    pool is unchanged.

    The expected pool is built element by element from the layout as the C
    header documents it (token o, feature d of block b: K at [b, h, o, d], V at
    [b, h, (o // T) * D + d, o % T] with T = 16 when 16 divides the block
    size), at block sizes 16 and 32, with NaN and finite poison.
    """
    for i, poison, bs, ns in [(1, "nan", None, None), (2, "finite", None, 6),
                              (5, "nan", 32, 12), (5, "finite", 32, 7)]:
        w = wl.make_config(i, seed=seed, poison=poison, block_size=bs, num_seqs=ns)
        k2, v2 = write_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping, w.block_size)
        raw = (lambda a: a.view(np.uint32)) if w.kv_dtype == "f32" else (lambda a: a)
        exp_k, exp_v = raw(w.k_cache).copy(), raw(w.v_cache).copy()
        T = 16 if w.block_size % 16 == 0 else w.block_size
        D = w.head_dim
        for t, slot in enumerate(w.slot_mapping):
            b, o = divmod(int(slot), w.block_size)
            for h in range(w.num_kv_heads):
                for d in range(D):
                    exp_k[b, h, o, d] = raw(w.k_new)[t, h, d]
                    exp_v[b, h, (o // T) * D + d, o % T] = raw(w.v_new)[t, h, d]
        assert np.array_equal(raw(k2), exp_k)
        assert np.array_equal(raw(v2), exp_v)


def pin_write_matches_packing(write_kv, seed=12):
    """P10 through the input generator's independently written placement
    (workloads.pack_logical): writing each sequence's last token into a pool
    that holds the others gives, bit for bit, the pool packed with every token.
    Block sizes 4, 16, 32 and 48 (one, two and three 16-token V sub-tiles),
    tokens at every offset class, fp32 and bf16."""
    rng = np.random.default_rng(seed)
    for (Hkv, D, bs, lens, dt) in [(2, 8, 4, [3, 9, 30], "f32"),
                                   (2, 16, 16, [1, 16, 17, 40], "bf16"),
                                   (3, 8, 32, [32, 17, 33, 64, 50, 2], "bf16"),
                                   (1, 4, 48, [48, 47, 100, 17, 33, 20], "f32")]:
        lk, lv, q, kc, vc, tables, L = _random_paged(rng, lens, Hkv, Hkv, D, bs, dtype=dt)
        fill = np.float32(np.nan) if dt == "f32" else np.uint16(0x7FC0)
        short_k = [x[:, :-1] for x in lk]
        short_v = [x[:, :-1] for x in lv]
        kc0, vc0 = wl.pack_logical(short_k, short_v, tables, kc.shape[0], bs, fill)
        slots = np.array([int(tables[s, (n - 1) // bs]) * bs + (n - 1) % bs
                          for s, n in enumerate(lens)], np.int32)
        k_new = np.stack([x[:, -1] for x in lk])
        v_new = np.stack([x[:, -1] for x in lv])
        k2, v2 = write_kv(kc0, vc0, k_new, v_new, slots, bs)
        raw = (lambda a: a.view(np.uint32)) if dt == "f32" else (lambda a: a)
        assert np.array_equal(raw(k2), raw(kc))
        assert np.array_equal(raw(v2), raw(vc))


def _read_golden():
    rows, opens, blocks = [], [], []
    bs, table = None, None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "block_size":
                bs = int(parts[1])
            elif parts[0] == "table":
                table = [int(x) for x in parts[1:]]
            elif parts[0] == "opens":
                opens.append((int(parts[1]), [int(x) for x in parts[2:]]))
            elif parts[0] == "blocks":
                blocks.append(tuple(int(x) for x in parts[1:]))
            else:
                rows.append((int(parts[0]), int(parts[1])))
    return bs, table, rows, opens, blocks


def pin_pages_mapping(decode, write_kv):
    """P11: the pages' own block-mapping example and allocation trigger.

    A pool where every slot holds its own slot number lets the oracle's
    table read be checked against the printed mapping: with q = 0 and one
    KV head, out is the mean of the V values the oracle gathered.  With
    L = 1 it is exactly the value stored at the first mapped slot.
    """
    bs, table, rows, opens, blocks = _read_golden()
    NB = max(table) + 1
    D = 1
    ids = np.arange(NB * bs, dtype=np.float32).reshape(NB, 1, bs, 1)   # slot number per slot
    kc = np.zeros((NB, 1, bs, D), np.float32)
    vc = ids.reshape(NB, 1, 1, bs).copy()
    tab = np.array([table], dtype=np.int32)
    q = np.zeros((1, 1, D), np.float32)
    for pos, slot in rows:
        out = decode(q, kc, vc, tab, np.array([pos + 1], np.int32), np.float32(1.0), bs, "f32")
        expect = np.mean([s for p, s in _all_slots(table, bs)[:pos + 1]])
        assert abs(out[0, 0, 0] - expect) < 1e-9, (pos, out, expect)
        assert _all_slots(table, bs)[pos][1] == slot
    # a write to the printed slot lands in the printed (block, offset)
    for pos, slot in rows:
        k2, v2 = write_kv(kc, vc, np.ones((1, 1, D), np.float32), np.full((1, 1, D), -7, np.float32),
                          np.array([slot], np.int32), bs)
        assert v2[table[pos // bs], 0, 0, pos % bs] == -7
        assert wl.new_token_slot(np.array(table), pos + 1, bs) == slot
    # the allocation trigger: blocks opened at lengths 1, bs+1, 2bs+1, ...
    for bsz, lengths in opens:
        got = [L for L in range(1, lengths[-1] + 1) if L % bsz == 1 or bsz == 1]
        assert got == lengths, (bsz, got)
    for bsz, L, n in blocks:
        assert (L + bsz - 1) // bsz == n
        w = wl.build_workload("g", np.random.default_rng(0), kv_dtype="f32", context_lens=[L],
                              num_heads=1, num_kv_heads=1, head_dim=2, block_size=bsz)
        assert int((w.block_tables[0] >= 0).sum()) == n


def _all_slots(table, bs):
    return [(p, table[p // bs] * bs + p % bs) for p in range(len(table) * bs)]


# ---------------------------------------------------------------------------
# the pins, on the oracle
# ---------------------------------------------------------------------------

def test_oracle_matches_sdpa():
    pin_library_routine(oracle.decode)


def test_oracle_brute_force_mpmath():
    pin_brute_force(oracle.decode)


def test_oracle_bf16_matches_sdpa():
    pin_library_routine_bf16(oracle.decode)


def test_oracle_bf16_brute_force_mpmath():
    pin_brute_force_bf16(oracle.decode)


def test_oracle_bf16_widening():
    pin_widen_bf16(oracle.widen)


def test_oracle_write_matches_packing():
    pin_write_matches_packing(oracle.write_kv)


def test_oracle_shuffle_invariance():
    pin_shuffle_invariance(oracle.decode)


def test_oracle_closed_forms():
    pin_closed_forms(oracle.decode)


def test_oracle_shared_blocks():
    pin_shared_blocks(oracle.decode)


def test_oracle_split_merge():
    pin_split_merge()


def test_oracle_write_readback():
    pin_write_readback(oracle.write_kv)


def test_oracle_pages_mapping_example():
    pin_pages_mapping(oracle.decode, oracle.write_kv)


def test_oracle_zero_length_sequence():
    """L = 0 is a no-op sequence: its output is zero and others are unaffected."""
    rng = np.random.default_rng(7)
    lk, lv, q, kc, vc, tables, L = _random_paged(rng, [5, 9], 2, 2, 4, 4)
    L0 = np.array([0, 9], np.int32)
    out = oracle.decode(q, kc, vc, tables, L0, np.float32(0.5), 4, "f32")
    ref = oracle.decode(q, kc, vc, tables, L, np.float32(0.5), 4, "f32")
    assert np.all(out[0] == 0)
    assert np.array_equal(out[1], ref[1])


# ---------------------------------------------------------------------------
# planted mistakes: each broken copy of the oracle must fail at least one pin
# ---------------------------------------------------------------------------

def _mutant_widen(kind):
    def widen(x, kv_dtype):
        with np.errstate(invalid="ignore"):
            return _widen(x, kv_dtype)

    def _widen(x, kv_dtype):
        if kv_dtype == "bf16" and kind == "bf16_as_fp16":      # bits read as IEEE half
            return x.view(np.float16).astype(np.float64)
        if kv_dtype == "bf16" and kind == "bf16_shift15":      # fraction misplaced by one bit
            return (x.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
        if kv_dtype == "bf16" and kind == "bf16_truncated":    # low fraction bit dropped
            return ((x & np.uint16(0xFFFE)).astype(np.uint32) << np.uint32(16)).view(
                np.float32).astype(np.float64)
        return oracle.widen(x, kv_dtype)
    return widen


def _mutant_decode(kind):
    wid = _mutant_widen(kind)

    def decode(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, kv_dtype):
        S, Hq, D = q.shape
        Hkv = k_cache.shape[1]
        G = Hq // Hkv
        sc = float(np.float32(scale))
        qd = wid(q, kv_dtype)
        out = np.zeros((S, Hq, D))
        for s in range(S):
            L = int(context_lens[s])
            if L == 0:
                continue
            Lr = L - 1 if (kind == "drop_last_token" and L > 1) else L
            pos = np.arange(Lr)
            bl = block_tables[s][pos // block_size].astype(np.int64)
            if kind == "offset_from_block":
                bl = block_tables[s][pos % max(1, (L + block_size - 1) // block_size)].astype(np.int64)
            off = pos % block_size
            K = wid(k_cache[bl, :, off, :], kv_dtype).transpose(1, 0, 2)
            if kind == "v_whole_block_tile":             # V feature-major over the whole block
                whole = v_cache.reshape(v_cache.shape[0], Hkv, D, block_size)
                V = wid(whole[bl, :, :, off], kv_dtype)
                V = V.transpose(1, 0, 2)
            elif kind == "v_as_k_layout":
                V = wid(v_cache.reshape(k_cache.shape)[bl, :, off, :], kv_dtype)
                V = V.transpose(1, 0, 2)
            else:
                T = v_cache.shape[3]           # feature-major sub-tiles of T tokens
                rows = (off // T)[:, None] * D + np.arange(D)[None, :]
                V = wid(v_cache[bl[:, None], :, rows, (off % T)[:, None]], kv_dtype)
                V = V.transpose(2, 0, 1)
            for h in range(Hq):
                kv = (h % Hkv) if kind == "gqa_modulo" else h // G
                x = (1.0 if kind == "no_scale" else sc) * (K[kv] @ qd[s, h])
                if kind == "neg_scores":
                    x = -x
                x = x - x.max()
                p = np.exp(x)
                den = p.sum() if kind != "no_normalise" else 1.0
                out[s, h] = (p @ V[kv]) / den
        return out
    return decode


def _fails_some_pin(dec):
    pins = [pin_library_routine, pin_brute_force, pin_library_routine_bf16, pin_brute_force_bf16,
            pin_shuffle_invariance, pin_closed_forms, pin_shared_blocks,
            lambda d: pin_pages_mapping(d, oracle.write_kv)]
    for pin in pins:
        try:
            if pin is pin_brute_force:
                pin(dec, cases=6)
            elif pin is pin_brute_force_bf16:
                pin(dec, cases=4)
            else:
                pin(dec)
        except (AssertionError, IndexError, ValueError):
            return True
    return False


@pytest.mark.parametrize("kind", ["drop_last_token", "offset_from_block", "v_as_k_layout",
                                  "v_whole_block_tile",
                                  "gqa_modulo", "no_scale", "neg_scores", "no_normalise",
                                  "bf16_as_fp16", "bf16_shift15", "bf16_truncated"])
def test_planted_mistake_is_caught(kind):
    assert _fails_some_pin(_mutant_decode(kind)), kind


@pytest.mark.parametrize("kind", ["bf16_as_fp16", "bf16_shift15", "bf16_truncated"])
def test_planted_widen_mistake_is_caught(kind):
    with pytest.raises(AssertionError):
        pin_widen_bf16(_mutant_widen(kind))


def test_unmutated_copy_passes_pins():
    assert not _fails_some_pin(_mutant_decode("none"))


def _mutant_write(kind):
    def write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, block_size):
        k, v = k_cache.copy(), v_cache.copy()
        D = k.shape[3]
        T = v.shape[3]
        for t, slot in enumerate(slot_mapping):
            if slot < 0:
                continue
            b, o = divmod(int(slot), block_size)
            if kind == "swap_block_offset":
                b, o = o % k.shape[0], b % block_size
            k[b, :, o, :] = k_new[t]
            row = (o // T) * D
            if kind == "v_subtile0":                 # every token into the first sub-tile
                row = 0
            if kind == "v_untransposed":
                v.reshape(k.shape)[b, :, o, :] = v_new[t]
            else:
                v[b, :, row:row + D, o % T] = v_new[t]
        return k, v
    return write_kv


def _write_fails_some_pin(write):
    for pin in (pin_write_readback, pin_write_matches_packing):
        try:
            pin(write)
        except (AssertionError, IndexError, ValueError):
            return True
    return False


@pytest.mark.parametrize("kind", ["swap_block_offset", "v_untransposed", "v_subtile0"])
def test_planted_write_mistake_is_caught(kind):
    assert _write_fails_some_pin(_mutant_write(kind)), kind


def test_unmutated_write_copy_passes_pins():
    assert not _write_fails_some_pin(_mutant_write("none"))
