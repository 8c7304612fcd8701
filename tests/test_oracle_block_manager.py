"""Pins of the block-manager model and the block copies in oracle/ (CPU only).

Each pin takes the implementation as an argument, so the same checks run on
the oracle's model here and on the C++ manager in test_block_manager.py.
What pins the model, independently of its own code:

* the pages' worked example ("How does vLLM PagedAttention manage Virtual
  Memory Pages ...", sections "Detail" and "Example"): the printed mapping of
  logical blocks 0 and 1 to physical blocks 42 and 105, the front-of-list
  allocation from list(range(total)), and the lengths at which a block opens
  (tests/golden/block_mapping_example.txt);
* a brute-force content model: every slot of a simulated pool holds the tag
  of the token written there; after every operation of long random operation
  sequences, each sequence read through its table must return exactly its own
  token history (paging moves tokens, it never changes them), reference
  counts must equal the number of table entries pointing at each block, and
  the free list must hold exactly the unreferenced blocks.  A missing
  copy-on-write, a free of a shared block, a fork without new references or a
  wrong swap mapping each break it;
* sharing counts ("PagedAttention and KV memory management", "Myths and
  failure modes" and "Key takeaways": forked samples share prompt blocks
  instead of multiplying KV by the sample count);
* closed forms of the waste measures.
Planted mistakes at the bottom check that each pin can fail.
"""
import os

import numpy as np
import pytest

from oracle import block_manager as obm
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_mapping_example.txt")


def _golden():
    table, rows, opens, blocks, bs = None, [], [], [], None
    for line in open(GOLDEN):
        parts = line.split()
        if not parts or parts[0].startswith("#"):
            continue
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


def model_factory(num_device_blocks, num_host_blocks, block_size, max_blocks, free_order=None):
    return obm.BlockManagerModel(num_device_blocks, num_host_blocks, block_size, max_blocks,
                                 device_free_order=free_order)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_pages_example(factory):
    bs, table, rows, opens, blocks = _golden()
    # the printed mapping: a pool whose free list starts 42, 105 gives that table
    NB = 200
    order = [table[0], table[1]] + [b for b in range(NB) if b not in table]
    m = factory(NB, 0, bs, 8, order)
    slots = m.add(0, 32)
    t, lens = m.tables([0])
    assert list(t[0, :2]) == table and lens[0] == 32
    for pos, slot in rows:
        assert slots[pos] == slot, (pos, slots[pos], slot)
    # the sketch's free list is list(range(total)) taken from the front
    m = factory(1000, 0, 16, 64)
    m.add(10, 0)
    m.add(11, 0)
    got = []
    for _ in range(33):
        got.append((m.append(10)[0] // 16, m.append(11)[0] // 16))
    assert got[0] == (0, 1) and got[16] == (2, 3) and got[32] == (4, 5), got
    # the allocation trigger: blocks open at lengths 1, bs+1, 2bs+1, ...
    for bsz, lengths in opens:
        m = factory(100, 0, bsz, 100)
        m.add(7, 0)
        opened = []
        for L in range(1, lengths[-1] + 1):
            before = m.num_free()
            m.append(7)
            if m.num_free() < before:
                opened.append(L)
        assert opened == lengths, (bsz, opened)
    for bsz, L, n in blocks:
        m = factory(100, 0, bsz, 100)
        m.add(1, L)
        assert 100 - m.num_free() == n


class ContentModel:
    """Simulated pools of token tags, driven through a manager's API."""

    def __init__(self, manager, nd, nh, bs):
        self.m, self.bs = manager, bs
        self.pool = [np.full(nd * bs, -1, np.int64), np.full(max(nh, 1) * bs, -1, np.int64)]
        self.hist = {}            # seq -> list of token tags
        self.where = {}
        self.next_tag = 0

    def _tag(self):
        self.next_tag += 1
        return self.next_tag

    def _copy(self, frm, to, pairs):
        for a, b in pairs:
            self.pool[to][b * self.bs:(b + 1) * self.bs] = self.pool[frm][a * self.bs:(a + 1) * self.bs]

    def add(self, sid, n):
        slots = self.m.add(sid, n)
        tags = [self._tag() for _ in range(n)]
        for s, t in zip(slots, tags):
            self.pool[0][s] = t
        self.hist[sid], self.where[sid] = tags, 0

    def append(self, sid):
        slot, src, dst = self.m.append(sid)
        if src >= 0:
            self._copy(0, 0, [(src, dst)])
        t = self._tag()
        self.pool[0][slot] = t
        self.hist[sid].append(t)

    def fork(self, parent, child):
        self.m.fork(parent, child)
        self.hist[child], self.where[child] = list(self.hist[parent]), self.where[parent]

    def free(self, sid):
        self.m.free_seq(sid)
        del self.hist[sid], self.where[sid]

    def swap(self, sids, out):
        pairs = self.m.swap_out(sids) if out else self.m.swap_in(sids)
        self._copy(0 if out else 1, 1 if out else 0, pairs)
        for s in sids:
            self.where[s] = 1 if out else 0

    def check(self, nd, nh):
        """Every invariant the content model can see."""
        refs = [np.zeros(nd, np.int64), np.zeros(max(nh, 1), np.int64)]
        for sid, h in self.hist.items():
            w = self.where[sid]
            table, L = self.m.seq_table(sid)
            assert L == len(h) and len(table) == -(-L // self.bs), (sid, L, len(h), len(table))
            assert len(set(table)) == len(table)
            for b in table:
                refs[w][b] += 1
            got = [self.pool[w][table[p // self.bs] * self.bs + p % self.bs] for p in range(L)]
            assert got == h, (sid, got, h)
        for w, n in ((0, nd), (1, nh)):
            if n == 0:
                continue
            assert list(self.m.refcounts(w)) == list(refs[w])
            free = self.m.free_list(w)
            assert sorted(free) == [b for b in range(n) if refs[w][b] == 0]


def pin_content(factory, seed=0, steps=400, nd=48, nh=24, bs=4, max_blocks=12):
    rng = np.random.default_rng(seed)
    m = factory(nd, nh, bs, max_blocks)
    cm = ContentModel(m, nd, nh, bs)
    next_id = 0
    for _ in range(steps):
        live = sorted(cm.hist)
        on_dev = [s for s in live if cm.where[s] == 0]
        on_host = [s for s in live if cm.where[s] == 1]
        op = rng.choice(["add", "append", "append", "append", "fork", "free", "out", "in"])
        try:
            if op == "add" or not live:
                cm.add(next_id, int(rng.integers(0, 3 * bs)))
                next_id += 1
            elif op == "append" and on_dev:
                cm.append(int(rng.choice(on_dev)))
            elif op == "fork":
                cm.fork(int(rng.choice(live)), next_id)
                next_id += 1
            elif op == "free":
                cm.free(int(rng.choice(live)))
            elif op == "out" and on_dev:
                k = int(rng.integers(1, min(3, len(on_dev)) + 1))
                cm.swap([int(x) for x in rng.choice(on_dev, k, replace=False)], True)
            elif op == "in" and on_host:
                k = int(rng.integers(1, min(3, len(on_host)) + 1))
                cm.swap([int(x) for x in rng.choice(on_host, k, replace=False)], False)
        except obm.BlockManagerError:
            pass                     # out of room: the operation must have changed nothing
        except ValueError as e:      # the C++ binding's error for the same cases
            if "no room" not in str(e) and "PA_ERR_NO_ROOM" not in str(e):
                raise
        cm.check(nd, nh)


def pin_sharing(factory):
    bs = 16
    # 8 samples of a block-aligned 2048-token prompt hold the prompt once
    m = factory(2000, 0, bs, 200)
    m.add(0, 2048)
    for c in range(1, 8):
        m.fork(0, c)
    assert 2000 - m.num_free() == 128
    cows = [m.append(c)[1:] for c in range(8)]
    assert all(src == -1 for src, _ in cows) and 2000 - m.num_free() == 136
    # an unaligned prompt: the last block is shared and partly filled, so
    # every writer but the last one to hold it takes a private copy
    m = factory(2000, 0, bs, 200)
    m.add(0, 2050)
    for c in range(1, 8):
        m.fork(0, c)
    shared_last = m.seq_table(0)[0][-1]
    res = [m.append(c) for c in range(8)]
    copies = [(s, d) for _, s, d in res if s >= 0]
    assert len(copies) == 7 and all(s == shared_last for s, _ in copies)
    assert res[-1][1] == -1 and res[-1][0] // bs == shared_last      # the last holder writes in place
    assert 2000 - m.num_free() == 129 + 7
    # freeing every sample returns every block
    for c in range(8):
        m.free_seq(c)
    assert m.num_free() == 2000


def pin_waste(waste_contiguous, waste_paged):
    # the pages' allocator diagram: 100 tokens used of a 4096-token reservation
    assert abs(waste_contiguous([100], 4096) - 3996 / 4096) < 1e-15
    # paged: 100 tokens take 7 blocks of 16 = 112 slots, 12 unused
    assert abs(waste_paged([100], 16) - 12 / 112) < 1e-15
    # block-aligned lengths waste nothing; one token past a boundary wastes bs-1 slots
    assert waste_paged([32, 64, 16], 16) == 0.0
    assert abs(waste_paged([17, 33], 16) - 30 / 80) < 1e-15
    # "roughly one partly filled block per sequence": never more than bs-1 slots each
    rng = np.random.default_rng(3)
    L = rng.integers(1, 5000, 300)
    wp = waste_paged(L, 16)
    assert wp * (-(-L // 16)).sum() * 16 <= 15 * len(L)
    # sharing: 8 samples of a 2048 prompt + private tails, prompt counted once
    tails = np.array([1, 5, 16, 17, 30, 31, 32, 2])
    lens = 2048 + tails
    w = waste_paged(lens, 16, shared_tokens=7 * 2048, shared_blocks=7 * 128)
    blocks = 128 + (-(-tails // 16)).sum()
    assert abs(w - (1 - (2048 + tails.sum()) / (blocks * 16))) < 1e-15


def pin_copy(copy_blocks, swap_blocks):
    rng = np.random.default_rng(11)
    NB, H, bs, D = 9, 2, 4, 3
    k = rng.standard_normal((NB, H, bs, D)).astype(np.float32)
    v = rng.standard_normal((NB, H, D, bs)).astype(np.float32)
    k.view(np.uint32)[3, 1, 2, 0] = 0x7FC00123          # a NaN payload travels as bits
    src, dst = np.array([3, 0, 5, -1, 2]), np.array([7, 8, 1, 4, 99])
    k2, v2 = copy_blocks(k, v, src, dst)
    for a, b in ((3, 7), (0, 8), (5, 1)):
        assert np.array_equal(k2[b].view(np.uint32), k[a].view(np.uint32))
        assert np.array_equal(v2[b].view(np.uint32), v[a].view(np.uint32))
    for b in (0, 2, 3, 4, 5, 6):                         # untouched (the -1 and 99 pairs skip)
        assert np.array_equal(k2[b].view(np.uint32), k[b].view(np.uint32))
        assert np.array_equal(v2[b].view(np.uint32), v[b].view(np.uint32))
    # the same content in a copied block gives the same attention bits
    q = rng.standard_normal((2, 4, D)).astype(np.float32)
    t1 = np.array([[3, 0, 5]], np.int32)
    t2 = np.array([[7, 8, 1]], np.int32)
    o1 = oracle.decode(q[:1], k2, v2, t1, np.array([11], np.int32), np.float32(0.5), bs, "f32")
    o2 = oracle.decode(q[:1], k2, v2, t2, np.array([11], np.int32), np.float32(0.5), bs, "f32")
    assert np.array_equal(o1.view(np.uint64), o2.view(np.uint64))
    # swap out to a second pool and back restores the bits
    hk = np.zeros((5, H, bs, D), np.float32)
    hv = np.zeros((5, H, D, bs), np.float32)
    hk2, hv2 = swap_blocks(hk, hv, k, v, np.array([6, 2]), np.array([0, 4]))
    k3, v3 = swap_blocks(np.zeros_like(k), np.zeros_like(v), hk2, hv2, np.array([4, 0]),
                         np.array([2, 6]))
    for b in (2, 6):
        assert np.array_equal(k3[b].view(np.uint32), k[b].view(np.uint32))
        assert np.array_equal(v3[b].view(np.uint32), v[b].view(np.uint32))
    assert not k3[0].any() and not v3[5].any()


# ---------------------------------------------------------------------------
# the pins, on the oracle
# ---------------------------------------------------------------------------

class _Wrapped:
    """Adds the inspection calls the content model needs to the oracle model."""

    def __init__(self, m):
        self._m = m

    def __getattr__(self, k):
        return getattr(self._m, k)

    def seq_table(self, sid):
        s = self._m.seqs[sid]
        return list(s["table"]), s["len"]

    def refcounts(self, where):
        return self._m.ref[where]

    def free_list(self, where):
        return list(self._m.free[where])


def wrapped_factory(cls=obm.BlockManagerModel):
    def f(nd, nh, bs, mb, order=None):
        return _Wrapped(cls(nd, nh, bs, mb, device_free_order=order))
    return f


def test_model_pages_example():
    pin_pages_example(wrapped_factory())


@pytest.mark.parametrize("seed", range(4))
def test_model_content(seed):
    pin_content(wrapped_factory(), seed=seed)


def test_model_sharing():
    pin_sharing(wrapped_factory())


def test_waste_closed_forms():
    pin_waste(obm.waste_contiguous, obm.waste_paged)


def test_copy_and_swap():
    pin_copy(obm.copy_blocks, obm.swap_blocks)


def test_model_rejects_without_change():
    m = obm.BlockManagerModel(4, 1, 4, 3)
    m.add(0, 8)
    with pytest.raises(obm.BlockManagerError):
        m.add(1, 12)                    # 3 blocks, 2 free
    assert m.num_free() == 2 and 1 not in m.seqs
    with pytest.raises(obm.BlockManagerError):
        m.swap_out([0])                 # 2 blocks, 1 host block
    assert m.seqs[0]["where"] == obm.DEVICE and m.num_free(obm.HOST) == 1


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

class _NoCow(obm.BlockManagerModel):
    def append(self, sid):
        s = self._seq(sid)
        p = s["len"]
        j, o = divmod(p, self.bs)
        if o == 0:
            s["table"].append(self._take(obm.DEVICE))
        s["len"] = p + 1
        return s["table"][j] * self.bs + o, -1, -1


class _Lifo(obm.BlockManagerModel):
    def _take(self, where):
        b = self.free[where].pop()
        self.ref[where][b] = 1
        return b


class _FreeIgnoresRefs(obm.BlockManagerModel):
    def _release(self, where, b):
        self.ref[where][b] = 0
        if b not in self.free[where]:
            self.free[where].append(b)


class _ForkNoRef(obm.BlockManagerModel):
    def fork(self, parent, child):
        s = self._seq(parent)
        self.seqs[child] = {"table": list(s["table"]), "len": s["len"], "where": s["where"]}


class _SwapNoDedupe(obm.BlockManagerModel):
    def _swap(self, sids, frm, to):
        pairs = []
        for sid in sids:
            s = self.seqs[sid]
            for j, b in enumerate(s["table"]):
                c = self._take(to)
                pairs.append((b, c))
                self._release(frm, b)
                s["table"][j] = c
            s["where"] = to
        return pairs


def _fails(factory):
    for pin in (pin_pages_example, pin_sharing,
                lambda f: [pin_content(f, seed=s) for s in range(4)]):
        try:
            pin(factory)
        except (AssertionError, IndexError, KeyError):
            return True
    return False


@pytest.mark.parametrize("cls", [_NoCow, _Lifo, _FreeIgnoresRefs, _ForkNoRef, _SwapNoDedupe],
                         ids=lambda c: c.__name__)
def test_planted_manager_mistake_is_caught(cls):
    assert _fails(wrapped_factory(cls))


def test_unmutated_manager_passes():
    assert not _fails(wrapped_factory())


def _copy_k_only(k, v, src, dst):
    k2, _ = obm.copy_blocks(k, v, src, dst)
    return k2, v.copy()


def _swap_reversed_pairs(dk, dv, sk, sv, src, dst):
    return obm.swap_blocks(dk, dv, sk, sv, dst, src)


@pytest.mark.parametrize("copy,swap", [(_copy_k_only, obm.swap_blocks),
                                       (obm.copy_blocks, _swap_reversed_pairs)])
def test_planted_copy_mistake_is_caught(copy, swap):
    with pytest.raises((AssertionError, IndexError)):
        pin_copy(copy, swap)
