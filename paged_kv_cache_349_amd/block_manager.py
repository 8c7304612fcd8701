"""Python binding of the host-side KV block manager in libpa.so.

Argument marshalling only: the free lists, tables, reference counts,
copy-on-write and swap bookkeeping run in C++ (include/block_manager.h).

    m = BlockManager(num_device_blocks, num_host_blocks, block_size, max_blocks_per_seq)
    slots = m.add(seq, num_tokens)                  # prompt slots
    slots, cow_src, cow_dst = m.append_batch(seqs)  # one token each + copy-on-write pairs
    m.fork(parent, child); m.free_seq(seq)
    src, dst = m.swap_out(seqs); src, dst = m.swap_in(seqs)
    tables, lens = m.tables(seqs)                   # int32 [n, max_blocks], [n]
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _check, load_library

PA_POOL_DEVICE = 0
PA_POOL_HOST = 1
PA_ERR_NO_ROOM = 5

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class _Usage(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("device_blocks_used", _i32), ("host_blocks_used", _i32),
                ("device_blocks_shared", _i32), ("device_tokens_logical", _i64),
                ("device_tokens_stored", _i64)]


_SIGNATURES = {
    "pa_bm_create": (ctypes.c_int, [_i32, _i32, _i32, _i32, _vp, ctypes.POINTER(_vp)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add": (ctypes.c_int, [_vp, _i64, _i32, _vp]),
    "pa_bm_append": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, ctypes.POINTER(_i32)]),
    "pa_bm_fork": (ctypes.c_int, [_vp, _i64, _i64]),
    "pa_bm_free": (ctypes.c_int, [_vp, _i64]),
    "pa_bm_swap_out": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_swap_in": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_block_tables": (ctypes.c_int, [_vp, _vp, _i32, _vp, _i32, _vp]),
    "pa_bm_prefix_groups": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, ctypes.POINTER(_i32)]),
    "pa_bm_sequence": (ctypes.c_int, [_vp, _i64, _vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                      ctypes.POINTER(_i32)]),
    "pa_bm_num_free": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_refcounts": (ctypes.c_int, [_vp, _i32, _vp]),
    "pa_bm_free_list": (ctypes.c_int, [_vp, _i32, _vp, ctypes.POINTER(_i32)]),
    "pa_bm_stats": (ctypes.c_int, [_vp, ctypes.POINTER(_Usage)]),
}

_bound = None


def _lib():
    global _bound
    lib = load_library()
    if _bound is not lib:
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _bound = lib
    return lib


class NoRoomError(ValueError):
    """A pool (or a table's max_blocks_per_seq) has no room; nothing changed."""


def _call(status):
    if status == PA_ERR_NO_ROOM:
        raise NoRoomError("PA_ERR_NO_ROOM: " + load_library().pa_last_error().decode())
    _check(status)


def _ptr(a):
    # the buffer's address as an int (ctypes passes it as a void*)
    return a.__array_interface__["data"][0] if a is not None and a.size else None


def _ids(seqs):
    if isinstance(seqs, np.ndarray) and seqs.dtype == np.int64 and seqs.ndim == 1 and \
            seqs.flags.c_contiguous:
        return seqs
    return np.ascontiguousarray(np.asarray(seqs, dtype=np.int64).reshape(-1))


class BlockManager:
    def __init__(self, num_device_blocks, num_host_blocks, block_size, max_blocks_per_seq,
                 device_free_order=None):
        lib = _lib()
        self.num_device_blocks = int(num_device_blocks)
        self.num_host_blocks = int(num_host_blocks)
        self.block_size = int(block_size)
        self.max_blocks = int(max_blocks_per_seq)
        order = None
        if device_free_order is not None:
            order = np.ascontiguousarray(np.asarray(device_free_order, dtype=np.int32))
            if order.shape != (self.num_device_blocks,):
                raise ValueError("device_free_order must list every device block once")
        h = _vp()
        _call(lib.pa_bm_create(self.num_device_blocks, self.num_host_blocks, self.block_size,
                               self.max_blocks, _ptr(order), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            _lib().pa_bm_destroy(self._h)
            self._h = None

    __del__ = close

    # -- operations --------------------------------------------------------
    def add(self, seq, num_tokens):
        slots = np.empty(max(int(num_tokens), 0), dtype=np.int32)
        _call(_lib().pa_bm_add(self._h, int(seq), int(num_tokens), _ptr(slots)))
        return slots

    def append_batch(self, seqs, out=None):
        """One token for each listed sequence: (slots, cow_src, cow_dst).

        out: optional (slots, src, dst) int32 arrays of at least len(seqs)
        entries to write into (e.g. pinned staging buffers); the returned
        arrays are then views of them.
        """
        ids = _ids(seqs)
        n = ids.size
        if out is None:
            out = (np.empty(n, np.int32), np.empty(n, np.int32), np.empty(n, np.int32))
        slots, src, dst = out
        if min(slots.size, src.size, dst.size) < n or not all(
                a.dtype == np.int32 and a.flags.c_contiguous for a in out):
            raise ValueError("out arrays: contiguous int32 with room for every sequence")
        nc = _i32(0)
        _call(_lib().pa_bm_append(self._h, _ptr(ids), n, _ptr(slots), _ptr(src), _ptr(dst),
                                  ctypes.byref(nc)))
        return slots[:n], src[:nc.value], dst[:nc.value]

    def append(self, seq):
        """One token for one sequence: (slot, cow_src, cow_dst), -1 when nothing to copy."""
        slots, src, dst = self.append_batch([seq])
        return int(slots[0]), (int(src[0]) if src.size else -1), (int(dst[0]) if dst.size else -1)

    def fork(self, parent, child):
        _call(_lib().pa_bm_fork(self._h, int(parent), int(child)))

    def free_seq(self, seq):
        _call(_lib().pa_bm_free(self._h, int(seq)))

    def _swap(self, fn, seqs):
        ids = _ids(seqs)
        cap = sum(self.sequence(int(s))[2] for s in ids) if ids.size else 0
        src = np.empty(max(cap, 1), np.int32)
        dst = np.empty(max(cap, 1), np.int32)
        n = _i32(0)
        _call(fn(self._h, _ptr(ids), ids.size, _ptr(src), _ptr(dst), cap, ctypes.byref(n)))
        return src[:n.value].copy(), dst[:n.value].copy()

    def swap_out(self, seqs):
        """Move sequences to the host pool; returns (device ids, host ids) to copy."""
        return self._swap(_lib().pa_bm_swap_out, seqs)

    def swap_in(self, seqs):
        """Move sequences back to the device pool; returns (host ids, device ids) to copy."""
        return self._swap(_lib().pa_bm_swap_in, seqs)

    # -- queries -----------------------------------------------------------
    def tables(self, seqs, stride=None, out=None):
        """Block tables [n, stride] (-1 padded) and lengths [n]; out=(tables, lens) to reuse."""
        ids = _ids(seqs)
        stride = self.max_blocks if stride is None else int(stride)
        if out is None:
            out = (np.empty((ids.size, stride), np.int32), np.empty(ids.size, np.int32))
        t, lens = out
        if t.shape != (ids.size, stride) or lens.shape != (ids.size,) or \
                t.dtype != np.int32 or lens.dtype != np.int32 or not t.flags.c_contiguous:
            raise ValueError("out arrays: int32 [n, stride] and [n]")
        _call(_lib().pa_bm_block_tables(self._h, _ptr(ids), ids.size, _ptr(t), stride, _ptr(lens)))
        return t, lens

    def prefix_groups(self, seqs):
        """(group_starts [G+1], prefix_blocks [G]) int32 for pa_decode_shared_prefix."""
        ids = _ids(seqs)
        gs = np.empty(ids.size + 1, np.int32)
        pb = np.empty(max(ids.size, 1), np.int32)
        ng = _i32(0)
        _call(_lib().pa_bm_prefix_groups(self._h, _ptr(ids), ids.size, _ptr(gs), _ptr(pb),
                                         ctypes.byref(ng)))
        return gs[:ng.value + 1].copy(), pb[:ng.value].copy()

    def sequence(self, seq):
        """(table, length, number of blocks, pool) of one sequence."""
        table = np.empty(self.max_blocks, np.int32)
        L, nb, pool = _i32(0), _i32(0), _i32(0)
        _call(_lib().pa_bm_sequence(self._h, int(seq), _ptr(table), ctypes.byref(L),
                                    ctypes.byref(nb), ctypes.byref(pool)))
        return table[:nb.value].copy(), L.value, nb.value, pool.value

    def num_free(self, pool=PA_POOL_DEVICE):
        n = _i32(0)
        _call(_lib().pa_bm_num_free(self._h, pool, ctypes.byref(n)))
        return n.value

    def refcounts(self, pool=PA_POOL_DEVICE):
        size = self.num_device_blocks if pool == PA_POOL_DEVICE else self.num_host_blocks
        out = np.empty(max(size, 1), np.int32)
        _call(_lib().pa_bm_refcounts(self._h, pool, _ptr(out)))
        return out[:size].copy()

    def free_list(self, pool=PA_POOL_DEVICE):
        size = self.num_device_blocks if pool == PA_POOL_DEVICE else self.num_host_blocks
        out = np.empty(max(size, 1), np.int32)
        n = _i32(0)
        _call(_lib().pa_bm_free_list(self._h, pool, _ptr(out), ctypes.byref(n)))
        return out[:n.value].copy()

    def stats(self):
        u = _Usage()
        _call(_lib().pa_bm_stats(self._h, ctypes.byref(u)))
        r = {k: int(getattr(u, k)) for k, _ in _Usage._fields_}
        used = r["device_blocks_used"] * self.block_size
        r["device_internal_waste"] = 1.0 - r["device_tokens_stored"] / used if used else 0.0
        return r


__all__ = ["BlockManager", "NoRoomError", "PA_POOL_DEVICE", "PA_POOL_HOST"]
