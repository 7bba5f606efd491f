"""ctypes binding of the host block manager (include/pa_block_manager.h): marshalling only.

The bookkeeping (free list, reference counts, prefix cache, copy-on-write) runs in the C++
code of libpa.so; this class passes numpy buffers to it and raises PAError on a non-zero
status.  Host only: nothing here touches the GPU.
"""
import ctypes

import numpy as np

from .pa import PAError, lib

_L = lib()
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)

_L.pa_bm_create.restype = _vp
_L.pa_bm_create.argtypes = [_i32, _i32, _i32]
_L.pa_bm_destroy.restype = None
_L.pa_bm_destroy.argtypes = [_vp]
_L.pa_bm_num_free_blocks.restype = _i32
_L.pa_bm_num_free_blocks.argtypes = [_vp]
_L.pa_bm_ref_count.restype = _i32
_L.pa_bm_ref_count.argtypes = [_vp, _i32]
_L.pa_bm_seq_len.restype = _i32
_L.pa_bm_seq_len.argtypes = [_vp, _i32]
_L.pa_bm_add_sequence.restype = ctypes.c_int
_L.pa_bm_add_sequence.argtypes = [_vp, _i32p, _i32, _i32p, _i32p]
_L.pa_bm_fork.restype = ctypes.c_int
_L.pa_bm_fork.argtypes = [_vp, _i32, _i32p]
_L.pa_bm_append.restype = ctypes.c_int
_L.pa_bm_append.argtypes = [_vp, _i32, _i32p, _i32, _i64p]
_L.pa_bm_slots.restype = ctypes.c_int
_L.pa_bm_slots.argtypes = [_vp, _i32, _i32, _i32, _i64p]
_L.pa_bm_free_sequence.restype = ctypes.c_int
_L.pa_bm_free_sequence.argtypes = [_vp, _i32]
_L.pa_bm_num_pending_copies.restype = ctypes.c_int64
_L.pa_bm_num_pending_copies.argtypes = [_vp]
_L.pa_bm_take_copies.restype = ctypes.c_int64
_L.pa_bm_take_copies.argtypes = [_vp, _i64p, ctypes.c_int64]
_L.pa_bm_set_host_blocks.restype = ctypes.c_int
_L.pa_bm_set_host_blocks.argtypes = [_vp, _i32]
_L.pa_bm_num_free_host_blocks.restype = ctypes.c_int32
_L.pa_bm_num_free_host_blocks.argtypes = [_vp]
for _fn in (_L.pa_bm_swap_out, _L.pa_bm_swap_in):
    _fn.restype = ctypes.c_int
    _fn.argtypes = [_vp, _i32, _i64p, ctypes.c_int64, _i64p]
_L.pa_bm_block_tables.restype = ctypes.c_int
_L.pa_bm_block_tables.argtypes = [_vp, _i32p, _i32, _i32, _i32p, _i32p]
_L.pa_bm_prefix_groups.restype = ctypes.c_int
_L.pa_bm_prefix_groups.argtypes = [_vp, _i32p, _i32, _i32, _i32p, _i32p, _i32p]


def _check(fn, code):
    if code != 0:
        raise PAError(fn, code)


def _ids(tokens):
    if tokens is None:
        return None, None
    a = np.ascontiguousarray(tokens, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


class BlockManager:
    """Owner of a pool's block bookkeeping; see include/pa_block_manager.h."""

    def __init__(self, num_blocks: int, block_size: int = 16, max_blocks_per_seq: int = 128):
        self._h = _L.pa_bm_create(int(num_blocks), int(block_size), int(max_blocks_per_seq))
        if not self._h:
            raise ValueError("pa_bm_create: invalid sizes")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.max_blocks_per_seq = int(max_blocks_per_seq)

    def close(self):
        if self._h:
            _L.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # ------------------------------------------------------------------ queries
    def num_free_blocks(self) -> int:
        return int(_L.pa_bm_num_free_blocks(self._h))

    def ref_count(self, block: int) -> int:
        return int(_L.pa_bm_ref_count(self._h, int(block)))

    def seq_len(self, seq: int) -> int:
        return int(_L.pa_bm_seq_len(self._h, int(seq)))

    # ------------------------------------------------------------------ sequences
    def add_sequence(self, num_tokens: int, token_ids=None):
        """Returns (seq_id, num_cached_tokens)."""
        a, p = _ids(token_ids)
        if a is not None:
            assert a.size == num_tokens
        sid, cached = ctypes.c_int32(), ctypes.c_int32()
        _check("pa_bm_add_sequence",
               _L.pa_bm_add_sequence(self._h, p, int(num_tokens), ctypes.byref(sid),
                                     ctypes.byref(cached)))
        return sid.value, cached.value

    def fork(self, parent: int) -> int:
        cid = ctypes.c_int32()
        _check("pa_bm_fork", _L.pa_bm_fork(self._h, int(parent), ctypes.byref(cid)))
        return cid.value

    def append(self, seq: int, num_tokens: int, token_ids=None) -> np.ndarray:
        """Grow `seq` by num_tokens; returns their slots (int64)."""
        a, p = _ids(token_ids)
        if a is not None:
            assert a.size == num_tokens
        out = np.empty(int(num_tokens), dtype=np.int64)
        _check("pa_bm_append", _L.pa_bm_append(self._h, int(seq), p, int(num_tokens),
                                               out.ctypes.data_as(_i64p)))
        return out

    def slots(self, seq: int, first: int, count: int) -> np.ndarray:
        out = np.empty(int(count), dtype=np.int64)
        _check("pa_bm_slots", _L.pa_bm_slots(self._h, int(seq), int(first), int(count),
                                             out.ctypes.data_as(_i64p)))
        return out

    def free_sequence(self, seq: int):
        _check("pa_bm_free_sequence", _L.pa_bm_free_sequence(self._h, int(seq)))

    # ------------------------------------------------------------------ swapping
    def set_host_blocks(self, num_host_blocks: int):
        _check("pa_bm_set_host_blocks", _L.pa_bm_set_host_blocks(self._h, int(num_host_blocks)))

    def num_free_host_blocks(self) -> int:
        return int(_L.pa_bm_num_free_host_blocks(self._h))

    def swap_out(self, seq: int) -> np.ndarray:
        """Move `seq` to host blocks; returns (device block, host block) pairs, int64 [n, 2],
        for pa_swap_blocks(..., SWAP_OUT)."""
        out, n = np.empty((self.max_blocks_per_seq, 2), dtype=np.int64), ctypes.c_int64()
        _check("pa_bm_swap_out", _L.pa_bm_swap_out(self._h, int(seq), out.ctypes.data_as(_i64p),
                                                   out.shape[0], ctypes.byref(n)))
        return out[:n.value].copy()

    def swap_in(self, seq: int) -> np.ndarray:
        """Bring `seq` back onto fresh device blocks; returns (host block, device block)
        pairs, int64 [n, 2], for pa_swap_blocks(..., SWAP_IN)."""
        out, n = np.empty((self.max_blocks_per_seq, 2), dtype=np.int64), ctypes.c_int64()
        _check("pa_bm_swap_in", _L.pa_bm_swap_in(self._h, int(seq), out.ctypes.data_as(_i64p),
                                                 out.shape[0], ctypes.byref(n)))
        return out[:n.value].copy()

    # ------------------------------------------------------------------ outputs
    def take_copies(self) -> np.ndarray:
        """Queued copy-on-write pairs, int64 [n, 2] (source, destination), oldest first."""
        n = int(_L.pa_bm_num_pending_copies(self._h))
        out = np.empty((n, 2), dtype=np.int64)
        got = int(_L.pa_bm_take_copies(self._h, out.ctypes.data_as(_i64p), n))
        assert got == n
        return out

    def block_tables(self, seq_ids, pad_block: int = 0):
        """(tables int32 [n, max_blocks_per_seq], context_lens int32 [n]) for pa_decode."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        tables = np.empty((ids.size, self.max_blocks_per_seq), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        _check("pa_bm_block_tables",
               _L.pa_bm_block_tables(self._h, ids.ctypes.data_as(_i32p), int(ids.size),
                                     int(pad_block), tables.ctypes.data_as(_i32p),
                                     lens.ctypes.data_as(_i32p)))
        return tables, lens

    def prefix_groups(self, seq_ids, min_blocks: int = 1):
        """(groups int32 [num_groups + 1], blocks int32 [num_groups]) for
        pa_decode_shared_prefix over the sequences in the order of seq_ids."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        groups = np.empty(ids.size + 1, dtype=np.int32)
        blocks = np.empty(max(ids.size, 1), dtype=np.int32)
        ng = ctypes.c_int32()
        _check("pa_bm_prefix_groups",
               _L.pa_bm_prefix_groups(self._h, ids.ctypes.data_as(_i32p), int(ids.size),
                                      int(min_blocks), groups.ctypes.data_as(_i32p),
                                      blocks.ctypes.data_as(_i32p), ctypes.byref(ng)))
        return groups[:ng.value + 1].copy(), blocks[:ng.value].copy()
