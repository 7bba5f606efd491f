"""ctypes wrapper of the fp64 CPU oracle (oracle/pa_ref.c).  TEST INFRASTRUCTURE ONLY.

Arrays are numpy; pools and stored tensors keep their storage dtype (float32, float16,
or uint16 holding bfloat16 bits).  Every function here only marshals arguments: the
arithmetic is in pa_ref.c.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpa_ref.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)
_vp = ctypes.c_void_p


class Geom(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("k_scale", ctypes.c_double),
                ("v_scale", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.pa_ref_k_offset.restype = ctypes.c_int64
        L.pa_ref_k_offset.argtypes = [ctypes.POINTER(Geom), ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32]
        L.pa_ref_v_offset.restype = ctypes.c_int64
        L.pa_ref_v_offset.argtypes = L.pa_ref_k_offset.argtypes
        L.pa_ref_to_double.restype = None
        L.pa_ref_to_double.argtypes = [_vp, ctypes.c_int32, ctypes.c_int64, _f64p]
        L.pa_ref_reshape_and_cache.restype = ctypes.c_int32
        L.pa_ref_reshape_and_cache.argtypes = [_vp, _vp, _vp, _vp, _i64p, ctypes.c_int64,
                                               ctypes.POINTER(Geom)]
        L.pa_ref_fp8_decode.restype = ctypes.c_double
        L.pa_ref_fp8_decode.argtypes = [ctypes.c_uint8]
        L.pa_ref_fp8_encode.restype = ctypes.c_uint8
        L.pa_ref_fp8_encode.argtypes = [ctypes.c_float]
        L.pa_ref_copy_blocks.restype = ctypes.c_int32
        L.pa_ref_swap_blocks.restype = ctypes.c_int32
        L.pa_ref_swap_blocks.argtypes = [_vp, _vp, ctypes.c_int64, _vp, _vp, ctypes.c_int64,
                                         _i64p, ctypes.c_int64, ctypes.POINTER(Geom)]
        L.pa_ref_copy_blocks.argtypes = [_vp, _vp, _i64p, ctypes.c_int64, ctypes.POINTER(Geom)]
        L.pa_ref_paged_attention.restype = ctypes.c_int32
        L.pa_ref_paged_attention.argtypes = [_f64p, _f64p, _vp, _vp, _vp, _i32p, _i32p, _i32p,
                                             ctypes.c_int32, ctypes.c_double, ctypes.POINTER(Geom),
                                             _i32p, ctypes.c_int32, ctypes.c_int32]
        L.pa_ref_partition_attention.restype = ctypes.c_int32
        L.pa_ref_partition_attention.argtypes = [_f64p, _f64p, _f64p, _vp, _vp, _vp, _i32p, _i32p,
                                                 _i32p, ctypes.c_int32, ctypes.c_double,
                                                 ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.POINTER(Geom), _i32p, ctypes.c_int32,
                                                 ctypes.c_int32]
        L.pa_ref_merge_partitions.restype = None
        L.pa_ref_merge_partitions.argtypes = [_f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int64,
                                              ctypes.c_int32, ctypes.c_int32]
        L.pa_ref_dense_attention.restype = None
        L.pa_ref_dense_attention.argtypes = [_f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_double]
        _lib = L
    return _lib


def make_geom(num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
              dtype, block_size=16, q_dtype=None, k_scale=1.0, v_scale=1.0):
    """dtype: the pools' element type; q_dtype (FP8 pools): that of q, key and value."""
    return Geom(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim),
                int(block_size), int(num_blocks), int(max_blocks_per_seq), DTYPE_CODE[dtype],
                -1 if q_dtype is None else DTYPE_CODE[q_dtype], float(k_scale), float(v_scale))


def _ptr(a, t):
    return a.ctypes.data_as(t) if a is not None else None


def _contig(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def k_offset(g, block, kv_head, token, dim):
    return int(lib().pa_ref_k_offset(ctypes.byref(g), block, kv_head, token, dim))


def v_offset(g, block, kv_head, token, dim):
    return int(lib().pa_ref_v_offset(ctypes.byref(g), block, kv_head, token, dim))


def to_double(a, dtype):
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float64)
    lib().pa_ref_to_double(_vp(a.ctypes.data), DTYPE_CODE[dtype], a.size, _ptr(out, _f64p))
    return out


def reshape_and_cache(key, value, k_pool, v_pool, slot_mapping, g):
    """In-place write of key/value [T, Hkv, D] into the pools (numpy, C-contiguous)."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    key, value = _contig(key), _contig(value)
    slot_mapping = _contig(slot_mapping, np.int64)
    rc = lib().pa_ref_reshape_and_cache(_vp(key.ctypes.data), _vp(value.ctypes.data),
                                        _vp(k_pool.ctypes.data), _vp(v_pool.ctypes.data),
                                        _ptr(slot_mapping, _i64p), len(slot_mapping),
                                        ctypes.byref(g))
    if rc != 0:
        raise ValueError("oracle reshape_and_cache: slot outside the pool")


def fp8_decode(code: int) -> float:
    return float(lib().pa_ref_fp8_decode(int(code)))


def fp8_encode(x: float) -> int:
    return int(lib().pa_ref_fp8_encode(float(x)))


def copy_blocks(k_pool, v_pool, block_mapping, g):
    """In-place copy of whole blocks: block_mapping int64 [n, 2] of (source, destination)."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    m = _contig(block_mapping, np.int64).reshape(-1, 2)
    rc = lib().pa_ref_copy_blocks(_vp(k_pool.ctypes.data), _vp(v_pool.ctypes.data),
                                  _ptr(m, _i64p), m.shape[0], ctypes.byref(g))
    if rc != 0:
        raise ValueError("oracle copy_blocks: bad arguments")


def swap_blocks(dst_k, dst_v, src_k, src_v, block_mapping, g):
    """Copies whole blocks from the src pools onto the dst pools (their own block counts, the
    first axis): block_mapping int64 [n, 2] of (source, destination)."""
    for a in (dst_k, dst_v, src_k, src_v):
        assert a.flags.c_contiguous
    m = _contig(block_mapping, np.int64).reshape(-1, 2)
    rc = lib().pa_ref_swap_blocks(_vp(dst_k.ctypes.data), _vp(dst_v.ctypes.data),
                                  dst_k.shape[0], _vp(src_k.ctypes.data),
                                  _vp(src_v.ctypes.data), src_k.shape[0], _ptr(m, _i64p),
                                  m.shape[0], ctypes.byref(g))
    if rc != 0:
        raise ValueError("oracle swap_blocks: bad arguments")


def paged_attention(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale, g,
                    rows=None, threads=0):
    """Returns (out [n, Hq, D] float64, lse [n, Hq] float64) for the selected rows."""
    q = _contig(q)
    bt = _contig(block_tables, np.int32)
    cl = _contig(context_lens, np.int32)
    qsl = _contig(query_start_loc, np.int32)
    rows = _contig(rows, np.int32)
    nq = q.shape[0]
    n = nq if rows is None else len(rows)
    out = np.zeros((n, g.num_q_heads, g.head_dim), dtype=np.float64)
    lse = np.zeros((n, g.num_q_heads), dtype=np.float64)
    rc = lib().pa_ref_paged_attention(_ptr(out, _f64p), _ptr(lse, _f64p), _vp(q.ctypes.data),
                                      _vp(k_pool.ctypes.data), _vp(v_pool.ctypes.data),
                                      _ptr(bt, _i32p), _ptr(cl, _i32p), _ptr(qsl, _i32p), nq,
                                      float(scale), ctypes.byref(g), _ptr(rows, _i32p), n,
                                      int(threads))
    if rc != 0:
        raise ValueError("oracle paged_attention: bad arguments")
    return out, lse


def partition_attention(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale, g,
                        partition_size, max_partitions, rows=None, threads=0):
    """Returns (o [n, Hq, P, D], m [n, Hq, P], l [n, Hq, P]) float64 partials."""
    q = _contig(q)
    bt = _contig(block_tables, np.int32)
    cl = _contig(context_lens, np.int32)
    qsl = _contig(query_start_loc, np.int32)
    rows = _contig(rows, np.int32)
    nq = q.shape[0]
    n = nq if rows is None else len(rows)
    P = int(max_partitions)
    o = np.zeros((n, g.num_q_heads, P, g.head_dim), dtype=np.float64)
    m = np.zeros((n, g.num_q_heads, P), dtype=np.float64)
    l = np.zeros((n, g.num_q_heads, P), dtype=np.float64)
    rc = lib().pa_ref_partition_attention(_ptr(o, _f64p), _ptr(m, _f64p), _ptr(l, _f64p),
                                          _vp(q.ctypes.data), _vp(k_pool.ctypes.data),
                                          _vp(v_pool.ctypes.data), _ptr(bt, _i32p),
                                          _ptr(cl, _i32p), _ptr(qsl, _i32p), nq, float(scale),
                                          int(partition_size), P, ctypes.byref(g),
                                          _ptr(rows, _i32p), n, int(threads))
    if rc != 0:
        raise ValueError("oracle partition_attention: bad arguments")
    return o, m, l


def merge_partitions(o, m, l):
    """o [..., P, D], m/l [..., P] -> (out [..., D], lse [...])."""
    lead = m.shape[:-1]
    P = m.shape[-1]
    D = o.shape[-1]
    items = int(np.prod(lead)) if lead else 1
    o = _contig(o, np.float64)
    m = _contig(m, np.float64)
    l = _contig(l, np.float64)
    out = np.zeros(lead + (D,), dtype=np.float64)
    lse = np.zeros(lead, dtype=np.float64)
    lib().pa_ref_merge_partitions(_ptr(out, _f64p), _ptr(lse, _f64p), _ptr(o, _f64p),
                                  _ptr(m, _f64p), _ptr(l, _f64p), items, D, P)
    return out, lse


def dense_attention(q, k, v, scale):
    """One query q [D] over contiguous keys k, v [n, D] (float64)."""
    q = _contig(q, np.float64)
    k = _contig(k, np.float64)
    v = _contig(v, np.float64)
    n, D = k.shape
    out = np.zeros(D, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    lib().pa_ref_dense_attention(_ptr(out, _f64p), _ptr(lse, _f64p), _ptr(q, _f64p),
                                 _ptr(k, _f64p), _ptr(v, _f64p), n, D, float(scale))
    return out, float(lse[0])
