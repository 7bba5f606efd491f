"""Thin ctypes binding of libpa.so (include/pa.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their device
pointers and the current HIP stream to the C entry point of the same name, and raises
PAError on a non-zero status.  All computation happens in the library's HIP kernels.
Importing this module raises ImportError when libpa.so has not been built.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_445_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
DTYPE_CODE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_UNSUPPORTED",
          -4: "PA_ERR_WORKSPACE", -5: "PA_ERR_HIP", -6: "PA_ERR_NO_BLOCKS"}


class Geom(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class PAError(RuntimeError):
    def __init__(self, fn, code):
        msg = _lib.pa_status_str(code).decode()
        super().__init__(f"{fn}: {STATUS.get(code, code)} ({msg})")
        self.code = code


_vp = ctypes.c_void_p
_G = ctypes.POINTER(Geom)
_lib.pa_status_str.restype = ctypes.c_char_p
_lib.pa_status_str.argtypes = [ctypes.c_int]
_lib.pa_kv_cache_bytes.restype = ctypes.c_size_t
_lib.pa_kv_cache_bytes.argtypes = [_G]
_lib.pa_workspace_size.restype = ctypes.c_size_t
_lib.pa_workspace_size.argtypes = [_G, ctypes.c_int32]
_lib.pa_reshape_and_cache.restype = ctypes.c_int
_lib.pa_reshape_and_cache.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int64, _G, _vp]
_lib.pa_copy_blocks.restype = ctypes.c_int
_lib.pa_copy_blocks.argtypes = [_vp, _vp, _vp, ctypes.c_int64, _G, _vp]
_lib.pa_swap_blocks.restype = ctypes.c_int
_lib.pa_swap_blocks.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                ctypes.c_int32, _G, _vp]
_lib.pa_decode.restype = ctypes.c_int
_lib.pa_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32,
                           ctypes.c_float, _vp, ctypes.c_size_t, _G, _vp]
_lib.pa_decode_scratch.restype = ctypes.c_int
_lib.pa_decode_scratch.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_float, _G, _vp]
_lib.pa_decode_partitioned.restype = ctypes.c_int
_lib.pa_decode_partitioned.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                       ctypes.c_int32, _G, _vp]
_lib.pa_shared_prefix_workspace_size.restype = ctypes.c_size_t
_lib.pa_shared_prefix_workspace_size.argtypes = [_G, ctypes.c_int32, ctypes.c_int32]
_lib.pa_decode_shared_prefix.restype = ctypes.c_int
_lib.pa_decode_shared_prefix.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                         ctypes.c_int32, _vp, _vp, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_float, _vp, ctypes.c_size_t,
                                         _G, _vp]
_lib.pa_decode_reduce.restype = ctypes.c_int
_lib.pa_decode_reduce.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _G, _vp]


_lib.pa_measure_stream_read.restype = ctypes.c_int
_lib.pa_measure_stream_read.argtypes = [_vp, ctypes.c_size_t, _vp, ctypes.c_int32, _vp]
_lib.pa_measure_tile_read.restype = ctypes.c_int
_lib.pa_measure_tile_read.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int32, _vp,
                                      ctypes.c_int32, _vp]


def lib():
    return _lib


def _code(dt):
    return DTYPE_CODE[dt] if isinstance(dt, torch.dtype) else int(dt)


def geom(num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
         kv_dtype, out_dtype=None, block_size=16, q_dtype=None, k_scale=1.0,
         v_scale=1.0) -> Geom:
    """kv_dtype: the pools' type (a torch dtype or a pa_dtype code, PA_FP8_E4M3 for FP8
    pools); q_dtype: that of q, key and value (default: kv_dtype; fp16 for FP8 pools);
    out_dtype: q_dtype or float32 (default q_dtype)."""
    kv = _code(kv_dtype)
    qd = (PA_F16 if kv == PA_FP8_E4M3 else kv) if q_dtype is None else _code(q_dtype)
    od = qd if out_dtype is None else _code(out_dtype)
    return Geom(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim),
                int(block_size), int(num_blocks), int(max_blocks_per_seq), kv, od, qd,
                float(k_scale), float(v_scale))


def _p(t):
    return None if t is None else _vp(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def _check(fn, code):
    if code != 0:
        raise PAError(fn, code)


def status_str(code: int) -> str:
    return _lib.pa_status_str(code).decode()


def kv_cache_bytes(g: Geom) -> int:
    return int(_lib.pa_kv_cache_bytes(ctypes.byref(g)))


def workspace_size(g: Geom, num_q_rows: int) -> int:
    return int(_lib.pa_workspace_size(ctypes.byref(g), int(num_q_rows)))


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, g: Geom, stream=None):
    _check("pa_reshape_and_cache",
           _lib.pa_reshape_and_cache(_p(key), _p(value), _p(k_cache), _p(v_cache),
                                     _p(slot_mapping), int(slot_mapping.numel()),
                                     ctypes.byref(g), _stream(stream)))


def copy_blocks(k_cache, v_cache, block_mapping, g: Geom, stream=None):
    """block_mapping: int64 tensor [num_pairs, 2] of (source, destination) block ids."""
    _check("pa_copy_blocks",
           _lib.pa_copy_blocks(_p(k_cache), _p(v_cache), _p(block_mapping),
                               int(block_mapping.shape[0]) if block_mapping.numel() else 0,
                               ctypes.byref(g), _stream(stream)))


SWAP_OUT, SWAP_IN = 0, 1


def swap_blocks(k_cache, v_cache, host_k, host_v, block_mapping, direction, g: Geom,
                stream=None):
    """Copies whole blocks between the device pools and host pools of the same layout
    (host_k / host_v: CPU tensors, pinned for asynchronous copies).  block_mapping: a CPU
    int64 tensor [num_pairs, 2] of (source, destination) ids; direction SWAP_OUT (device to
    host) or SWAP_IN (host to device)."""
    if block_mapping.device.type != "cpu" or host_k.device.type != "cpu" or \
            host_v.device.type != "cpu":
        raise ValueError("swap_blocks: block_mapping and the host pools live in host memory")
    m = block_mapping.contiguous()
    _check("pa_swap_blocks",
           _lib.pa_swap_blocks(_p(k_cache), _p(v_cache), _p(host_k), _p(host_v),
                               int(host_k.shape[0]), _p(m),
                               int(m.shape[0]) if m.numel() else 0, int(direction),
                               ctypes.byref(g), _stream(stream)))


def decode(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
           workspace, g: Geom, stream=None, max_query_len: int = 0):
    """max_query_len: with query_start_loc, an upper bound of any sequence's rows (0: unknown)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode",
           _lib.pa_decode(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                          _p(context_lens), _p(query_start_loc), int(q.shape[0]),
                          int(max_query_len), float(scale), _p(workspace), ws_bytes,
                          ctypes.byref(g), _stream(stream)))


def shared_prefix_workspace_size(g: Geom, num_q_rows: int, max_prefix_blocks: int) -> int:
    return int(_lib.pa_shared_prefix_workspace_size(ctypes.byref(g), int(num_q_rows),
                                                    int(max_prefix_blocks)))


def decode_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                         prefix_groups, prefix_blocks, max_prefix_blocks, scale, workspace,
                         g: Geom, stream=None, max_query_len: int = 0):
    """pa_decode_shared_prefix.  prefix_groups: int32 [num_groups + 1] sequence ranges,
    prefix_blocks: int32 [num_groups] claimed shared leading blocks (device tensors, or None
    for no group)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ng = 0 if prefix_blocks is None else int(prefix_blocks.numel())
    _check("pa_decode_shared_prefix",
           _lib.pa_decode_shared_prefix(_p(out), _p(q), _p(k_cache), _p(v_cache),
                                        _p(block_tables), _p(context_lens),
                                        _p(query_start_loc), int(q.shape[0]),
                                        int(max_query_len), _p(prefix_groups),
                                        _p(prefix_blocks), ng, int(max_prefix_blocks),
                                        float(scale), _p(workspace), ws_bytes, ctypes.byref(g),
                                        _stream(stream)))


DECODE_SCRATCH_BYTES = 36 << 20  # PA_DECODE_SCRATCH_BYTES


def decode_scratch(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
                   g: Geom, stream=None, max_query_len: int = 0):
    """pa_decode_scratch: pa_decode with the library's static device workspace (allocates
    nothing; calls that overlap on one device race)."""
    _check("pa_decode_scratch",
           _lib.pa_decode_scratch(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                                  _p(context_lens), _p(query_start_loc), int(q.shape[0]),
                                  int(max_query_len), float(scale), ctypes.byref(g),
                                  _stream(stream)))


def decode_partitioned(tmp_out, max_logits, exp_sums, q, k_cache, v_cache, block_tables,
                       context_lens, query_start_loc, scale, partition_size, max_partitions,
                       g: Geom, stream=None):
    """query_start_loc: int32 [num_seqs + 1] or None (one row per sequence)."""
    _check("pa_decode_partitioned",
           _lib.pa_decode_partitioned(_p(tmp_out), _p(max_logits), _p(exp_sums), _p(q),
                                      _p(k_cache), _p(v_cache), _p(block_tables),
                                      _p(context_lens), _p(query_start_loc), int(q.shape[0]),
                                      float(scale), int(partition_size), int(max_partitions),
                                      ctypes.byref(g), _stream(stream)))


def decode_reduce(out, tmp_out, max_logits, exp_sums, max_partitions, g: Geom, stream=None):
    _check("pa_decode_reduce",
           _lib.pa_decode_reduce(_p(out), _p(tmp_out), _p(max_logits), _p(exp_sums),
                                 int(out.shape[0]), int(max_partitions), ctypes.byref(g),
                                 _stream(stream)))


# ---- read ceilings (include/pa_measure.h): measurement kernels, not the attention path

def measure_stream_read(buf, sink, workgroups=0, stream=None):
    """Reads every byte of the device tensor buf; sink: uint32 device tensor, one entry per
    workgroup."""
    _check("pa_measure_stream_read",
           _lib.pa_measure_stream_read(_p(buf), buf.numel() * buf.element_size(), _p(sink),
                                       int(workgroups), _stream(stream)))


def measure_tile_read(base, tile_offsets, tile_bytes, sink, workgroups=0, stream=None):
    """Reads tiles of tile_bytes at base + tile_offsets (int64 device tensor of byte offsets)."""
    _check("pa_measure_tile_read",
           _lib.pa_measure_tile_read(_p(base), _p(tile_offsets), int(tile_offsets.numel()),
                                     int(tile_bytes), _p(sink), int(workgroups),
                                     _stream(stream)))
