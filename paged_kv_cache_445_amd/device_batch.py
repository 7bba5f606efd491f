"""A synthetic batch resident in GPU memory, and one decode step over it.

Torch provides the device memory and the stream; every step of the path runs in libpa.so
through the binding (`pa`).  Used by the GPU tests, the smoke check and the benchmark.
"""
import numpy as np
import torch

from . import pa
from . import workloads as W

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_NAN_FILL = {"f32": (torch.int32, W.NAN_BITS["f32"]), "f16": (torch.int16, W.NAN_BITS["f16"]),
             "bf16": (torch.int16, W.NAN_BITS["bf16"]), "fp8": (torch.uint8, W.NAN_BITS["fp8"])}


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage-dtype numpy array -> torch tensor of the same bits on `device`."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def nan_fill_(pool: torch.Tensor, dtype: str) -> torch.Tensor:
    view_dtype, bits = _NAN_FILL[dtype]
    pool.view(view_dtype).fill_(bits)
    return pool


class DeviceBatch:
    def __init__(self, b: W.Batch, device="cuda:0", out_f32: bool = True):
        self.b = b
        self.device = torch.device(device)
        dt = TORCH_DTYPE[b.dtype]
        self.dtype = dt
        dev = self.device
        self.q = to_device(b.q, b.dtype, dev)
        self.key_hist = to_device(b.key[b.history], b.dtype, dev)
        self.value_hist = to_device(b.value[b.history], b.dtype, dev)
        self.slot_hist = torch.from_numpy(b.slot[b.history].astype(np.int64)).to(dev)
        self.key_new = to_device(b.key[b.new], b.dtype, dev)
        self.value_new = to_device(b.value[b.new], b.dtype, dev)
        self.slot_new = torch.from_numpy(b.slot[b.new].astype(np.int64)).to(dev)
        self.block_tables = torch.from_numpy(b.block_tables.astype(np.int32)).to(dev)
        self.context_lens = torch.from_numpy(b.context_lens.astype(np.int32)).to(dev)
        self.qsl = None if b.query_start_loc is None else \
            torch.from_numpy(b.query_start_loc.astype(np.int32)).to(dev)
        fp8 = b.pool_dtype == "fp8"
        pool_dt = torch.uint8 if fp8 else dt  # FP8 pools: raw E4M3 bytes
        self.k_cache = nan_fill_(torch.empty(b.k_pool_shape(), dtype=pool_dt, device=dev),
                                 b.pool_dtype)
        self.v_cache = nan_fill_(torch.empty(b.v_pool_shape(), dtype=pool_dt, device=dev),
                                 b.pool_dtype)
        out_dt = torch.float32 if out_f32 else dt
        self.geom = pa.geom(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, b.num_blocks,
                            b.max_blocks_per_seq, pa.PA_FP8_E4M3 if fp8 else dt, out_dt,
                            b.block_size, q_dtype=dt, k_scale=b.k_scale, v_scale=b.v_scale)
        self.out = torch.zeros((b.num_q_rows, b.num_q_heads, b.head_dim), dtype=out_dt,
                               device=dev)
        ws = pa.workspace_size(self.geom, b.num_q_rows)
        # zeroed once: pa_decode keeps its arrival counters at zero between calls
        self.workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=dev)
        self.scale = float(b.scale)
        self.max_query_len = int(b.rows_per_seq().max()) if b.num_seqs else 0
        self.prefix = None  # shared-prefix groups (set_shared_prefix)

    def set_shared_prefix(self, groups, blocks, max_prefix_blocks: int):
        """Decode through pa_decode_shared_prefix from now on: groups int [num_groups + 1]
        (sequence ranges), blocks int [num_groups] (claimed shared leading blocks)."""
        dev = self.device
        g = torch.from_numpy(np.asarray(groups, dtype=np.int32)).to(dev)
        k = torch.from_numpy(np.asarray(blocks, dtype=np.int32)).to(dev)
        ws = pa.shared_prefix_workspace_size(self.geom, self.b.num_q_rows, max_prefix_blocks)
        # zeroed once: the decode keeps its arrival counters at zero between calls
        self.prefix = (g, k, int(max_prefix_blocks),
                       torch.zeros(max(ws, 16), dtype=torch.uint8, device=dev))

    # ------------------------------------------------------------------ the method
    def prefill(self, stream=None):
        """Write the cached history (everything before this step) into the pools."""
        pa.reshape_and_cache(self.key_hist, self.value_hist, self.k_cache, self.v_cache,
                             self.slot_hist, self.geom, stream)

    def write_new(self, stream=None):
        pa.reshape_and_cache(self.key_new, self.value_new, self.k_cache, self.v_cache,
                             self.slot_new, self.geom, stream)

    def attend(self, stream=None):
        if self.prefix is not None:
            g, k, mpb, ws = self.prefix
            pa.decode_shared_prefix(self.out, self.q, self.k_cache, self.v_cache,
                                    self.block_tables, self.context_lens, self.qsl, g, k, mpb,
                                    self.scale, ws, self.geom, stream,
                                    max_query_len=self.max_query_len)
            return
        pa.decode(self.out, self.q, self.k_cache, self.v_cache, self.block_tables,
                  self.context_lens, self.qsl, self.scale, self.workspace, self.geom, stream,
                  max_query_len=self.max_query_len)

    def step(self, stream=None):
        """One pass of the hot path: cache write of this step's tokens, then attention."""
        self.write_new(stream)
        self.attend(stream)

    # ------------------------------------------------------------------ host copies
    def pools_host(self):
        """(k_pool, v_pool) as numpy arrays in the storage dtype."""
        out = []
        for t in (self.k_cache, self.v_cache):
            c = t.detach().cpu()
            if self.b.pool_dtype == "bf16":
                out.append(c.view(torch.int16).numpy().view(np.uint16))
            else:
                out.append(c.numpy())
        return out

    def out_host(self) -> np.ndarray:
        return self.out.detach().float().cpu().numpy().astype(np.float64)
