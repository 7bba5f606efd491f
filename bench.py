"""Paged-attention decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload llama7b_f16]

One step is one pass of the whole hot path over one synthetic decode batch resident in
HBM: the cache write of the step's new tokens (pa_reshape_and_cache) followed by
attention over every sequence's paged context (pa_decode).  Several copies of the K/V
pools are rotated between steps so that no step finds the previous step's blocks in the
256 MB last-level cache: every step reads its KV bytes from HBM.

Prints ONE JSON line.  `value` is the effective KV-read bandwidth of the whole step:
algorithmic KV bytes (every context token's K and V read once per KV head) divided by
the wall time per step of the timed region.  `roofline` rates pa_decode alone: right after
the timed steps the same pa_decode calls run back to back between one pair of HIP events
on the stream they run on, and their average duration is compared with the 8 TB/s HBM
peak (or the matrix-core peak when the flops dominate).  `cpu_baseline` times the fp64
CPU oracle on the same batch on the host cores.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}  # dense; fp32 on the VALU
# rocprof-derived HBM traffic of the decode kernels, with the hash of the sources it was
# measured on; reported only while those sources are unchanged
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{workload}.txt")
KERNEL_SOURCES = ["pa_device.h", "pa_internal.h", "pa_mfma.h", "decode_valu.hip",
                  "decode_mfma.hip", "reduce.hip", "chunk.hip", "pa_api.cpp"]

def runs_chunk_kernel(b) -> bool:
    """Whether pa_decode launches its multi-row kernel for this batch: the decode kernel
    takes sequences of up to 16 / G rows (G = query heads per KV head) on 16-bit and FP8
    pools, one row on fp32 pools."""
    if b.query_start_loc is None:
        return False
    takes = 16 // (b.num_q_heads // b.num_kv_heads) if b.pool_dtype != "f32" else 1
    return int(b.rows_per_seq().max()) > takes


DESCRIPTIONS = {
    "llama7b_f16": "LLaMA-7B-shaped decode: 32 seqs x 32 heads (MHA), head_dim 128, fp16 KV, "
                   "block 16, ctx U[256,2048], 8192-block pool, permuted block table",
    "llama7b_f16_bs8": "LLaMA-7B-shaped decode with 8-token blocks: 32 seqs x 32 heads (MHA), "
                       "head_dim 128, fp16 KV, block 8, ctx U[256,2048], 8192-block pool, "
                       "permuted block table",
    "gqa_long_bf16": "GQA decode: 64 seqs, 64 q / 8 kv heads, head_dim 128, bf16 KV, block 16, "
                     "ctx log-uniform [128,32768]",
    "prefix_shared_f16": "prefix-shared decode: 128 seqs x 32 heads, head_dim 128, fp16 KV, "
                         "32 shared leading blocks + private tail U[16,1024]",
    "mixed_chunked_bf16": "mixed step: 8 x 512-row causal chunks + 120 decode rows, 32 q / 8 kv "
                          "heads, head_dim 128, bf16 KV",
    "tiny_f32": "tiny decode: 4 seqs x 4 heads, head_dim 64, fp32 KV",
    "prefill_chunks_bf16": "the mixed step's chunked-prefill rows alone: 8 x 512-row causal "
                           "chunks over prior U[0,7488], 32 q / 8 kv heads, head_dim 128, bf16 KV",
    "llama7b_fp8": "LLaMA-7B-shaped decode with FP8 E4M3 KV (per-pool scales 6.5/448): 32 seqs "
                   "x 32 heads (MHA), head_dim 128, fp16 q, block 16, ctx U[256,2048], "
                   "8192-block pool, permuted block table",
    "gqa_long_fp8": "GQA decode with FP8 E4M3 KV (per-pool scales 3.25/448): 64 seqs, 64 q / 8 kv "
                    "heads, head_dim 128, fp16 q, block 16, ctx log-uniform [128,32768]",
    "spec_verify_f16": "speculative verify step: 32 seqs x 6 causal rows (last token + 5 "
                       "drafts) x 32 heads (MHA), head_dim 128, fp16 KV, prior ctx U[256,2048]",
    "spec_verify_gqa_bf16": "speculative verify step: 64 seqs x 4 causal rows, 32 q / 8 kv "
                            "heads, head_dim 128, bf16 KV, prior ctx U[512,4096]",
    "spec_verify_fp8": "speculative verify step with FP8 E4M3 KV (per-pool scales 6.5/448): "
                       "32 seqs x 6 causal rows x 32 heads (MHA), head_dim 128, fp16 q, prior "
                       "ctx U[256,2048]",
    "mixed_chunked_fp8": "mixed step with FP8 E4M3 KV (per-pool scales 6.5/448): 8 x 512-row "
                         "causal chunks + 120 decode rows, 32 q / 8 kv heads, head_dim 128, bf16 q",
    "swap_f16": "block swap: 256 scattered LLaMA-7B blocks (128 KiB per pool) out to a pinned "
                "host pool and 256 back in onto scattered device blocks, per step",
    "cow_copy_f16": "copy-on-write block copies: 256 (source, destination) pairs of LLaMA-7B "
                    "blocks (32 kv heads x 128 x 16 tokens fp16, 128 KiB per pool) in an "
                    "8192-block pool",
    "hbm_read_ceiling": "HBM read ceiling: a contiguous 640 MiB buffer read front to back per "
                        "step, three buffers rotated (1.9 GiB, past the 256 MB last-level "
                        "cache)",
    "tile_replay_llama7b_f16": "HBM read ceiling of the LLaMA-7B decode's access pattern: every "
                               "4 KiB K and V tile of the llama7b_f16 batch (585 MB) read in "
                               "(sequence, block, head) order with no arithmetic, split evenly "
                               "over the waves; three pool copies rotated",
}
MEASURE_WORKLOADS = ("cow_copy_f16", "swap_f16", "hbm_read_ceiling", "tile_replay_llama7b_f16")


def sources_digest():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_445_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()


def read_traffic(workload):
    """HBM bytes per pa_decode call from a committed rocprof counter summary, or None."""
    path = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_call:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_b or m_sha.group(1) != sources_digest():
        return None
    return float(m_b.group(1))


def row_keys(b):
    """Visible keys of every query row (its position + 1)."""
    import numpy as np
    n = b.rows_per_seq()
    keys = []
    for s in range(b.num_seqs):
        ctx = int(b.context_lens[s])
        keys.extend(range(ctx - int(n[s]) + 1, ctx + 1))
    return np.asarray(keys, dtype=np.int64)


def attention_flops(b):
    """QK^T and P.V multiply-adds of one pass: 4 * head_dim flops per (row, head, key)."""
    return int(row_keys(b).sum()) * b.num_q_heads * 4 * b.head_dim


def cpu_baseline(b, min_seconds, threads, max_key_heads=3e8, single_seconds=3.0):
    """fp64 oracle over the batch, repeated until min_seconds have passed, on `threads`
    threads; then on one thread for single_seconds on a smaller row sample.  The oracle's
    pools are written by its own cache write from the batch's token records.  Batches
    larger than max_key_heads (row, head, key) triples run on an evenly spaced row sample."""
    import numpy as np
    import oracle
    from paged_kv_cache_445_amd import workloads as W
    fp8 = b.pool_dtype == "fp8"
    g = oracle.make_geom(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, b.num_blocks,
                         b.max_blocks_per_seq, b.pool_dtype, b.block_size,
                         q_dtype=b.dtype if fp8 else None, k_scale=b.k_scale, v_scale=b.v_scale)
    kp = W.nan_pool(b.k_pool_shape(), b.pool_dtype)
    vp = W.nan_pool(b.v_pool_shape(), b.pool_dtype)
    oracle.reshape_and_cache(b.key, b.value, kp, vp, b.slot, g)
    keys = row_keys(b)
    total = float(keys.sum()) * b.num_q_heads
    rows = None
    frac = 1.0
    if total > max_key_heads:
        step = int(np.ceil(total / max_key_heads))
        rows = np.arange(0, b.num_q_rows, step, dtype=np.int32)
        frac = float(keys[rows].sum()) / float(keys.sum())
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.paged_attention(b.q, kp, vp, b.block_tables, b.context_lens, b.query_start_loc,
                               b.scale, g, rows=rows, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    per = el / reps / frac  # seconds for the whole batch at the sampled rate
    what = (f"the whole {b.name} batch ({b.num_q_rows} rows" if rows is None else
            f"every {int(rows[1] - rows[0]) if len(rows) > 1 else 1}th row of {b.name} "
            f"({len(rows)} of {b.num_q_rows} rows, {100 * frac:.1f}% of the key-heads")
    # one thread, on every k-th row so that a pass takes about a tenth of single_seconds
    single = None
    if single_seconds > 0:
        per_row = per / b.num_q_rows * threads  # one thread's seconds per row, roughly
        k = max(1, int(np.ceil(per_row * b.num_q_rows / (single_seconds / 10))))
        rows1 = np.arange(0, b.num_q_rows, k, dtype=np.int32)
        frac1 = float(keys[rows1].sum()) / float(keys.sum())
        reps1, t1 = 0, time.perf_counter()
        while True:
            oracle.paged_attention(b.q, kp, vp, b.block_tables, b.context_lens,
                                   b.query_start_loc, b.scale, g, rows=rows1, threads=1)
            reps1 += 1
            el1 = time.perf_counter() - t1
            if el1 >= single_seconds:
                break
        per1 = el1 / reps1 / frac1
        single = {"value": round(b.kv_bytes() / per1 / 1e9, 4), "unit": "GB/s", "threads": 1,
                  "sample": f"every {k}th row ({len(rows1)} rows, {100 * frac1:.2f}% of the "
                            f"key-heads), {reps1} passes in {el1:.1f} s; "
                            f"{per1 * 1e3:.0f} ms per whole batch"}
    return {"value": round(b.kv_bytes() / per / 1e9, 4), "unit": "GB/s", "cores": threads,
            "threads": threads, "host_cores": os.cpu_count(), "kind": "oracle",
            "sample": f"{what} x {b.num_q_heads} heads, {b.kv_bytes() / 1e6:.1f} MB of KV in "
                      f"the batch), {reps} passes in {el:.1f} s on {threads} threads; scaled to "
                      f"the whole batch: {per * 1e3:.1f} ms per pass, "
                      f"{b.num_q_rows * b.num_q_heads / per:.0f} row-heads/s",
            "single_thread": single}


def bench_copy(args):
    """pa_copy_blocks alone: one step is one call over COPY_PAIRS block pairs; value is the
    HBM bytes it must move (every pair reads and writes one block of each pool)."""
    import numpy as np
    import torch
    from paged_kv_cache_445_amd import pa
    dev = torch.device("cuda:0")
    NB, Hkv, D, pairs = 8192, 32, 128, 256
    rng = np.random.default_rng(4457)
    g = pa.geom(1, Hkv, Hkv, D, NB, 1, torch.float16)
    shape_k, shape_v = (NB, Hkv, D // 8, 16, 8), (NB, Hkv, D, 16)
    copies = args.copies or 3
    pools = [(torch.randn(shape_k, device=dev, dtype=torch.float16),
              torch.randn(shape_v, device=dev, dtype=torch.float16)) for _ in range(copies)]
    # sources in the lower half of the pool, distinct destinations in the upper half
    maps = []
    for _ in range(copies):
        src = rng.choice(NB // 2, size=pairs, replace=False)
        dst = NB // 2 + rng.choice(NB // 2, size=pairs, replace=False)
        maps.append(torch.from_numpy(np.stack([src, dst], 1).astype(np.int64)).to(dev))
    block_bytes = Hkv * 16 * D * 2
    moved = pairs * 2 * 2 * block_bytes  # K and V, read and written
    stream = torch.cuda.current_stream()

    def step(i):
        kc, vc = pools[i % copies]
        pa.copy_blocks(kc, vc, maps[i % copies], g)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = ev[0].elapsed_time(ev[1]) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    achieved = moved / (call_ms * 1e-3) / 1e9

    cpu = None
    if args.cpu_seconds > 0:
        # the oracle's copy (one thread, element by element through the layout) on a
        # 512-block host pool of the same geometry, the same number of pairs
        import oracle
        og = oracle.make_geom(1, Hkv, Hkv, D, 512, 1, "f16")
        kp = np.zeros((512, Hkv, D // 8, 16, 8), dtype=np.float16)
        vp = np.zeros((512, Hkv, D, 16), dtype=np.float16)
        m = np.stack([rng.choice(256, size=pairs, replace=False),
                      256 + rng.choice(256, size=pairs, replace=False)], 1)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.copy_blocks(kp, vp, m, og)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 10.0):
                break
        cpu = {"value": round(moved * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{pairs} pairs of the same blocks in a 512-block host pool, {reps} "
                         f"calls in {el:.1f} s"}
    line = {
        "metric": "copy-on-write block copy: HBM GB/s (read + write)",
        "value": round(moved / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "cow_copy_f16", "description": DESCRIPTIONS["cow_copy_f16"],
                   "pairs": pairs, "bytes_per_step": moved, "pool_copies_rotated": copies},
        "pa_copy_blocks_us": round(call_ms * 1e3, 3),
        "roofline": {"bound": "hbm", "kernel": "pa_copy_blocks", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes, 128b/130b)


def bench_swap(args):
    """pa_swap_blocks alone: one step swaps SWAP_PAIRS LLaMA-7B blocks (scattered device ids)
    out to a pinned host pool and another SWAP_PAIRS back in onto scattered free device
    blocks; value is the bytes that cross PCIe per second (both pools, both directions)."""
    import numpy as np
    import torch
    from paged_kv_cache_445_amd import pa
    dev = torch.device("cuda:0")
    NB, NH, Hkv, D, pairs = 8192, 1024, 32, 128, 256
    rng = np.random.default_rng(4458)
    g = pa.geom(1, Hkv, Hkv, D, NB, 1, torch.float16)
    shape_k, shape_v = (Hkv, D // 8, 16, 8), (Hkv, D, 16)
    kc = torch.randn((NB,) + shape_k, device=dev, dtype=torch.float16)
    vc = torch.randn((NB,) + shape_v, device=dev, dtype=torch.float16)
    hk = torch.empty((NH,) + shape_k, dtype=torch.float16, pin_memory=True)
    hv = torch.empty((NH,) + shape_v, dtype=torch.float16, pin_memory=True)
    hk.normal_()
    hv.normal_()
    maps = []
    for i in range(4):
        dsrc = rng.choice(NB // 2, size=pairs, replace=False)  # out: scattered device blocks
        hdst = (i % 2) * (NH // 2) + np.arange(pairs)          # ... to a run of host blocks
        hsrc = ((i + 1) % 2) * (NH // 2) + rng.permutation(pairs)  # in: the other host half
        ddst = NB // 2 + rng.choice(NB // 2, size=pairs, replace=False)
        maps.append((torch.from_numpy(np.stack([dsrc, hdst], 1).astype(np.int64)),
                     torch.from_numpy(np.stack([hsrc, ddst], 1).astype(np.int64))))
    block_bytes = Hkv * 16 * D * 2
    moved = 2 * pairs * 2 * block_bytes  # out and in, K and V
    stream = torch.cuda.current_stream()

    def step(i):
        mo, mi = maps[i % len(maps)]
        pa.swap_blocks(kc, vc, hk, hv, mo, pa.SWAP_OUT, g)
        pa.swap_blocks(kc, vc, hk, hv, mi, pa.SWAP_IN, g)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = ev[0].elapsed_time(ev[1]) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    achieved = moved / (call_ms * 1e-3) / 1e9
    line = {
        "metric": "KV block swap to and from host memory: PCIe GB/s (both directions)",
        "value": round(moved / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "swap_f16", "description": DESCRIPTIONS["swap_f16"],
                   "pairs_each_way": pairs, "bytes_per_step": moved},
        "pa_swap_blocks_us": round(call_ms * 1e3, 3),
        "roofline": {"bound": "pcie", "kernel": "pa_swap_blocks (one kernel per 224 pairs over "
                     "device-mapped pinned host memory)", "achieved": round(achieved, 2),
                     "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PCIE_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def _timed(args, step, stream):
    """Warm-up steps, then args.steps steps between one pair of HIP events on `stream`;
    returns (wall seconds, event milliseconds per step)."""
    import torch
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, ev[0].elapsed_time(ev[1]) / args.steps


def _ceiling_line(args, workload, moved, wall, call_ms, kernel, extra):
    ms_per_step = wall * 1e3 / args.steps
    achieved = moved / (call_ms * 1e-3) / 1e9
    line = {
        "metric": "HBM read ceiling: GB/s of a read-only kernel",
        "value": round(moved / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic",
        "config": dict({"workload": workload, "description": DESCRIPTIONS[workload],
                        "bytes_per_step": moved}, **extra),
        "kernel_us": round(call_ms * 1e3, 3),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_read_ceiling(args):
    """pa_measure_stream_read over one of three 640 MiB buffers per step."""
    import torch
    from paged_kv_cache_445_amd import pa
    dev = torch.device("cuda:0")
    n = 640 << 20
    copies = args.copies or 3
    bufs = [torch.empty(n, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(copies)]
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    wall, call_ms = _timed(args, lambda i: pa.measure_stream_read(bufs[i % copies], sink), stream)
    _ceiling_line(args, "hbm_read_ceiling", n, wall, call_ms,
                  "pa_measure_stream_read (two 256-thread workgroups per CU, 16 KiB in flight per wave)",
                  {"buffer_bytes": n, "buffers_rotated": copies})


def bench_tile_replay(args):
    """pa_measure_tile_read over the K and V tiles of the llama7b_f16 batch: for every
    sequence, 16-token block and KV head, the block's K tile then its V tile."""
    import numpy as np
    import torch
    from paged_kv_cache_445_amd import pa
    from paged_kv_cache_445_amd import workloads as W
    dev = torch.device("cuda:0")
    b = W.make("llama7b_f16")
    H, D = b.num_kv_heads, b.head_dim
    tile = 16 * D * 2
    pool = b.num_blocks * H * tile  # bytes of one pool
    offs = []
    for s in range(b.num_seqs):
        nblk = -(-int(b.context_lens[s]) // 16)
        blk = b.block_tables[s, :nblk].astype(np.int64)
        o = (blk[:, None] * H + np.arange(H)[None, :]) * tile  # [block][head]
        offs.append(np.stack([o, o + pool], axis=-1).reshape(-1))  # K then V (second pool)
    offs = np.concatenate(offs)
    moved = len(offs) * tile
    copies = args.copies or 3
    pools = [torch.empty(2 * pool, dtype=torch.uint8, device=dev).fill_(i + 1)
             for i in range(copies)]
    off_t = torch.from_numpy(offs).to(dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    wall, call_ms = _timed(args, lambda i: pa.measure_tile_read(pools[i % copies], off_t, tile,
                                                                sink), stream)
    _ceiling_line(args, "tile_replay_llama7b_f16", moved, wall, call_ms,
                  "pa_measure_tile_read (two 256-thread workgroups per CU, 8 tiles in flight per wave)",
                  {"tiles": int(len(offs)), "tile_bytes": tile, "pool_copies_rotated": copies,
                   "algorithmic_kv_bytes_of_the_batch": b.kv_bytes()})


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b_f16",
                    choices=sorted(DESCRIPTIONS))
    ap.add_argument("--copies", type=int, default=0,
                    help="K/V pool copies rotated between steps (0: enough for >= 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time of the CPU-oracle leg (0 skips it)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (0: min(16, host cores))")
    ap.add_argument("--partitioned", type=int, default=0, metavar="PS",
                    help="time pa_decode_partitioned with PS-token partitions + pa_decode_reduce "
                         "in place of pa_decode")
    ap.add_argument("--path", choices=("auto", "decode", "shared_prefix"), default="auto",
                    help="pa_decode, or pa_decode_shared_prefix with the batch's shared leading "
                         "blocks as one group (auto: the latter for batches built with a shared "
                         "prefix)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, copy a MIB-sized device buffer 3 times "
                         "(a reference kernel of known traffic for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the decode shards by KV head with no exchange inside attention, so there is "
              "no multi-GPU step to time here)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_445_amd import workloads as W
    from paged_kv_cache_445_amd.device_batch import DeviceBatch
    from paged_kv_cache_445_amd import pa

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "cow_copy_f16":
        return bench_copy(args)
    if args.workload == "swap_f16":
        return bench_swap(args)
    if args.workload == "hbm_read_ceiling":
        return bench_read_ceiling(args)
    if args.workload == "tile_replay_llama7b_f16":
        return bench_tile_replay(args)

    print(f"[bench] building workload {args.workload}", file=sys.stderr, flush=True)
    b = W.make(args.workload)
    kv_bytes = b.kv_bytes()
    db = DeviceBatch(b, device=dev)
    db.prefill()
    torch.cuda.synchronize()
    # the history staging tensors are not needed after the pools are written
    db.key_hist = db.value_hist = db.slot_hist = None

    copies = args.copies or max(2, math.ceil((1 << 30) / kv_bytes) + 1)
    pools = [(db.k_cache, db.v_cache)] + [(db.k_cache.clone(), db.v_cache.clone())
                                           for _ in range(copies - 1)]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def write(i):
        kc, vc = pools[i % copies]
        pa.reshape_and_cache(db.key_new, db.value_new, kc, vc, db.slot_new, db.geom)

    PS = args.partitioned
    if PS:
        P = -(-b.max_blocks_per_seq * b.block_size // PS)
        tmp = torch.empty((b.num_q_rows, b.num_q_heads, P, b.head_dim), dtype=torch.float32,
                          device=dev)
        ml = torch.empty((b.num_q_rows, b.num_q_heads, P), dtype=torch.float32, device=dev)
        es = torch.empty_like(ml)

    shared = int(b.meta.get("shared_prefix_blocks", 0))
    use_prefix = not PS and (args.path == "shared_prefix" or (args.path == "auto" and shared > 0))
    if use_prefix:
        if shared <= 0:
            print("bench.py: --path shared_prefix needs a batch with a shared prefix",
                  file=sys.stderr)
            sys.exit(2)
        db.set_shared_prefix([0, b.num_seqs], [shared], shared)
        pg, pk, pmax, pws = db.prefix

    def decode(i):
        kc, vc = pools[i % copies]
        if use_prefix:
            pa.decode_shared_prefix(db.out, db.q, kc, vc, db.block_tables, db.context_lens,
                                    db.qsl, pg, pk, pmax, db.scale, pws, db.geom,
                                    max_query_len=db.max_query_len)
        elif PS:
            pa.decode_partitioned(tmp, ml, es, db.q, kc, vc, db.block_tables, db.context_lens,
                                  db.qsl, db.scale, PS, P, db.geom)
            pa.decode_reduce(db.out, tmp, ml, es, P, db.geom)
        else:
            pa.decode(db.out, db.q, kc, vc, db.block_tables, db.context_lens, db.qsl, db.scale,
                      db.workspace, db.geom, max_query_len=db.max_query_len)

    print(f"[bench] warmup {args.warmup} steps, {copies} pool copies", file=sys.stderr,
          flush=True)
    for i in range(args.warmup):
        write(i)
        decode(i)
    torch.cuda.synchronize()

    # timed region: K whole steps (cache write + decode), nothing else on the stream
    ev_steps = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_steps[0].record(stream)
    for i in range(args.steps):
        write(args.warmup + i)
        decode(args.warmup + i)
    ev_steps[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {wall:.4f} s "
          f"(events: {ev_steps[0].elapsed_time(ev_steps[1]):.3f} ms)", file=sys.stderr, flush=True)

    # pa_decode's own duration: the same calls back to back between one pair of HIP events
    # on the stream it runs on (an event between two kernels stalls the next dispatch, so
    # per-call events would add their own gap to every call)
    ev_dec = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev_dec[0].record(stream)
    for i in range(args.steps):
        decode(args.warmup + i)
    ev_dec[1].record(stream)
    torch.cuda.synchronize()
    dec_ms = [ev_dec[0].elapsed_time(ev_dec[1]) / args.steps]
    # the same calls on one pool copy (no rotation): part of the pools stays in the
    # last-level cache from call to call
    ev_hot = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev_hot[0].record(stream)
    for i in range(args.steps):
        decode(0)
    ev_hot[1].record(stream)
    torch.cuda.synchronize()
    hot_ms = ev_hot[0].elapsed_time(ev_hot[1]) / args.steps

    ms_per_step = wall * 1e3 / args.steps
    dec_avg_ms = float(np.mean(dec_ms))
    seq_heads = b.num_q_rows * b.num_q_heads
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    flops = attention_flops(b)
    # HBM must deliver each distinct cached token once (a shared prefix is read from HBM
    # once and then from cache)
    hbm_bytes = b.kv_unique_bytes()
    # the bound of pa_decode: HBM for the KV bytes, or the matrix cores for its flops
    t_hbm = hbm_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS[b.dtype] * 1e12)
    if t_mfma > t_hbm:
        bound, achieved, peak, punit = "mfma", flops / (dec_avg_ms * 1e-3) / 1e12, \
            MFMA_PEAK_TFLOPS[b.dtype], "TFLOP/s"
    else:
        bound, achieved, peak, punit = "hbm", hbm_bytes / (dec_avg_ms * 1e-3) / 1e9, \
            HBM_PEAK_GBS, "GB/s"
    traffic_name = args.workload + (f"_part{PS}" if PS else "_decode" if shared and not use_prefix
                                    else "")
    traffic = read_traffic(traffic_name) if bound == "hbm" else None

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x {n} bytes", file=sys.stderr, flush=True)
        del src, dst

    cpu = None
    if args.cpu_seconds > 0:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        print(f"[bench] cpu oracle leg, {threads} threads", file=sys.stderr, flush=True)
        cpu = cpu_baseline(b, args.cpu_seconds, threads)

    line = {
        "metric": "paged-attn decode: effective KV-read HBM GB/s (% of peak) and seq-heads/sec",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"fp8_e4m3 KV, {b.dtype} q" if b.pool_dtype == "fp8" else b.dtype,
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "description": DESCRIPTIONS[args.workload],
            "num_seqs": b.num_seqs, "num_q_rows": b.num_q_rows,
            "num_q_heads": b.num_q_heads, "num_kv_heads": b.num_kv_heads,
            "head_dim": b.head_dim, "block_size": b.block_size,
            "kv_dtype": b.pool_dtype, "accumulate": "f32",
            "context_tokens": int(b.context_lens.astype(np.int64).sum()),
            "kv_bytes_per_step": kv_bytes,
            "kv_unique_bytes_per_step": hbm_bytes,
            "attention_flops_per_step": flops,
            "pool_copies_rotated": copies,
            "path": (f"pa_decode_partitioned({PS}) + pa_decode_reduce" if PS else
                     "pa_decode_shared_prefix (one group)" if use_prefix else "pa_decode"),
        },
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(seq_heads / (ms_per_step * 1e-3), 1),
        "pa_decode_us": round(dec_avg_ms * 1e3, 3),
        "pa_decode_hot_us": round(hot_ms * 1e3, 3),
        "roofline": {
            "bound": bound,
            "kernel": (f"pa_decode_partitioned ({PS}-token partitions) + pa_decode_reduce"
                       + (" (+ chunk kernel)" if b.query_start_loc is not None else "")
                       if PS else
                       "pa_decode_shared_prefix (prefix kernel + decode kernel with in-kernel "
                       "split merge and prefix fold)" if use_prefix else
                       "pa_decode (decode kernel with in-kernel split merge"
                       + (" + chunk kernel)" if runs_chunk_kernel(b) else ")")),
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": punit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
