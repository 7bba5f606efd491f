"""Host-side checks of bench.py's contract (no GPU): the one-GPU guard, workload names and
the multi-row kernel label."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_every_preset_has_a_bench_description():
    import bench
    from paged_kv_cache_445_amd import workloads as W
    for name in W.PRESETS:
        assert name in bench.DESCRIPTIONS, name
    extra = set(bench.DESCRIPTIONS) - set(W.PRESETS)
    assert extra == set(bench.MEASURE_WORKLOADS)
    assert {"hbm_read_ceiling", "tile_replay_llama7b_f16"} <= extra


@pytest.mark.parametrize("dtype,Hq,Hkv,rows,fp8,chunk", [
    ("f16", 8, 8, 1, False, False),     # decode rows only
    ("f16", 8, 8, 6, False, False),     # MHA verify rows: up to 16 a sequence
    ("bf16", 8, 2, 4, False, False),    # G = 4: up to 4 rows
    ("bf16", 8, 2, 5, False, True),
    ("f16", 8, 8, 6, True, False),      # FP8 pools route like 16-bit ones
    ("bf16", 8, 2, 40, True, True),
    ("f32", 4, 4, 2, False, True)])     # fp32: one row a sequence
def test_chunk_kernel_label_follows_the_row_counts(dtype, Hq, Hkv, rows, fp8, chunk):
    import numpy as np
    import bench
    from paged_kv_cache_445_amd import workloads as W
    rng = np.random.default_rng(5)
    n = np.array([1, rows, 1])
    b = W.build_batch("label", dtype, n + 20, n, Hq, Hkv, 64, rng)
    if fp8:
        b.kv_dtype = "fp8"
    assert bench.runs_chunk_kernel(b) is chunk
