"""pa_decode_scratch (the allocation-free pa_decode) through the C ABI against pa_decode and
the fp64 oracle: two calls in a row on one device, the second on a smaller batch, so the
second call finds the static workspace as the first left it."""
import numpy as np
import pytest

from paged_kv_cache_445_amd import workloads as W
from tests import helpers as H

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def _log(msg):
    print(msg, flush=True)


def _both(b):
    """pa_decode (own workspace) and pa_decode_scratch on the same device batch; returns both
    outputs and the oracle's."""
    import torch
    from paged_kv_cache_445_amd import pa
    from paged_kv_cache_445_amd.device_batch import DeviceBatch
    _log(f"[no_alloc] {b.name} {b.dtype} S={b.num_seqs} rows={b.num_q_rows} "
         f"Hq={b.num_q_heads} Hkv={b.num_kv_heads} D={b.head_dim}")
    db = DeviceBatch(b)
    db.prefill()
    db.write_new()
    db.attend()
    torch.cuda.synchronize()
    ref = db.out_host()
    out = torch.full_like(db.out, float("nan"))
    pa.decode_scratch(out, db.q, db.k_cache, db.v_cache, db.block_tables, db.context_lens,
                      db.qsl, db.scale, db.geom, max_query_len=db.max_query_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want, _ = H.oracle_attention(b, *H.oracle_pools(b))
    return got, ref, want


def _check(got, want, tol, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want).max()
    assert err <= tol, f"{what}: max abs err {err:.3e} (tol {tol})"


def test_scratch_decode_matches_pa_decode_twice():
    """A larger GQA batch (matrix-core path, segments split over workgroups and merged in
    the kernel), then a smaller MHA batch (vector path): bit for bit pa_decode's output and
    within tolerance of the oracle, both times."""
    rng = np.random.default_rng(4700)
    big = W.build_batch("scratch_big", "bf16", rng.integers(1, 6000, size=40), np.ones(40), 16,
                        2, 128, rng)
    small = W.build_batch("scratch_small", "f16", rng.integers(1, 900, size=9), np.ones(9), 8,
                          8, 128, rng)
    for b in (big, small):
        got, ref, want = _both(b)
        assert np.array_equal(got, ref), f"{b.name}: differs from pa_decode"
        _check(got, want, TOL[b.dtype], b.name)


def test_scratch_decode_multi_row_then_smaller():
    """Chunked-prefill and verify rows (the chunk kernel then the decode kernel on one
    stream), then a smaller decode-only batch."""
    rng = np.random.default_rng(4701)
    n = np.array([130, 1, 4, 1, 37, 2])
    prior = np.array([300, 55, 2000, 17, 0, 900])
    rows = W.build_batch("scratch_rows", "bf16", prior + n, n, 16, 4, 128, rng)
    small = W.build_batch("scratch_small2", "bf16", rng.integers(1, 700, size=5), np.ones(5), 16,
                          4, 128, rng)
    got, ref, want = _both(rows)
    _check(got, want, TOL["bf16"], "multi-row, scratch")
    _check(got, ref, TOL["bf16"], "multi-row, scratch vs pa_decode")
    got, ref, want = _both(small)
    assert np.array_equal(got, ref), "second call: differs from pa_decode"
    _check(got, want, TOL["bf16"], "second call")
