"""Seeded synthetic paged-KV batches: the inputs both the GPU library and the CPU oracle see.

This module holds no attention arithmetic.  It plays the caller's role: it draws context
lengths and values, assigns physical blocks from a seeded permutation the way a block
manager would ("vLLM 深度拆解" §3.2 block pool, §3.3 block table; "vLLM 架构源码解析 第1篇"
§3.3.2 block_tables / slot_mapping / query_start_loc), and hands out

  * block_tables  int32 [S, MB]   logical block j of seq s -> physical block
  * context_lens  int32 [S]       tokens in the context, including this step's new ones
  * query_start_loc int32 [S+1]   or None when every sequence has exactly one query row
  * q             [Nq, Hq, D]     storage dtype
  * token records: key/value [R, Hkv, D] and slot [R] (slot = block * 16 + offset, the
    caller's metadata), split into `history` (already cached) and `new` (written by
    this step's reshape_and_cache)
  * seq_tokens    per sequence, the record index of every context position

Storage dtypes: "f32" -> float32, "f16" -> float16, "bf16" -> uint16 holding bfloat16 bits
(float32 values rounded to nearest-even).  Pools are filled with a NaN pattern before any
write, so any slot the method must not read (unassigned blocks, the sentinel block that
pads block-table rows, the slots past the context in a last block) is NaN.

Configurations (seed 4450 + i, numpy default_rng; draw order: context lengths, block
permutation, q, history K, history V, new K, new V):
  tiny_f32            4 seqs, 4/4 heads, D 64, fp32, ctx U[1,200], 64 blocks
  llama7b_f16         32 seqs, 32/32 heads, D 128, fp16, ctx U[256,2048], 8192 blocks
  gqa_long_bf16       64 seqs, 64/8 heads, D 128, bf16, ctx log-uniform [128,32768], sigma 0.5
  prefix_shared_f16   128 seqs, 32/32 heads, D 128, fp16, 32 shared leading blocks,
                      private tail U[16,1024], one new token per seq
  mixed_chunked_bf16  8 chunk seqs (512 rows, prior ctx U[0,7488]) + 120 decode seqs
                      (ctx U[64,4096]); 32/8 heads, D 128, bf16
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "fp8": 0x7F}


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to the storage dtype (bf16: round-to-nearest-even of float32)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16)
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    return ((b + (0x7FFF + ((b >> 16) & 1))) >> 16).astype(np.uint16)


def storage_to_float32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float32 (every f16/bf16 value is a float32)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def nan_pool(shape, dtype: str) -> np.ndarray:
    pool = np.empty(shape, dtype=STORAGE[dtype])
    if dtype == "f32":
        pool.view(np.uint32).fill(NAN_BITS[dtype])
    elif dtype == "fp8":
        pool.fill(NAN_BITS[dtype])
    else:
        pool.view(np.uint16).fill(NAN_BITS[dtype])
    return pool


def _normal(rng, n: int, sigma: float, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """n normal values (float32 draws, in chunks of 2^24) rounded to the storage dtype."""
    out = np.empty(n, dtype=STORAGE[dtype])
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        out[a:b] = to_storage(rng.standard_normal(b - a, dtype=np.float32) * np.float32(sigma),
                              dtype)
    return out


@dataclass
class Batch:
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: np.float32
    context_lens: np.ndarray
    query_start_loc: np.ndarray | None
    block_tables: np.ndarray
    q: np.ndarray
    key: np.ndarray
    value: np.ndarray
    slot: np.ndarray
    history: np.ndarray
    new: np.ndarray
    seq_tokens: list
    sentinel_block: int
    block_size: int = BLOCK_SIZE
    partition_size: int = 512
    meta: dict = field(default_factory=dict)
    kv_dtype: str = ""      # the pools' element type when it differs from dtype ("fp8")
    k_scale: float = 1.0    # FP8 pools: per-pool scales (calibration inputs)
    v_scale: float = 1.0

    @property
    def pool_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def num_q_rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def x(self) -> int:
        """Elements per 16-byte chunk of the K pool's innermost dimension."""
        return 16 // ELEM_BYTES[self.pool_dtype]

    def k_pool_shape(self):
        """[NB][Hkv][D/X][16][X] for 16-token blocks; a larger block is R = block_size / 16
        sub-blocks of 16 tokens, [NB][R][Hkv][D/X][16][X] (the pool layout of the ABI)."""
        D, X = self.head_dim, self.x
        T = min(self.block_size, 16)
        R = self.block_size // T
        if R == 1:
            return (self.num_blocks, self.num_kv_heads, D // X, T, X)
        return (self.num_blocks, R, self.num_kv_heads, D // X, T, X)

    def v_pool_shape(self):
        T = min(self.block_size, 16)
        R = self.block_size // T
        if R == 1:
            return (self.num_blocks, self.num_kv_heads, self.head_dim, T)
        return (self.num_blocks, R, self.num_kv_heads, self.head_dim, T)

    def rows_per_seq(self) -> np.ndarray:
        if self.query_start_loc is None:
            return np.ones(self.num_seqs, dtype=np.int64)
        return np.diff(self.query_start_loc).astype(np.int64)

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes of one decode pass: every context token's K and V read once
        per KV head (GQA sharing not multiplied)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * \
            self.head_dim * 2 * ELEM_BYTES[self.pool_dtype]

    def kv_unique_bytes(self) -> int:
        """KV bytes of the distinct cached tokens a pass reads: a token shared by several
        sequences (a common prefix block) counts once."""
        distinct = np.unique(np.concatenate(self.seq_tokens)) if self.num_seqs else []
        return int(len(distinct)) * self.num_kv_heads * self.head_dim * 2 * \
            ELEM_BYTES[self.pool_dtype]

    def step_slots(self) -> np.ndarray:
        return self.slot[self.new]


def build_batch(name: str, dtype: str, context_lens, rows_per_seq, num_q_heads: int,
                num_kv_heads: int, head_dim: int, rng, sigma: float = 1.0,
                num_blocks: int | None = None, max_blocks_per_seq: int | None = None,
                shared_prefix_blocks: int = 0, partition_size: int = 512,
                force_qsl: bool = False, block_size: int = BLOCK_SIZE) -> Batch:
    """Assemble a batch from already-drawn context lengths (rng continues from there)."""
    BS = int(block_size)
    ctx = np.asarray(context_lens, dtype=np.int64)
    nrows = np.asarray(rows_per_seq, dtype=np.int64)
    S = len(ctx)
    assert len(nrows) == S
    nblk = (ctx + BS - 1) // BS
    shared = int(shared_prefix_blocks)
    if shared:
        assert np.all(ctx - nrows >= shared * BS), "new tokens must land in private blocks"
    private = np.maximum(nblk - shared, 0)
    needed = shared + int(private.sum())
    if num_blocks is None:
        num_blocks = ((needed + 63) // 64) * 64 + 64
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(nblk.max()) if S else 1)
    assert needed < num_blocks, "pool too small (one block is kept as the sentinel)"
    assert S == 0 or nblk.max() <= max_blocks_per_seq

    # ---- physical blocks: one seeded permutation; its last entry is never assigned
    perm = rng.permutation(num_blocks).astype(np.int64)
    sentinel = int(perm[-1])
    tables = np.full((S, max_blocks_per_seq), sentinel, dtype=np.int32)
    cursor = shared
    for s in range(S):
        tables[s, :min(shared, nblk[s])] = perm[:min(shared, nblk[s])]
        k = int(private[s])
        tables[s, shared:shared + k] = perm[cursor:cursor + k]
        cursor += k

    # ---- query rows
    nq = int(nrows.sum())
    q = _normal(rng, nq * num_q_heads * head_dim, sigma, dtype).reshape(nq, num_q_heads, head_dim)
    qsl = None
    if force_qsl or np.any(nrows != 1):
        qsl = np.zeros(S + 1, dtype=np.int32)
        qsl[1:] = np.cumsum(nrows)

    # ---- token records: shared prefix once, then each sequence's private history, then
    #      the new tokens (the last n_s positions of each sequence)
    seq_tokens = [np.empty(int(c), dtype=np.int64) for c in ctx]
    rec_seq, rec_pos = [], []
    prefix_tokens = shared * BS
    if shared:
        rec_seq.append(np.zeros(prefix_tokens, dtype=np.int64))
        rec_pos.append(np.arange(prefix_tokens, dtype=np.int64))
        for s in range(S):
            seq_tokens[s][:prefix_tokens] = np.arange(prefix_tokens)
    r = prefix_tokens
    for s in range(S):
        a, b = prefix_tokens, int(ctx[s] - nrows[s])
        if b > a:
            rec_seq.append(np.full(b - a, s, dtype=np.int64))
            rec_pos.append(np.arange(a, b, dtype=np.int64))
            seq_tokens[s][a:b] = np.arange(r, r + b - a)
            r += b - a
    num_history = r
    for s in range(S):
        a, b = max(int(ctx[s] - nrows[s]), 0), int(ctx[s])
        if b > a:
            rec_seq.append(np.full(b - a, s, dtype=np.int64))
            rec_pos.append(np.arange(a, b, dtype=np.int64))
            seq_tokens[s][a:b] = np.arange(r, r + b - a)
            r += b - a
    R = r
    rec_seq = np.concatenate(rec_seq) if rec_seq else np.zeros(0, np.int64)
    rec_pos = np.concatenate(rec_pos) if rec_pos else np.zeros(0, np.int64)
    # caller metadata: slot = physical block * block_size + offset in the block
    slot = tables[rec_seq, rec_pos // BS].astype(np.int64) * BS + rec_pos % BS

    per = num_kv_heads * head_dim
    kh = _normal(rng, num_history * per, sigma, dtype)
    vh = _normal(rng, num_history * per, sigma, dtype)
    kn = _normal(rng, (R - num_history) * per, sigma, dtype)
    vn = _normal(rng, (R - num_history) * per, sigma, dtype)
    key = np.concatenate([kh, kn]).reshape(R, num_kv_heads, head_dim)
    value = np.concatenate([vh, vn]).reshape(R, num_kv_heads, head_dim)

    return Batch(name=name, dtype=dtype, num_seqs=S, num_q_heads=num_q_heads,
                 num_kv_heads=num_kv_heads, head_dim=head_dim, num_blocks=int(num_blocks),
                 max_blocks_per_seq=int(max_blocks_per_seq),
                 scale=np.float32(1.0 / math.sqrt(head_dim)),
                 context_lens=ctx.astype(np.int32), query_start_loc=qsl, block_tables=tables,
                 q=q, key=key, value=value, slot=slot,
                 history=np.arange(num_history, dtype=np.int64),
                 new=np.arange(num_history, R, dtype=np.int64), seq_tokens=seq_tokens,
                 sentinel_block=sentinel, partition_size=partition_size, block_size=BS,
                 meta={"shared_prefix_blocks": shared} if shared else {})


# --------------------------------------------------------------------------- presets

def tiny_f32(seed: int = 4450) -> Batch:
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, 201, size=4)
    return build_batch("tiny_f32", "f32", ctx, np.ones(4), 4, 4, 64, rng,
                       num_blocks=64, max_blocks_per_seq=13)


def llama7b_f16(seed: int = 4451, num_seqs: int = 32) -> Batch:
    rng = np.random.default_rng(seed)
    ctx = rng.integers(256, 2049, size=num_seqs)
    return build_batch("llama7b_f16", "f16", ctx, np.ones(num_seqs), 32, 32, 128, rng,
                       num_blocks=8192, max_blocks_per_seq=128)


def llama7b_f16_bs8(seed: int = 4451, num_seqs: int = 32) -> Batch:
    """The LLaMA-7B-shaped batch (same context lengths and values) with 8-token blocks
    ("vLLM 架构源码解析 第1篇" §5.1 weighs block sizes 8, 16 and 32): 8192 blocks of 8 tokens,
    256 table entries per sequence."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(256, 2049, size=num_seqs)
    return build_batch("llama7b_f16_bs8", "f16", ctx, np.ones(num_seqs), 32, 32, 128, rng,
                       num_blocks=8192, max_blocks_per_seq=256, block_size=8)


def gqa_long_bf16(seed: int = 4452, num_seqs: int = 64, max_ctx: int = 32768) -> Batch:
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(128), math.log(max_ctx), size=num_seqs)
    ctx = np.clip(np.rint(np.exp(u)), 128, max_ctx).astype(np.int64)
    return build_batch("gqa_long_bf16", "bf16", ctx, np.ones(num_seqs), 64, 8, 128, rng,
                       sigma=0.5, max_blocks_per_seq=(max_ctx + 15) // 16, partition_size=512)


def prefix_shared_f16(seed: int = 4453, num_seqs: int = 128) -> Batch:
    rng = np.random.default_rng(seed)
    tail = rng.integers(16, 1025, size=num_seqs)
    ctx = 512 + tail + 1  # shared 512-token prefix + private tail + the token written now
    return build_batch("prefix_shared_f16", "f16", ctx, np.ones(num_seqs), 32, 32, 128, rng,
                       max_blocks_per_seq=97, shared_prefix_blocks=32)


def mixed_chunked_bf16(seed: int = 4454, num_chunk: int = 8, num_decode: int = 120,
                       chunk: int = 512, prior_zero: bool = False) -> Batch:
    rng = np.random.default_rng(seed)
    prior = np.zeros(num_chunk, dtype=np.int64) if prior_zero else \
        rng.integers(0, 7489, size=num_chunk)
    dec = rng.integers(64, 4097, size=num_decode)
    ctx = np.concatenate([prior + chunk, dec])
    rows = np.concatenate([np.full(num_chunk, chunk), np.ones(num_decode, dtype=np.int64)])
    return build_batch("mixed_chunked_bf16", "bf16", ctx, rows, 32, 8, 128, rng,
                       max_blocks_per_seq=500)


def prefill_chunks_bf16(seed: int = 4454, num_chunk: int = 8, chunk: int = 512) -> Batch:
    """The chunked-prefill rows of the mixed step alone: 8 sequences of 512 causal rows over
    prior contexts U[0, 7488] (the same prior draws), 32 q / 8 KV heads, head_dim 128, bf16."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(0, 7489, size=num_chunk)
    rng.integers(64, 4097, size=120)  # the mixed step's decode contexts, not used here
    return build_batch("prefill_chunks_bf16", "bf16", prior + chunk, np.full(num_chunk, chunk),
                       32, 8, 128, rng, max_blocks_per_seq=500)


def llama7b_fp8(seed: int = 4451, num_seqs: int = 32) -> Batch:
    """The LLaMA-7B-shaped batch (same draws) with FP8 E4M3 pools: fp16 q, keys and values,
    quantised by the cache write with per-pool scales 6.5 / 448 (N(0, 1) values beyond 6.5
    saturate; none is expected at this size)."""
    b = llama7b_f16(seed, num_seqs)
    b.name = "llama7b_fp8"
    b.kv_dtype = "fp8"
    b.k_scale = b.v_scale = float(np.float32(6.5 / 448))
    return b


def gqa_long_fp8(seed: int = 4452, num_seqs: int = 64, max_ctx: int = 32768) -> Batch:
    """The GQA long-context batch's shape (64 q / 8 KV heads, log-uniform contexts to 32768)
    with FP8 E4M3 pools and fp16 q, keys and values (N(0, 0.5); per-pool scales 3.25 / 448)."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(128), math.log(max_ctx), size=num_seqs)
    ctx = np.clip(np.rint(np.exp(u)), 128, max_ctx).astype(np.int64)
    b = build_batch("gqa_long_fp8", "f16", ctx, np.ones(num_seqs), 64, 8, 128, rng, sigma=0.5,
                    max_blocks_per_seq=(max_ctx + 15) // 16, partition_size=512)
    b.kv_dtype = "fp8"
    b.k_scale = b.v_scale = float(np.float32(3.25 / 448))
    return b


def spec_verify_f16(seed: int = 4455, num_seqs: int = 32, num_draft: int = 5) -> Batch:
    """Speculative-decoding verify step on the LLaMA-7B shape ("vLLM 深度拆解" §5.1: the
    target model checks num_draft drafted tokens in one pass): every sequence runs the last
    accepted token plus its num_draft drafts as num_draft + 1 causal query rows over a
    prior context U[256, 2048]."""
    rng = np.random.default_rng(seed)
    n = num_draft + 1
    prior = rng.integers(256, 2049, size=num_seqs)
    return build_batch("spec_verify_f16", "f16", prior + n, np.full(num_seqs, n), 32, 32, 128,
                       rng, num_blocks=8192, max_blocks_per_seq=129)


def spec_verify_gqa_bf16(seed: int = 4456, num_seqs: int = 64, num_draft: int = 3) -> Batch:
    """The verify step on a GQA shape (32 query / 8 KV heads): 4 causal rows per sequence,
    prior context U[512, 4096]."""
    rng = np.random.default_rng(seed)
    n = num_draft + 1
    prior = rng.integers(512, 4097, size=num_seqs)
    return build_batch("spec_verify_gqa_bf16", "bf16", prior + n, np.full(num_seqs, n), 32, 8,
                       128, rng, max_blocks_per_seq=257)


def mixed_chunked_fp8(seed: int = 4454) -> Batch:
    """The mixed chunked-prefill step (same draws) with FP8 E4M3 pools behind bf16 queries,
    per-pool scales 6.5 / 448."""
    b = mixed_chunked_bf16(seed)
    b.name = "mixed_chunked_fp8"
    b.kv_dtype = "fp8"
    b.k_scale = b.v_scale = float(np.float32(6.5 / 448))
    return b


def spec_verify_fp8(seed: int = 4455, num_seqs: int = 32, num_draft: int = 5) -> Batch:
    """The LLaMA-7B verify step (same draws) with FP8 E4M3 pools at per-pool scales
    6.5 / 448."""
    b = spec_verify_f16(seed, num_seqs, num_draft)
    b.name = "spec_verify_fp8"
    b.kv_dtype = "fp8"
    b.k_scale = b.v_scale = float(np.float32(6.5 / 448))
    return b


PRESETS = {
    "tiny_f32": tiny_f32,
    "llama7b_f16": llama7b_f16,
    "llama7b_f16_bs8": llama7b_f16_bs8,
    "gqa_long_bf16": gqa_long_bf16,
    "prefix_shared_f16": prefix_shared_f16,
    "mixed_chunked_bf16": mixed_chunked_bf16,
    "llama7b_fp8": llama7b_fp8,
    "gqa_long_fp8": gqa_long_fp8,
    "spec_verify_f16": spec_verify_f16,
    "spec_verify_gqa_bf16": spec_verify_gqa_bf16,
    "spec_verify_fp8": spec_verify_fp8,
    "mixed_chunked_fp8": mixed_chunked_fp8,
    "prefill_chunks_bf16": prefill_chunks_bf16,
}


def make(name: str, **kw) -> Batch:
    return PRESETS[name](**kw)


def chunk_split(num_tokens: int, chunk: int = 512) -> list:
    """Chunked-prefill split of a prompt into chunk-sized pieces plus a remainder."""
    return [min(chunk, num_tokens - a) for a in range(0, num_tokens, chunk)]
