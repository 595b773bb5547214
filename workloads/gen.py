"""Seeded synthetic inputs for attention over a paged KV cache.

This module draws random numbers and lays them out in the pool / block-table /
slot-mapping form that the library consumes.  It computes nothing of the
attention method itself (no gather, no dot products, no softmax), so the oracle
and the HIP path can both consume its output without sharing any of the
method's arithmetic.

Layout conventions (all row-major, numpy):

* ``k_pool``, ``v_pool``: ``[num_blocks, 16, num_kv_heads, head_dim]``.  bf16
  pools are ``np.uint16`` bit patterns, fp32 pools are ``np.float32``.  The
  fixed-size blocks drawn from one shared pool, and the block size of 16, follow
  "09 — Mini Inference Engine (The Capstone)", Week 4 — Paged KV cache.
* ``block_tables``: ``int32 [num_seqs, max_blocks_per_seq]``, logical block i of
  a sequence -> physical block id (same page and section).
* ``slot_mapping``: ``int32 [num_new_tokens]``; the flat slot of a token at
  position ``pos`` of sequence ``s`` is ``table[s][pos // 16] * 16 + pos % 16``,
  i.e. the row index in the pool viewed as ``[num_blocks * 16, heads * dim]``.
  ``-1`` marks a padding token that must not be written.
* ``context_lens`` count every token the attention call sees, including the
  ones written in this step.

Poisoning: every pool position that no sequence may read (unused blocks, the
slots past a sequence's length in its last block) and every position that the
KV write of this step must fill is set to NaN, and block-table padding points
at a NaN block when the pool has one.  A kernel that reads what it should not
therefore produces NaN.

Draw order from ``numpy.random.default_rng(seed)`` (PCG64): lengths, one
permutation of the physical block ids, Q, K, V, new-token K and V.  Values are
standard normal fp32, rounded to bf16 (round to nearest even) for bf16 batches.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK = 16
BF16_NAN = np.uint16(0x7FC0)
F16_NAN = np.uint16(0x7E00).view(np.float16)
F32_NAN_BITS = np.uint32(0x7FC00000)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.

    Finite inputs only (the generator never draws NaN or inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass
class PagedBatch:
    """One batch of attention work over a paged KV pool (host arrays)."""

    name: str
    seed: int
    dtype: str                    # "bf16" (uint16 bit patterns), "f16" or "f32"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context_lens: np.ndarray      # int32 [S]
    query_lens: np.ndarray        # int32 [S]; 1 for a decode sequence
    query_start_loc: np.ndarray   # int32 [S + 1]
    block_tables: np.ndarray      # int32 [S, max_blocks_per_seq]
    k_pool: np.ndarray            # [NB, 16, Hkv, D], state before the KV write
    v_pool: np.ndarray
    q: np.ndarray                 # [total_query_tokens, Hq, D]
    new_k: np.ndarray             # [T_new, Hkv, D]
    new_v: np.ndarray
    slot_mapping: np.ndarray      # int32 [T_new]
    num_prefill_seqs: int
    recipe: str
    shared_prefix_tokens: int = 0   # leading tokens every sequence's table shares

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def total_query_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def used_block_ids(self) -> np.ndarray:
        """Physical ids referenced by some sequence within its length."""
        bs = self.k_pool.shape[1]
        ids = [self.block_tables[s, : -(-int(L) // bs)] for s, L in enumerate(self.context_lens)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)


def _values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x.astype(np.float16) if dtype == "f16" else x    # fp32 -> fp16 rounds to nearest even


def _poison_value(dtype: str):
    if dtype == "bf16":
        return BF16_NAN
    return F16_NAN if dtype == "f16" else F32_NAN_BITS.view(np.float32)


def make_batch(
    seed: int,
    *,
    name: str,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    draw_lens,
    draw_query_lens=None,
    pool_factor: float = 1.2,
    pool_blocks: int | None = None,
    shared_prefix_blocks: int = 0,
    num_prefill_seqs: int = 0,
    extra_table_cols: int = 0,
    pad_slots: int = 0,
    block_size: int = BLOCK,
    recipe: str = "",
) -> PagedBatch:
    """Draw one batch.

    ``draw_lens(rng) -> int array`` gives the context lengths (first draw).
    ``draw_query_lens(rng, lens)`` gives per-sequence new-token counts (default
    1 everywhere, i.e. a decode step); it may only use ``lens`` and constants,
    not the rng, so the documented draw order holds.
    ``shared_prefix_blocks``: logical blocks 0..n-1 of every sequence map to the
    same physical blocks (read-only aliasing, as a prefix-cache hit produces).
    ``pad_slots``: extra new tokens with slot -1 appended to the write.
    ``block_size``: tokens per pool block (16, the pages' choice, by default).
    """
    bs = block_size
    assert dtype in ("bf16", "f16", "f32")
    rng = np.random.default_rng(seed)
    lens = np.asarray(draw_lens(rng), dtype=np.int64)
    S = int(lens.shape[0])
    qlens = (np.ones(S, np.int64) if draw_query_lens is None
             else np.asarray(draw_query_lens(rng, lens), np.int64))
    assert np.all(qlens >= 0) and np.all(qlens <= lens)
    nblk = -(-lens // bs)                      # blocks each sequence occupies
    assert np.all(nblk >= shared_prefix_blocks)
    private = nblk - shared_prefix_blocks
    used = int(shared_prefix_blocks + private.sum())
    if pool_blocks is None:
        pool_blocks = int(math.ceil(pool_factor * used))
    assert pool_blocks >= used

    # (2) one permutation of the physical ids, dealt in order: shared prefix
    # first, then each sequence's private logical blocks.
    perm = rng.permutation(pool_blocks).astype(np.int64)
    max_blocks = int(nblk.max()) + extra_table_cols if S else 1
    tables = np.zeros((S, max(max_blocks, 1)), np.int64)
    shared_ids = perm[:shared_prefix_blocks]
    cursor = shared_prefix_blocks
    for s in range(S):
        tables[s, :shared_prefix_blocks] = shared_ids
        n = int(private[s])
        tables[s, shared_prefix_blocks:shared_prefix_blocks + n] = perm[cursor:cursor + n]
        cursor += n
    unused_ids = perm[cursor:]
    pad_id = int(unused_ids[0]) if unused_ids.size else 0
    for s in range(S):
        tables[s, int(nblk[s]):] = pad_id

    T = int(qlens.sum())
    qsl = np.zeros(S + 1, np.int64)
    qsl[1:] = np.cumsum(qlens)

    # (3)-(6) values.
    q = _values(rng, (T, num_q_heads, head_dim), dtype)
    pool_shape = (pool_blocks, bs, num_kv_heads, head_dim)
    k_pool = _values(rng, pool_shape, dtype)
    v_pool = _values(rng, pool_shape, dtype)
    new_k = _values(rng, (T + pad_slots, num_kv_heads, head_dim), dtype)
    new_v = _values(rng, (T + pad_slots, num_kv_heads, head_dim), dtype)

    # Poison: unused blocks, slots past each length, and the slots this step's
    # KV write must fill.  Build the flat slot of every new token.
    poison = _poison_value(dtype)
    k_rows = k_pool.reshape(pool_blocks * bs, num_kv_heads, head_dim)
    v_rows = v_pool.reshape(pool_blocks * bs, num_kv_heads, head_dim)
    if unused_ids.size:
        k_pool[unused_ids] = poison
        v_pool[unused_ids] = poison
    slots = np.full(T + pad_slots, -1, np.int64)
    for s in range(S):
        L, n = int(lens[s]), int(qlens[s])
        if L == 0:
            continue
        last = int(tables[s, (L - 1) // bs])
        tail = (L - 1) % bs + 1
        k_pool[last, tail:] = poison
        v_pool[last, tail:] = poison
        pos = np.arange(L - n, L)
        rows = tables[s, pos // bs] * bs + pos % bs
        slots[qsl[s]:qsl[s] + n] = rows
        k_rows[rows] = poison
        v_rows[rows] = poison

    return PagedBatch(
        name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim,
        context_lens=lens.astype(np.int32), query_lens=qlens.astype(np.int32),
        query_start_loc=qsl.astype(np.int32), block_tables=tables.astype(np.int32),
        k_pool=k_pool, v_pool=v_pool, q=q, new_k=new_k, new_v=new_v,
        slot_mapping=slots.astype(np.int32), num_prefill_seqs=num_prefill_seqs,
        recipe=recipe, shared_prefix_tokens=shared_prefix_blocks * bs,
    )


def packed_qkv(b: PagedBatch, pad_cols: int = 0) -> np.ndarray:
    """The batch's new-token q, k and v as the rows of one packed projection
    output, [T, (Hq + 2*Hkv) * D + pad_cols]: q heads, then k heads, then v
    heads (pad columns hold poison).  Reuses the batch's draws."""
    T = b.q.shape[0]
    hq, hkv, d = b.num_q_heads, b.num_kv_heads, b.head_dim
    parts = [b.q.reshape(T, hq * d), b.new_k[:T].reshape(T, hkv * d), b.new_v[:T].reshape(T, hkv * d)]
    if pad_cols:
        parts.append(np.full((T, pad_cols), _poison_value(b.dtype), dtype=b.q.dtype))
    return np.ascontiguousarray(np.concatenate(parts, axis=1))


def norm_weights(b: PagedBatch, seed: int):
    """Per-head RMSNorm weights for q and k, [D] each: 1 + 0.1 * N(0, 1),
    stored like the batch (drawn from their own generator)."""
    rng = np.random.default_rng(seed)
    w = (1.0 + 0.1 * rng.standard_normal(size=(2, b.head_dim))).astype(np.float32)
    w = f32_to_bf16_bits(w) if b.dtype == "bf16" else (w.astype(np.float16) if b.dtype == "f16" else w)
    return w[0].copy(), w[1].copy()


# ---------------------------------------------------------------------------
# Workloads shaped like the pages' benchmarks.  Head shapes follow the model
# each page names; the sizes keyword arguments shrink them for parity tests.
# ---------------------------------------------------------------------------

def tiny_f32(seed: int = 1) -> PagedBatch:
    """4 sequences of lengths 5, 17, 33, 64; 2 q heads / 1 kv head, dim 64,
    fp32, a pool of 32 blocks with permuted ids; one write of 4 new tokens."""
    return make_batch(
        seed, name="tiny_f32", dtype="f32", num_q_heads=2, num_kv_heads=1,
        head_dim=64, draw_lens=lambda rng: np.array([5, 17, 33, 64]),
        pool_blocks=32,
        recipe="lens {5,17,33,64}; pool 32 blocks; N(0,1) fp32")


def qwen25_05b_decode(seed: int = 2, batch: int = 32, lo: int = 128, hi: int = 1024,
                      dtype: str = "bf16", block_size: int = BLOCK) -> PagedBatch:
    """Qwen2.5-0.5B-shaped decode step: 14 q / 2 kv heads, dim 64, bf16,
    lengths uniform in [lo, hi]; pool 1.2x the blocks in use."""
    return make_batch(
        seed, name="qwen25_05b_decode", dtype=dtype, block_size=block_size, num_q_heads=14,
        num_kv_heads=2, head_dim=64,
        draw_lens=lambda rng: rng.integers(lo, hi + 1, size=batch),
        recipe=f"B={batch}, L~U[{lo},{hi}], pool 1.2x, N(0,1)->bf16")


def qwen3_06b_decode(seed: int = 3, batch: int = 256, prompt=(100, 1024),
                     gen=(0, 1024), cap: int = 2048, dtype: str = "bf16",
                     block_size: int = BLOCK) -> PagedBatch:
    """Qwen3-0.6B-shaped decode step: 16 q / 8 kv heads, dim 128, bf16,
    length = prompt U[100,1024] + generated U[0,1024], capped at 2048; pool
    1.2x the blocks in use with permuted ids."""
    def lens(rng):
        p = rng.integers(prompt[0], prompt[1] + 1, size=batch)
        g = rng.integers(gen[0], gen[1] + 1, size=batch)
        return np.minimum(p + g, cap)
    return make_batch(
        seed, name="qwen3_06b_decode", dtype=dtype, block_size=block_size, num_q_heads=16,
        num_kv_heads=8, head_dim=128, draw_lens=lens,
        recipe=f"B={batch}, L=min(U{list(prompt)}+U{list(gen)},{cap}), pool 1.2x, N(0,1)->bf16")


def mixed_prefill(seed: int = 4, chunks: int = 4, chunk_len: int = 512,
                  prior_hi: int = 1536, n_decode: int = 192,
                  dec_lo: int = 256, dec_hi: int = 2048, num_q_heads: int = 16,
                  num_kv_heads: int = 8, head_dim: int = 128,
                  chunk_lens=None, dtype: str = "bf16", block_size: int = BLOCK) -> PagedBatch:
    """Mixed chunked-prefill batch, by default the Qwen3-0.6B head shape (16 / 8 / 128, bf16):
    ``chunks`` prefill chunks of ``chunk_len`` new tokens (or the lengths listed
    in ``chunk_lens``) after a cached prior context U[0, prior_hi], followed by
    ``n_decode`` decode sequences with length U[dec_lo, dec_hi].  Prefill
    sequences come first."""
    if chunk_lens is not None:
        chunks = len(chunk_lens)
        new_tokens = np.asarray(chunk_lens, np.int64)
    else:
        new_tokens = np.full(chunks, chunk_len, np.int64)

    def lens(rng):
        prior = rng.integers(0, prior_hi + 1, size=chunks)
        dec = rng.integers(dec_lo, dec_hi + 1, size=n_decode)
        return np.concatenate([prior + new_tokens, dec])

    def qlens(rng, L):
        return np.concatenate([new_tokens, np.ones(n_decode, np.int64)])
    return make_batch(
        seed, name="mixed_prefill", dtype=dtype, block_size=block_size, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, draw_lens=lens, draw_query_lens=qlens,
        num_prefill_seqs=chunks,
        recipe=(f"{chunks} chunks x {[int(x) for x in new_tokens] if chunk_lens is not None else chunk_len} "
                f"after prior U[0,{prior_hi}]; "
                f"{n_decode} decode seqs L~U[{dec_lo},{dec_hi}]; pool 1.2x; N(0,1)->bf16"))


def long_context(seed: int = 5, batch: int = 64, ctx: int = 8192,
                 shared_blocks: int = 256, block_size: int = BLOCK) -> PagedBatch:
    """Qwen2.5-7B-shaped long-context decode: 28 q / 4 kv heads, dim 128,
    bf16, every sequence at ``ctx`` tokens, whose first ``shared_blocks``
    logical blocks (of 16 tokens: the shared prefix is 16 * shared_blocks
    tokens at any block size) are the same physical blocks for all
    sequences; the pool holds exactly the blocks in use."""
    return make_batch(
        seed, name="long_context", dtype="bf16", num_q_heads=28, num_kv_heads=4,
        head_dim=128, draw_lens=lambda rng: np.full(batch, ctx), block_size=block_size,
        pool_factor=1.0, shared_prefix_blocks=shared_blocks * BLOCK // block_size,
        recipe=f"B={batch}, L={ctx}, shared prefix {shared_blocks} blocks, N(0,1)->bf16")


PRESETS = {
    "tiny_f32": tiny_f32,
    "qwen25_05b_decode": qwen25_05b_decode,
    "qwen3_06b_decode": qwen3_06b_decode,
    "mixed_prefill": mixed_prefill,
    "long_context": long_context,
}
