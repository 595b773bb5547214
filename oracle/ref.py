"""Plain fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only the test suite, the package's smoke check and the
CPU-baseline leg of the benchmark may import this module.  It shares no code
with the HIP library and imports nothing from it; it is slow on purpose and
written so that each step can be checked against the pages by eye.

What it follows:

* The KV pool is one shared set of fixed-size blocks (block size 16), and each
  sequence owns a block table mapping its logical block i to a physical block
  id; attention gathers K/V through that table.  ("09 — Mini Inference Engine
  (The Capstone)", Week 4 — Paged KV cache; "mini-vllm", Milestones item 2.)
* Each step's new K/V is written into the pool at a flat slot (the KV-cache
  write that "mini_engine", Next: fused kernels, lists as a fusion target; the
  slot derivation of "mini-vllm", Milestones item 7).  Reading: slot =
  physical_block * 16 + offset_in_block; a negative slot is a padding token.
* The model uses grouped-query attention ("mini_engine", What it does): query
  head h reads kv head h // G, G = num_q_heads / num_kv_heads (contiguous
  groups, the repeat-KV convention).
* Decode attention runs batched over a ragged set of sequences ("mini-vllm",
  Milestones item 6) and prefill may arrive in chunks under a token budget,
  mixed with decodes in one batch ("mini_engine", What it does; "09 — Mini
  Inference Engine (The Capstone)", Week 3 option B and the design-decision
  table's chunked-prefill entry).  Reading: a chunk of n new query tokens of a
  sequence with context length L sits at positions L-n .. L-1 and its row i
  sees keys 0 .. L-n+i (causal, aligned to the end of the context).
* The result itself is textbook attention, softmax(q K^T * scale) V with
  scale = 1/sqrt(head_dim), computed here in float64 over the gathered keys.
  There is no split-context path here: every GPU path must equal this one.

Every function below is parity-pinned by the CPU tests (dense-vs-paged,
physical-id permutation, closed forms, brute force on 1-3 tokens, GQA against
repeated-KV MHA, prefill reductions, write round trip, hand-derived golden
cases).
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact decode of stored values to float64.

    bf16 arrives as uint16 bit patterns: placing them in the top half of an
    fp32 word gives the same number exactly.  fp16 and fp32 widen exactly."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def kv_write(k_pool, v_pool, new_k, new_v, slot_mapping):
    """Return copies of the pools with each new token's K/V rows stored.

    Token t goes to block slot // B, offset slot % B for a pool of B-token
    blocks (B = 16 unless the pool says otherwise); slot < 0 is skipped.  Bits
    are copied unchanged (no arithmetic)."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    bsz = k_pool.shape[1]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(slot, bsz)
        k_out[block, offset] = new_k[t]
        v_out[block, offset] = new_v[t]
    return k_out, v_out


def gather(pool, table_row, n_tokens):
    """Logical token j of a sequence lives at pool[table_row[j // B], j % B],
    B the pool's block size (16 by default)."""
    bsz = pool.shape[1]
    phys = [int(table_row[j // bsz]) for j in range(n_tokens)]
    offs = [j % bsz for j in range(n_tokens)]
    return pool[phys, offs] if n_tokens else pool[:0, 0]


def softmax_attention(q, keys, values, scale):
    """Textbook attention for one query vector over one key/value list.

    q [D], keys [n, D], values [n, D], all float64.  n == 0 gives zeros."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    scores = (keys @ q) * scale
    scores = scores - scores.max()
    weights = np.exp(scores)
    weights = weights / weights.sum()
    return weights @ values


def attention(q, query_start_loc, k_pool, v_pool, block_tables, context_lens,
              scale, dtype):
    """Causal attention of every query row over its sequence's paged context.

    q [T, Hq, D] (rows of sequence s are query_start_loc[s] .. [s+1]-1);
    pools [NB, 16, Hkv, D]; returns float64 [T, Hq, D].  A decode step is the
    special case of one query row per sequence."""
    qf = to_f64(q, dtype)
    T, Hq, D = qf.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = Hq // Hkv
    out = np.zeros((T, Hq, D), dtype=np.float64)
    qsl = np.asarray(query_start_loc).tolist()
    for s, L in enumerate(np.asarray(context_lens).tolist()):
        rows = range(qsl[s], qsl[s + 1])
        n = len(rows)
        K = to_f64(gather(k_pool, block_tables[s], L), dtype)   # [L, Hkv, D]
        V = to_f64(gather(v_pool, block_tables[s], L), dtype)
        for i, r in enumerate(rows):
            visible = L - n + i + 1                 # keys 0 .. L-n+i
            for h in range(Hq):
                g = h // group
                out[r, h] = softmax_attention(qf[r, h], K[:visible, g], V[:visible, g], scale)
    return out


def decode(q, k_pool, v_pool, block_tables, context_lens, scale, dtype):
    """Batched decode: one query row per sequence, q [S, Hq, D]."""
    S = len(context_lens)
    qsl = np.arange(S + 1)
    return attention(q, qsl, k_pool, v_pool, block_tables, context_lens, scale, dtype)
