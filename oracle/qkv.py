"""Plain fp64 CPU oracle for the fused QKV split + RoPE + KV-cache write.

TEST INFRASTRUCTURE, like the rest of this package: only the test suite, the
package's smoke check and the benchmark's CPU-baseline leg may use it.

What it follows:

* The model packs the Q, K and V projections into one GEMM ("mini_engine",
  What it does), so each token arrives as one row [q heads | k heads | v heads].
* The fusion target "QKV split and KV-cache write" together with "Fused RoPE"
  ("mini_engine", Next: fused kernels), and the GPU-side slot derivation of
  "mini-vllm", Milestones item 7: the slot of a token is found on the device
  from its sequence's block table and its position, instead of being handed in.
* Qwen3 applies RMSNorm and RoPE ("mini_engine", What it does lists both for the
  decoder); the pages fix neither the rotary convention nor where the norms sit.
  Readings taken (each stated where it is used below): rotary embedding with the
  rotate-half pairing over the whole head (dims i and i + D/2 form a pair,
  inverse frequency theta ** (-2i / D)), the convention of the Qwen model
  family; optional per-head RMSNorm of q and k before the rotation (Qwen3's
  q/k norms), absent when no weights are given.
* Positions follow the attention call's causal alignment: token i of a
  sequence with n new tokens and context length L (which counts the new
  tokens, write first then attend) sits at position L - n + i.

Pinned by tests/test_oracle_qkv.py: the rotation against the rotary embedding
of the `transformers` Qwen2 model (a library routine), norm preservation,
identity at position 0, the relative-position property of rotated dot
products, RMSNorm against torch's float64 rms_norm, slot derivation against
the input generator's independently computed slot mapping and a write/gather
round trip, and planted mistakes.
"""
from __future__ import annotations

import numpy as np

from .ref import BLOCK_SIZE, to_f64  # noqa: F401  (BLOCK_SIZE: the default block size)


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * weight over the last axis (float64)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(weight, np.float64)


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half pairing (reading: the Qwen convention).

    x: [T, H, D] float64; positions: [T].  Pair (i, i + D/2) of every head of
    token t turns by the angle positions[t] * theta ** (-2i / D)."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(positions, np.float64)[:, None] * inv_freq[None, :]   # [T, D/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def token_positions(query_start_loc, context_lens, num_tokens):
    """(sequence, position) of every token.  query_start_loc None means one
    token per sequence (token t is sequence t)."""
    seq = np.zeros(num_tokens, np.int64)
    pos = np.zeros(num_tokens, np.int64)
    if query_start_loc is None:
        for t in range(num_tokens):
            seq[t], pos[t] = t, int(context_lens[t]) - 1
        return seq, pos
    for s in range(len(query_start_loc) - 1):
        lo, hi = int(query_start_loc[s]), int(query_start_loc[s + 1])
        n, L = hi - lo, int(context_lens[s])
        for i in range(n):
            seq[lo + i], pos[lo + i] = s, L - n + i
    return seq, pos


def derive_slots(query_start_loc, context_lens, block_tables, num_tokens, num_blocks,
                 block_size=BLOCK_SIZE):
    """Flat pool slot of every token: table[seq][pos // B] * B + pos % B for
    B-token blocks.  A position outside the table, or a table entry outside
    the pool, gives -1 (nothing is written for that token)."""
    seq, pos = token_positions(query_start_loc, context_lens, num_tokens)
    slots = np.full(num_tokens, -1, np.int64)
    width = block_tables.shape[1]
    for t in range(num_tokens):
        p = int(pos[t])
        if p < 0 or p >= width * block_size:
            continue
        blk = int(block_tables[seq[t], p // block_size])
        if 0 <= blk < num_blocks:
            slots[t] = blk * block_size + p % block_size
    return slots


def to_stored(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the stored element type: fp32 or fp16 (nearest
    even), or bf16 bit patterns (fp32 first, then the upper 16 bits with
    nearest-even rounding of the lower 16)."""
    if dtype == "f16":
        return np.asarray(x, np.float64).astype(np.float16)   # nearest even
    f = np.asarray(x, np.float64).astype(np.float32)
    if dtype == "f32":
        return f
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    nan = np.isnan(f)
    r = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r)   # keep NaN a (quiet) NaN
    return r.astype(np.uint16)


def qkv_rope_write(qkv, query_start_loc, context_lens, block_tables, k_pool, v_pool,
                   num_q_heads, num_kv_heads, theta, dtype, q_norm=None, k_norm=None,
                   eps=1e-6):
    """Split the packed rows, (norm,) rotate q and k, and store k and v.

    qkv: [T, >= (Hq + 2*Hkv) * D] stored values.  Returns (q_out float64
    [T, Hq, D], k_pool', v_pool' (copies, stored type), slots [T], k_rot
    float64 [T, Hkv, D]).  The K row stored is k_rot rounded to the stored
    type; the V row is the input's bits unchanged."""
    d = k_pool.shape[-1]
    T = qkv.shape[0]
    hq, hkv = num_q_heads, num_kv_heads
    x = qkv[:, :(hq + 2 * hkv) * d]
    q = to_f64(x[:, :hq * d], dtype).reshape(T, hq, d)
    k = to_f64(x[:, hq * d:(hq + hkv) * d], dtype).reshape(T, hkv, d)
    v_bits = x[:, (hq + hkv) * d:].reshape(T, hkv, d)
    if q_norm is not None:
        q = rms_norm(q, to_f64(q_norm, dtype), eps)
    if k_norm is not None:
        k = rms_norm(k, to_f64(k_norm, dtype), eps)
    _, pos = token_positions(query_start_loc, context_lens, T)
    q_out = rope(q, pos, theta)
    k_rot = rope(k, pos, theta)
    slots = derive_slots(query_start_loc, context_lens, block_tables, T, k_pool.shape[0], k_pool.shape[1])
    kp, vp = k_pool.copy(), v_pool.copy()
    krow, vrow = kp.reshape(-1, hkv, d), vp.reshape(-1, hkv, d)
    k_store = to_stored(k_rot, dtype)
    for t in range(T):
        if slots[t] >= 0:
            krow[slots[t]] = k_store[t]
            vrow[slots[t]] = v_bits[t]
    return q_out, kp, vp, slots, k_rot
