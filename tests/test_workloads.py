"""The seeded generator: bf16 rounding, layout and poisoning invariants."""
import numpy as np
import torch

from workloads import (BLOCK, f32_to_bf16_bits, long_context, mixed_prefill,
                       qwen25_05b_decode, qwen3_06b_decode, tiny_f32)


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        # exact ties (low 16 bits 0x8000) with even and odd kept halves
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00018000, 0x7F7F8000],
                 np.uint32).view(np.float32),
        np.array([0.0, -0.0, 1.0, -2.5, 65504.0], np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), want)


def is_nan(a, dtype):
    if dtype == "bf16":
        return ((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)
    return np.isnan(a)


def check_layout(b):
    NB, Hkv, D = b.num_blocks, b.num_kv_heads, b.head_dim
    assert b.k_pool.shape == (NB, BLOCK, Hkv, D) and b.v_pool.shape == b.k_pool.shape
    assert b.q.shape == (b.total_query_tokens, b.num_q_heads, D)
    assert b.block_tables.dtype == np.int32 and b.block_tables.min() >= 0
    assert b.block_tables.max() < NB
    nk = b.new_k.shape[0]
    assert b.slot_mapping.shape == (nk,)
    assert np.array_equal(np.diff(b.query_start_loc), b.query_lens)
    k_rows = b.k_pool.reshape(NB * BLOCK, Hkv, D)
    used = set()
    for s, L in enumerate(b.context_lens.tolist()):
        n = int(b.query_lens[s])
        nblk = -(-L // BLOCK)
        for j in range(L):
            row = int(b.block_tables[s, j // BLOCK]) * BLOCK + j % BLOCK
            nan = is_nan(k_rows[row], b.dtype)
            if j < L - n:
                assert not nan.any()          # history is present
            else:
                assert nan.all()              # to be filled by this step's write
                t = int(b.query_start_loc[s]) + j - (L - n)
                assert b.slot_mapping[t] == row
        if L:
            last = int(b.block_tables[s, nblk - 1])
            assert is_nan(b.k_pool[last, (L - 1) % BLOCK + 1:], b.dtype).all()
        used.update(b.block_tables[s, :nblk].tolist())
    unused = sorted(set(range(NB)) - used)
    assert is_nan(b.k_pool[unused], b.dtype).all() and is_nan(b.v_pool[unused], b.dtype).all()
    # distinct slots among the real new tokens
    real = b.slot_mapping[b.slot_mapping >= 0]
    assert len(np.unique(real)) == len(real)


def test_tiny_layout():
    b = tiny_f32()
    assert b.context_lens.tolist() == [5, 17, 33, 64] and b.num_blocks == 32
    assert b.dtype == "f32" and b.k_pool.dtype == np.float32
    check_layout(b)


def test_small_variants_layout():
    check_layout(qwen25_05b_decode(batch=7, lo=1, hi=90))
    check_layout(qwen3_06b_decode(batch=5, prompt=(1, 50), gen=(0, 40)))
    b = mixed_prefill(chunks=2, chunk_len=20, prior_hi=33, n_decode=5, dec_lo=1, dec_hi=60)
    check_layout(b)
    assert b.num_prefill_seqs == 2 and b.query_lens.tolist()[:2] == [20, 20]
    b = long_context(batch=3, ctx=100, shared_blocks=3)
    check_layout(b)
    assert (b.block_tables[:, :3] == b.block_tables[0, :3]).all()
    assert len(np.unique(b.block_tables[:, 3:])) == b.block_tables[:, 3:].size


def test_seeded_and_reproducible():
    a = qwen25_05b_decode(batch=4, lo=10, hi=40)
    b = qwen25_05b_decode(batch=4, lo=10, hi=40)
    for f in ("context_lens", "block_tables", "k_pool", "v_pool", "q", "new_k", "slot_mapping"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
