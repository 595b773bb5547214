"""pa_kv_write on the GPU: whole pools bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from helpers import DeviceBatch, bits, dev, ensure_built
from workloads import (long_context, mixed_prefill, qwen25_05b_decode, qwen3_06b_decode,
                       tiny_f32, make_batch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    ensure_built()
    import paged_kv_attention_22_amd as m
    return m


CASES = {
    "tiny_f32": tiny_f32,
    "qwen25_small": lambda: qwen25_05b_decode(batch=9, lo=1, hi=200),
    "qwen3_full": qwen3_06b_decode,
    "mixed_full": mixed_prefill,
    "long_small": lambda: long_context(batch=4, ctx=1000, shared_blocks=20),
    "qwen3_f16": lambda: qwen3_06b_decode(batch=30, prompt=(1, 300), gen=(0, 100), dtype="f16"),
    "mixed_f16": lambda: mixed_prefill(chunks=2, chunk_len=50, prior_hi=100, n_decode=6, dtype="f16"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_kv_write_bit_exact(pa, name):
    b = CASES[name]()
    print(f"[kv_write] {name} T={b.new_k.shape[0]} pool={b.k_pool.shape}", flush=True)
    d = DeviceBatch(b)
    pa.kv_write(d.new_k, d.new_v, d.slot_mapping, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    assert np.array_equal(bits(d.k_pool), k_ref.view(bits(d.k_pool).dtype))
    assert np.array_equal(bits(d.v_pool), v_ref.view(bits(d.v_pool).dtype))


def test_kv_write_padding_slots_and_strided_rows(pa):
    """Slots of -1 are skipped; k/v may be views into a packed QKV buffer."""
    b = make_batch(31, name="pad", dtype="bf16", num_q_heads=16, num_kv_heads=8, head_dim=128,
                   draw_lens=lambda rng: rng.integers(1, 90, size=7), pad_slots=5)
    assert (b.slot_mapping[-5:] == -1).all()
    d = DeviceBatch(b)
    T, hq, hkv, D = b.new_k.shape[0], 16, 8, 128
    qkv = torch.zeros(T, (hq + 2 * hkv) * D, dtype=torch.bfloat16, device="cuda")
    qkv[:, hq * D:(hq + hkv) * D] = d.new_k.reshape(T, -1)
    qkv[:, (hq + hkv) * D:] = d.new_v.reshape(T, -1)
    k_view = qkv[:, hq * D:(hq + hkv) * D].view(T, hkv, D)
    v_view = qkv[:, (hq + hkv) * D:].view(T, hkv, D)
    assert k_view.stride(0) == (hq + 2 * hkv) * D
    pa.kv_write(k_view, v_view, d.slot_mapping, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    assert np.array_equal(bits(d.k_pool), k_ref)
    assert np.array_equal(bits(d.v_pool), v_ref)


def test_kv_write_rejects_and_leaves_pool(pa):
    b = tiny_f32()
    d = DeviceBatch(b)
    before = bits(d.k_pool).copy()
    buf = torch.zeros(d.new_k.numel() + 4, dtype=d.new_k.dtype, device="cuda")
    bad = buf[1:1 + d.new_k.numel()].view(d.new_k.shape)    # 4 bytes off 16-byte alignment
    with pytest.raises(pa.PAError) as e:
        pa.kv_write(bad, d.new_v, d.slot_mapping, d.k_pool, d.v_pool)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert np.array_equal(bits(d.k_pool), before)


def test_kv_write_out_of_range_slots_skipped(pa):
    """Slots past the pool are skipped (documented memory-safety clamp)."""
    b = tiny_f32()
    d = DeviceBatch(b)
    slots = b.slot_mapping.copy()
    slots[1] = b.num_blocks * 16 + 5
    pa.kv_write(d.new_k, d.new_v, dev(slots), d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    s2 = slots.copy()
    s2[1] = -1
    k_ref, _ = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, s2)
    assert np.array_equal(bits(d.k_pool), k_ref.view(np.uint32))
