"""CPU pins of the fused QKV split + RoPE + KV write oracle (oracle/qkv.py).

Each pin is something other than the oracle's own formula: the rotary
embedding of the `transformers` Qwen2 model, torch's float64 rms_norm,
properties every rotation has (norm preservation, identity at position 0,
dot products depending on relative position only), the input generator's
independently computed slot mapping and a write/gather round trip.  The
planted mistakes at the end each fail at least one pin."""
import numpy as np
import pytest
import torch

import oracle
from workloads import mixed_prefill, norm_weights, packed_qkv, qwen25_05b_decode

RNG = np.random.default_rng(1234)


def hf_rope(x, positions, theta):
    """transformers' Qwen2 rotary embedding applied to x [T, H, D] (float64)."""
    from transformers import Qwen2Config
    from transformers.models.qwen2 import modeling_qwen2 as m
    T, H, D = x.shape
    cfg = Qwen2Config(hidden_size=H * D, num_attention_heads=H, num_key_value_heads=H, head_dim=D,
                      rope_theta=theta)
    rot = m.Qwen2RotaryEmbedding(cfg)
    xt = torch.from_numpy(x).permute(1, 0, 2)[None]            # [1, H, T, D]
    cos, sin = rot(xt, torch.from_numpy(np.asarray(positions))[None])
    q, _ = m.apply_rotary_pos_emb(xt, xt, cos, sin)
    return q[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("D,theta", [(128, 1e6), (64, 1e4), (128, 1e4)])
def test_rope_matches_transformers_qwen(D, theta):
    x = RNG.standard_normal((40, 3, D))
    pos = RNG.integers(0, 64, size=40)
    want = hf_rope(x, pos, theta)
    got = oracle.rope(x, pos, theta)
    # transformers builds the inverse frequencies in float32: angles differ
    # by ~pos * 1e-7 at most
    assert np.abs(got - want).max() <= 2e-5 * np.abs(x).max()


def test_rope_properties():
    D = 128
    x = RNG.standard_normal((50, 4, D))
    pos = RNG.integers(0, 4096, size=50)
    y = oracle.rope(x, pos, 1e6)
    # each pair (i, i + D/2) keeps its length
    n0 = x[..., :D // 2] ** 2 + x[..., D // 2:] ** 2
    n1 = y[..., :D // 2] ** 2 + y[..., D // 2:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=1e-12)
    # position 0 is the identity
    assert np.array_equal(oracle.rope(x, np.zeros(50, np.int64), 1e6), x)
    # <rope(q, m), rope(k, n)> depends on m - n only
    q, k = RNG.standard_normal((1, 1, D)), RNG.standard_normal((1, 1, D))
    for m_, n_, d_ in [(5, 2, 100), (0, 17, 1000), (300, 300, 7)]:
        a = np.sum(oracle.rope(q, [m_], 1e4) * oracle.rope(k, [n_], 1e4))
        b = np.sum(oracle.rope(q, [m_ + d_], 1e4) * oracle.rope(k, [n_ + d_], 1e4))
        assert abs(a - b) <= 1e-9 * (1 + abs(a))
    # a quarter turn at the first pair: theta ** 0 = 1, so position p turns pair 0 by p radians
    e = np.zeros((1, 1, D))
    e[0, 0, 0] = 1.0
    y = oracle.rope(e, [3], 1e6)
    assert np.isclose(y[0, 0, 0], np.cos(3.0)) and np.isclose(y[0, 0, D // 2], np.sin(3.0))


def test_rms_norm_matches_torch():
    x = RNG.standard_normal((30, 5, 64))
    w = 1 + 0.1 * RNG.standard_normal(64)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-6).numpy()
    assert np.allclose(oracle.rms_norm(x, w, 1e-6), want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("make", [lambda: mixed_prefill(chunks=3, chunk_len=37, prior_hi=90, n_decode=5),
                                  lambda: qwen25_05b_decode(batch=6, lo=1, hi=70)])
def test_slots_equal_generator_slot_mapping(make):
    """The generator lays out every new token's slot from its own loop over the
    tables; the oracle derives it from (sequence, position)."""
    b = make()
    T = b.q.shape[0]
    qsl = b.query_start_loc if b.num_prefill_seqs else None
    slots = oracle.derive_slots(qsl, b.context_lens, b.block_tables, T, b.k_pool.shape[0])
    assert np.array_equal(slots, b.slot_mapping[:T].astype(np.int64))
    # positions: the chunk's last token is at L - 1
    _, pos = oracle.token_positions(qsl, b.context_lens, T)
    ends = (b.query_start_loc[1:] - 1) if qsl is not None else np.arange(T)
    assert np.array_equal(pos[ends], b.context_lens.astype(np.int64) - 1)


def test_slot_edge_cases():
    bt = np.array([[3, 1, 99], [2, 0, 0]], np.int32)       # 99: outside a 4-block pool
    lens = np.array([40, 16], np.int32)
    qsl = np.array([0, 3, 4], np.int32)                    # 3 tokens of seq 0, 1 of seq 1
    s = oracle.derive_slots(qsl, lens, bt, 4, 4)
    # seq 0 tokens at positions 37, 38, 39 -> block index 2 -> id 99 -> skipped
    assert s.tolist()[:3] == [-1, -1, -1]
    assert s[3] == 2 * 16 + 15
    # a position past the table is skipped too
    assert oracle.derive_slots(np.array([0, 1]), np.array([49]), bt[:1], 1, 4).tolist() == [-1]


def test_write_then_gather_round_trip():
    b = mixed_prefill(chunks=2, chunk_len=21, prior_hi=60, n_decode=4)
    x = packed_qkv(b, pad_cols=8)
    qn, kn = norm_weights(b, 5)
    T, hq, hkv, d = b.q.shape[0], b.num_q_heads, b.num_kv_heads, b.head_dim
    q_out, kp, vp, slots, k_rot = oracle.qkv_rope_write(
        x, b.query_start_loc, b.context_lens, b.block_tables, b.k_pool, b.v_pool, hq, hkv, 1e6,
        b.dtype, q_norm=qn, k_norm=kn)
    assert (slots >= 0).all()
    seq, pos = oracle.token_positions(b.query_start_loc, b.context_lens, T)
    for t in range(T):
        s, p = int(seq[t]), int(pos[t])
        kg = oracle.gather(kp, b.block_tables[s], p + 1)[p]
        vg = oracle.gather(vp, b.block_tables[s], p + 1)[p]
        assert np.array_equal(vg, x[t, (hq + hkv) * d:(hq + 2 * hkv) * d].reshape(hkv, d))
        assert np.array_equal(kg, oracle.to_stored(k_rot[t], b.dtype))
    # every other slot unchanged
    mask = np.ones(kp.shape[0] * 16, bool)
    mask[slots] = False
    assert np.array_equal(kp.reshape(-1, hkv, d)[mask], b.k_pool.reshape(-1, hkv, d)[mask])
    assert np.array_equal(vp.reshape(-1, hkv, d)[mask], b.v_pool.reshape(-1, hkv, d)[mask])
    # q: norm then rotation, checked with torch's rms_norm and transformers' rotary embedding
    qin = oracle.to_f64(x[:, :hq * d], b.dtype).reshape(T, hq, d)
    qnorm = torch.nn.functional.rms_norm(torch.from_numpy(qin), (d,),
                                         torch.from_numpy(oracle.to_f64(qn, b.dtype)), eps=1e-6).numpy()
    small = pos < 64
    assert np.abs(q_out[small] - hf_rope(qnorm[small], pos[small], 1e6)).max() <= 1e-4


def test_to_stored_rounds_to_nearest_even():
    # bf16 keeps 7 fraction bits: one unit in the last place at 1.0 is 2^-7
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 3 * 2 ** -8, -2.5, 0.0], np.float64)
    got = oracle.to_stored(x, "bf16")
    # half a unit: tie, to the even 1.0; 3/4 of a unit: up; 3/2 units: tie, to the even 2 units
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F81, 0x3F82, 0xC020, 0x0000]


def test_to_stored_f16_rounds_to_nearest_even():
    # fp16 keeps 10 fraction bits (one unit in the last place at 1.0 is 2^-10),
    # 5 exponent bits (largest finite 65504, smallest normal 2^-14) and
    # subnormals down to 2^-24; each expected pattern is worked out by hand.
    x = np.array([
        1.0 + 2 ** -11,             # half a unit: tie, to the even 1.0          -> 0x3C00
        1.0 + 3 * 2 ** -11,         # tie between 1+2^-10 (odd) and 1+2^-9: up   -> 0x3C02
        1.0 + 2 ** -11 + 2 ** -20,  # just past half a unit: up                  -> 0x3C01
        65504.0,                    # largest finite                             -> 0x7BFF
        65519.0,                    # below the midpoint 65520: down             -> 0x7BFF
        65520.0,                    # midpoint, 65504's last bit odd: to inf     -> 0x7C00
        2.0 ** -14,                 # smallest normal                            -> 0x0400
        2.0 ** -24,                 # smallest subnormal                         -> 0x0001
        2.0 ** -25,                 # half of it: tie, to the even 0             -> 0x0000
        3 * 2.0 ** -25,             # 1.5 subnormal units: tie, to the even 2    -> 0x0002
        -2.5,                       # sign, exponent 1, fraction 0.25            -> 0xC100
        0.0,
    ], np.float64)
    got = oracle.to_stored(x, "f16").view(np.uint16)
    assert got.tolist() == [0x3C00, 0x3C02, 0x3C01, 0x7BFF, 0x7BFF, 0x7C00, 0x0400, 0x0001, 0x0000,
                            0x0002, 0xC100, 0x0000]


# --- planted mistakes --------------------------------------------------------

def rope_interleaved(x, positions, theta):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    inv = float(theta) ** (-np.arange(d // 2) * 2.0 / d)
    a = np.asarray(positions, np.float64)[:, None] * inv
    c, s = np.cos(a)[:, None, :], np.sin(a)[:, None, :]
    x1, x2 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2], y[..., 1::2] = x1 * c - x2 * s, x2 * c + x1 * s
    return y


def rope_wrong_sign(x, positions, theta):
    return oracle.rope(x, -np.asarray(positions), theta)


def rope_wrong_freq(x, positions, theta):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = float(theta) ** (-np.arange(half) * 1.0 / d)
    a = np.asarray(positions, np.float64)[:, None] * inv
    c, s = np.cos(a)[:, None, :], np.sin(a)[:, None, :]
    return np.concatenate([x[..., :half] * c - x[..., half:] * s, x[..., half:] * c + x[..., :half] * s], -1)


@pytest.mark.parametrize("mutant", [rope_interleaved, rope_wrong_sign, rope_wrong_freq])
def test_planted_rope_mistakes_are_caught(mutant):
    x = RNG.standard_normal((20, 2, 64))
    pos = RNG.integers(1, 64, size=20)
    assert np.abs(mutant(x, pos, 1e4) - hf_rope(x, pos, 1e4)).max() > 1e-3


def test_planted_slot_mistake_is_caught():
    b = mixed_prefill(chunks=2, chunk_len=19, prior_hi=40, n_decode=3)
    T = b.q.shape[0]
    seq, pos = oracle.token_positions(b.query_start_loc, b.context_lens, T)
    off_by_one = np.array([b.block_tables[s, (p + 1) // 16] * 16 + (p + 1) % 16 for s, p in zip(seq, pos)])
    assert not np.array_equal(off_by_one, b.slot_mapping[:T])
