"""Pools of 8- and 32-token blocks on the GPU.

The kernels walk a sequence in 16-token chunks whatever the pool's block size
(a chunk is two blocks of 8, or half a block of 32), so:

* every path (vector and matrix-core decode, both launch shapes of the chunk
  kernel, the KV write and the fused QKV write) matches the fp64 oracle on
  batches drawn natively at block sizes 8 and 32, poison (NaN) past every
  length and in every unused block included;
* the same logical K/V content laid out at block sizes 8, 16 and 32 gives
  bit-identical attention outputs (the same arithmetic in the same order; only
  the addresses differ)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from helpers import DeviceBatch, assert_close, bits, dev, ensure_built, f64
from workloads import make_batch, mixed_prefill, packed_qkv, qwen25_05b_decode, qwen3_06b_decode

pytestmark = pytest.mark.gpu

SIZES = [8, 32]


@pytest.fixture(scope="module")
def pa():
    ensure_built()
    import paged_kv_attention_22_amd as m
    return m


DECODE = {
    # vector path: G = 2 at head_dim 128, G = 3 at head_dim 64, fp32 (4 elements a lane)
    "qwen3": lambda bs: qwen3_06b_decode(batch=19, prompt=(1, 400), gen=(0, 300), block_size=bs),
    "g3_d64": lambda bs: make_batch(71, name="g3_d64", dtype="bf16", num_q_heads=6, num_kv_heads=2,
                                    head_dim=64, block_size=bs,
                                    draw_lens=lambda rng: rng.integers(1, 700, size=13)),
    "f32": lambda bs: make_batch(72, name="f32_g2", dtype="f32", num_q_heads=4, num_kv_heads=2,
                                 head_dim=128, block_size=bs,
                                 draw_lens=lambda rng: rng.integers(1, 300, size=7)),
    # matrix-core path: G = 7 at head_dim 64, G = 4 at head_dim 128 (bf16 and fp16)
    "qwen25": lambda bs: qwen25_05b_decode(batch=15, lo=1, hi=800, block_size=bs),
    "g4_d128": lambda bs: make_batch(73, name="g4_d128", dtype="bf16", num_q_heads=16, num_kv_heads=4,
                                     head_dim=128, block_size=bs,
                                     draw_lens=lambda rng: rng.integers(1, 700, size=17)),
    "g4_d128_f16": lambda bs: make_batch(74, name="g4_d128_f16", dtype="f16", num_q_heads=16,
                                         num_kv_heads=4, head_dim=128, block_size=bs,
                                         draw_lens=lambda rng: rng.integers(1, 700, size=17)),
}

PREFILL = {
    # small launch (key halves), with vector-path chunks of 3 and 7 rows
    "mixed_small": lambda bs: mixed_prefill(seed=81, chunk_lens=[3, 40, 7, 61], prior_hi=300, n_decode=6,
                                            dec_lo=1, dec_hi=400, block_size=bs),
    "mixed_d64": lambda bs: mixed_prefill(seed=82, chunks=3, chunk_len=50, prior_hi=200, n_decode=5,
                                          dec_lo=1, dec_hi=600, num_q_heads=14, num_kv_heads=2, head_dim=64,
                                          block_size=bs),
    # large launch (two row tiles per wave)
    "mixed_large": lambda bs: mixed_prefill(seed=83, chunks=4, chunk_len=300, prior_hi=600, n_decode=10,
                                            dec_lo=1, dec_hi=900, block_size=bs),
    "mixed_f16": lambda bs: mixed_prefill(seed=84, chunks=3, chunk_len=45, prior_hi=250, n_decode=4,
                                          dec_lo=1, dec_hi=500, dtype="f16", block_size=bs),
}


def raw(a):
    """Stored values as raw bits (fp32 as uint32, fp16 and bf16 as uint16)."""
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def write_and_check(pa, b, d):
    """pa_kv_write into the device pools; the pools must equal the oracle's write bit for bit."""
    kp, vp = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    pa.kv_write(d.new_k, d.new_v, d.slot_mapping, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    assert np.array_equal(bits(d.k_pool), raw(kp)) and np.array_equal(bits(d.v_pool), raw(vp))
    return kp, vp


@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("name", list(DECODE))
def test_decode_matches_oracle(pa, name, bs):
    b = DECODE[name](bs)
    assert b.k_pool.shape[1] == bs
    d = DeviceBatch(b)
    kp, vp = write_and_check(pa, b, d)
    ref = oracle.decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
    for part in [-1, 0, 16, 64]:
        print(f"[block size {bs}] decode {name} B={b.num_seqs} part={part}", flush=True)
        out = pa.decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.max_context_len,
                        scale=b.scale, partition_tokens=part)
        torch.cuda.synchronize()
        assert_close(f64(out), ref, b.dtype, f"{name} bs={bs} part={part}")


@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_matches_oracle(pa, name, bs):
    b = PREFILL[name](bs)
    d = DeviceBatch(b)
    kp, vp = write_and_check(pa, b, d)
    ref = oracle.attention(b.q, b.query_start_loc, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
    for part in [0, 64]:
        print(f"[block size {bs}] prefill {name} T={b.total_query_tokens} part={part}", flush=True)
        out = pa.prefill_chunk(d.q, d.query_start_loc, b.num_prefill_seqs, b.max_query_len, d.k_pool,
                               d.v_pool, d.block_tables, d.context_lens, b.max_context_len, scale=b.scale,
                               partition_tokens=part)
        torch.cuda.synchronize()
        assert_close(f64(out), ref, b.dtype, f"{name} bs={bs} part={part}")


@pytest.mark.parametrize("bs", SIZES)
def test_fused_qkv_write(pa, bs):
    """Slots derived on the device from 8- or 32-token tables, rows written there."""
    for b in [qwen3_06b_decode(batch=12, prompt=(1, 200), gen=(0, 100), block_size=bs),
              mixed_prefill(seed=85, chunks=2, chunk_len=37, prior_hi=90, n_decode=5, dec_lo=1, dec_hi=200,
                            block_size=bs)]:
        T = b.q.shape[0]
        qsl = b.query_start_loc if b.num_prefill_seqs else None
        x = packed_qkv(b)
        print(f"[block size {bs}] fused write {b.name} T={T}", flush=True)
        _, kp_ref, vp_ref, slots_ref, _ = oracle.qkv_rope_write(
            x, qsl, b.context_lens, b.block_tables, b.k_pool, b.v_pool, b.num_q_heads, b.num_kv_heads,
            1e6, b.dtype)
        assert np.array_equal(slots_ref, b.slot_mapping[:T].astype(np.int64))
        kp, vp = dev(b.k_pool), dev(b.v_pool)
        so = torch.full((T,), -7, dtype=torch.int32, device="cuda")
        pa.qkv_rope_write(dev(x), b.num_q_heads, dev(b.context_lens), dev(b.block_tables), kp, vp, 1e6,
                          query_start_loc=None if qsl is None else dev(qsl), slot_mapping_out=so)
        torch.cuda.synchronize()
        assert np.array_equal(so.cpu().numpy(), slots_ref.astype(np.int32))
        hkv, dd = b.num_kv_heads, b.head_dim
        vrow = bits(vp).reshape(-1, hkv, dd)
        assert np.array_equal(vrow, raw(vp_ref).reshape(-1, hkv, dd))  # V rows copied bit for bit
        written = np.zeros(vrow.shape[0], bool)
        written[slots_ref] = True
        krow = bits(kp).reshape(-1, hkv, dd)
        assert np.array_equal(krow[~written], raw(kp_ref).reshape(-1, hkv, dd)[~written])


# --- the same content at three block sizes ------------------------------------

def relayout(b, kp, vp, bs, seed):
    """The batch's written pools re-laid at `bs` tokens per block: each
    sequence's logical tokens 0..L-1 copied into freshly permuted blocks, NaN
    everywhere else."""
    rng = np.random.default_rng(seed)
    S = b.num_seqs
    lens = b.context_lens.astype(np.int64)
    nblk = -(-lens // bs)
    nb = int(nblk.sum()) + 3
    perm = rng.permutation(nb)
    width = max(int(nblk.max()), 1)
    tables = np.full((S, width), perm[-1], np.int64)
    poison = np.float32("nan") if b.dtype == "f32" else (np.uint16(0x7FC0) if b.dtype == "bf16"
                                                          else np.float16("nan"))
    shape = (nb, bs) + kp.shape[2:]
    k2, v2 = np.full(shape, poison, kp.dtype), np.full(shape, poison, vp.dtype)
    cur = 0
    for s in range(S):
        n = int(nblk[s])
        tables[s, :n] = perm[cur:cur + n]
        cur += n
        L = int(lens[s])
        src_k = oracle.gather(kp, b.block_tables[s], L)
        src_v = oracle.gather(vp, b.block_tables[s], L)
        j = np.arange(L)
        k2[tables[s, j // bs], j % bs] = src_k
        v2[tables[s, j // bs], j % bs] = src_v
    return dataclasses.replace(b, k_pool=k2, v_pool=v2, block_tables=tables.astype(np.int32))


@pytest.mark.parametrize("kind", ["decode_vector", "decode_mfma", "prefill"])
def test_layouts_agree_bitwise(pa, kind):
    if kind == "decode_vector":
        b = qwen3_06b_decode(batch=23, prompt=(1, 500), gen=(0, 300))
    elif kind == "decode_mfma":
        b = qwen25_05b_decode(batch=21, lo=1, hi=900)
    else:
        b = mixed_prefill(seed=86, chunk_lens=[5, 70, 200], prior_hi=300, n_decode=7, dec_lo=1, dec_hi=600)
    kp, vp = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    base = dataclasses.replace(b, k_pool=kp, v_pool=vp)
    outs, o16 = {}, None
    for bs in [16, 8, 32]:
        lb = base if bs == 16 else relayout(b, kp, vp, bs, seed=bs)
        d = DeviceBatch(lb)
        for part in [-1, 64]:
            print(f"[layouts] {kind} block size {bs} part={part}", flush=True)
            if kind == "prefill":
                o = pa.prefill_chunk(d.q, d.query_start_loc, lb.num_prefill_seqs, lb.max_query_len, d.k_pool,
                                     d.v_pool, d.block_tables, d.context_lens, lb.max_context_len,
                                     scale=lb.scale, partition_tokens=part)
            else:
                o = pa.decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, lb.max_context_len,
                              scale=lb.scale, partition_tokens=part)
            torch.cuda.synchronize()
            outs[(bs, part)] = bits(o)
            if (bs, part) == (16, -1):
                o16 = f64(o)
    for part in [-1, 64]:
        assert np.array_equal(outs[(8, part)], outs[(16, part)]), f"{kind} part={part}: 8 vs 16"
        assert np.array_equal(outs[(32, part)], outs[(16, part)]), f"{kind} part={part}: 32 vs 16"
    ref = oracle.attention(b.q, b.query_start_loc, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
    assert_close(o16, ref, b.dtype, f"{kind} vs oracle")
