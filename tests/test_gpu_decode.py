"""pa_decode on the GPU against the fp64 oracle, plus exactness pins.

Every case writes the step's new tokens with pa_kv_write first, then attends
(context lengths include those tokens), exactly as the oracle does."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from helpers import DeviceBatch, assert_close, bits, dev, ensure_built, f64
from workloads import (f32_to_bf16_bits, long_context, make_batch, qwen25_05b_decode,
                       qwen3_06b_decode, tiny_f32)

pytestmark = pytest.mark.gpu

PARTS = [-1, 0, 16, 64, 256]


@pytest.fixture(scope="module")
def pa():
    ensure_built()
    import paged_kv_attention_22_amd as m
    return m


WORKLOADS = {
    "tiny_f32": tiny_f32,
    "qwen25_small": lambda: qwen25_05b_decode(batch=11, lo=1, hi=300),
    "qwen25_full": qwen25_05b_decode,
    "qwen3_small": lambda: qwen3_06b_decode(batch=13, prompt=(1, 300), gen=(0, 200)),
    "qwen3_full": qwen3_06b_decode,
    "long_small": lambda: long_context(batch=3, ctx=1500, shared_blocks=40),
    "long_full": long_context,
    # the matrix-core decode path (bf16, group >= 4) at both head dims
    "g4_d128": lambda: make_batch(61, name="g4_d128", dtype="bf16", num_q_heads=16, num_kv_heads=4,
                                  head_dim=128, draw_lens=lambda rng: rng.integers(1, 700, size=21)),
    "g8_d64": lambda: make_batch(62, name="g8_d64", dtype="bf16", num_q_heads=16, num_kv_heads=2,
                                 head_dim=64, draw_lens=lambda rng: rng.integers(1, 900, size=19)),
    # more than 256 rows at G = 7 in one pass: the matrix-core decode's
    # eight-wave workgroups rank the lengths themselves (threads past the
    # first 256 hold no items)
    "g7_d128_ranked": lambda: make_batch(65, name="g7_d128_ranked", dtype="bf16", num_q_heads=28,
                                         num_kv_heads=4, head_dim=128,
                                         draw_lens=lambda rng: rng.integers(1, 260, size=300)),
    "g5_d128_f32": lambda: make_batch(63, name="g5_d128_f32", dtype="f32", num_q_heads=10,
                                      num_kv_heads=2, head_dim=128,
                                      draw_lens=lambda rng: rng.integers(1, 300, size=6)),
    # fp16 pools: the vector path (G = 2) and the matrix-core path (G = 7, G = 4)
    "qwen3_f16": lambda: qwen3_06b_decode(batch=40, prompt=(1, 600), gen=(0, 400), dtype="f16"),
    "qwen25_f16": lambda: qwen25_05b_decode(batch=17, lo=1, hi=900, dtype="f16"),
    "g4_d128_f16": lambda: make_batch(64, name="g4_d128_f16", dtype="f16", num_q_heads=16, num_kv_heads=4,
                                      head_dim=128, draw_lens=lambda rng: rng.integers(1, 700, size=21)),
    # the group sizes no other case takes: 1 (plain multi-head attention) and
    # 3 on the vector path, 6 on the matrix-core path (fp16)
    "g1_d128": lambda: make_batch(66, name="g1_d128", dtype="bf16", num_q_heads=8, num_kv_heads=8,
                                  head_dim=128, draw_lens=lambda rng: rng.integers(1, 800, size=12)),
    "g3_d64": lambda: make_batch(67, name="g3_d64", dtype="bf16", num_q_heads=12, num_kv_heads=4,
                                 head_dim=64, draw_lens=lambda rng: rng.integers(1, 900, size=15)),
    "g6_d128_f16": lambda: make_batch(68, name="g6_d128_f16", dtype="f16", num_q_heads=24, num_kv_heads=4,
                                      head_dim=128, draw_lens=lambda rng: rng.integers(1, 1200, size=9)),
    # one sequence of 65,536 tokens: the library splits it into 1,024-token
    # partitions, and 16-token partitions give 4,096 partial states per row
    # for the merge
    "one_64k": lambda: make_batch(69, name="one_64k", dtype="bf16", num_q_heads=28, num_kv_heads=4,
                                  head_dim=128, draw_lens=lambda rng: np.array([65536]), pool_factor=1.05),
}

_cache = {}


def prepared(name):
    """(batch, oracle output) with the KV write applied; cached per module."""
    if name not in _cache:
        b = WORKLOADS[name]()
        kp, vp = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
        ref = oracle.decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
        _cache[name] = (b, ref)
    return _cache[name]


def run_decode(pa, d, b, part, out=None):
    pa.kv_write(d.new_k, d.new_v, d.slot_mapping, d.k_pool, d.v_pool)
    o = pa.decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.max_context_len,
                  scale=b.scale, out=out, partition_tokens=part)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_decode_matches_oracle(pa, name):
    b, ref = prepared(name)
    d = DeviceBatch(b)
    for part in PARTS:
        print(f"[decode] {name} B={b.num_seqs} Hq={b.num_q_heads} Hkv={b.num_kv_heads} "
              f"D={b.head_dim} part={part}", flush=True)
        d.k_pool.copy_(dev(b.k_pool))  # fresh pools: the write must happen in this call
        d.v_pool.copy_(dev(b.v_pool))
        out = run_decode(pa, d, b, part)
        assert_close(f64(out), ref, b.dtype, f"{name} part={part}")


def test_split_sizes_agree(pa):
    """Split-size invariance: one pass and every partition size agree to the
    tolerance (and each agrees with the oracle above)."""
    b, ref = prepared("qwen3_small")
    d = DeviceBatch(b)
    outs = {p: f64(run_decode(pa, d, b, p)) for p in [-1, 16, 32, 48, 128, 512]}
    for p, o in outs.items():
        assert_close(o, outs[-1], b.dtype, f"part {p} vs one pass")


def needle_batch(D, hq, hkv, lens, seed):
    """K rows are zero in dim 0 except one needle token per (seq, kv head)
    whose dim 0 is c; q = c * e0.  With c*c*scale >= 128 every other weight is
    below 2^-180 and vanishes in fp32, so the output is the needle's V row
    exactly.  V rows are distinct values in [1, 2)."""
    b = make_batch(seed, name="needle", dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                   head_dim=D, draw_lens=lambda rng: np.array(lens))
    rng = np.random.default_rng(seed + 100)
    c = 64.0
    k_rows = b.k_pool.reshape(-1, hkv, D)
    v_rows = b.v_pool.reshape(-1, hkv, D)
    new_k = b.new_k.copy()
    new_v = b.new_v.copy()
    needles = np.zeros((len(lens), hkv), np.int64)
    for s, L in enumerate(lens):
        for g in range(hkv):
            needles[s, g] = rng.integers(0, L)
        for j in range(L):
            row = b.block_tables[s, j // 16] * 16 + j % 16
            is_new = j == L - 1
            kk = new_k[s] if is_new else k_rows[row]
            vv = new_v[s] if is_new else v_rows[row]
            for g in range(hkv):
                kk[g, 0] = f32_to_bf16_bits(np.array([c if j == needles[s, g] else 0.0]))[0]
                vv[g] = f32_to_bf16_bits((1 + rng.random(D)).astype(np.float32))
    q = np.zeros_like(b.q)
    q[:, :, 0] = f32_to_bf16_bits(np.array([c]))[0]
    b.q, b.new_k, b.new_v = q, new_k, new_v
    return b, needles


@pytest.mark.parametrize("part", [-1, 16, 64])
def test_needle_exact(pa, part):
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 100, 255, 256, 257, 700, 1024]
    for D, hq, hkv in [(128, 16, 8), (64, 14, 2)]:
        print(f"[needle] D={D} Hq={hq} Hkv={hkv} part={part}", flush=True)
        b, needles = needle_batch(D, hq, hkv, lens, seed=40 + D)
        d = DeviceBatch(b)
        out = bits(run_decode(pa, d, b, part))
        kp, vp = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
        G = hq // hkv
        for s, L in enumerate(lens):
            for h in range(hq):
                j = needles[s, h // G]
                want = vp[b.block_tables[s, j // 16], j % 16, h // G]
                assert np.array_equal(out[s, h], want), (s, h, L, j)


def test_single_token_and_empty(pa):
    """L = 1 gives V[0] exactly; L = 0 gives zeros (fp32 and bf16)."""
    for dtype in ("bf16", "f32"):
        b = make_batch(50, name="l1", dtype=dtype, num_q_heads=4, num_kv_heads=2, head_dim=64,
                       draw_lens=lambda rng: np.array([1, 0, 1, 0, 1]),
                       draw_query_lens=lambda rng, L: np.minimum(L, 1))
        # sequences with L = 0 have no new token; pad the write's q rows
        d = DeviceBatch(b)
        pa.kv_write(d.new_k, d.new_v, d.slot_mapping, d.k_pool, d.v_pool)
        q = dev(np.concatenate([b.q[:1], b.q[:1], b.q[1:2], b.q[1:2], b.q[2:3]]))
        for part in (-1, 16):
            o = bits(pa.decode(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, 1,
                               partition_tokens=part))
            torch.cuda.synchronize()
            for s, L in enumerate([1, 0, 1, 0, 1]):
                if L == 0:
                    assert not o[s].any()
                else:
                    t = [0, None, 1, None, 2][s]
                    for h in range(4):
                        assert np.array_equal(o[s, h], b.new_v.view(o.dtype)[t, h // 2])


def test_physical_permutation_invariance(pa):
    """Relabelling physical block ids (moving the data with them) leaves the
    output bit-identical."""
    b, _ = prepared("qwen3_small")
    d = DeviceBatch(b)
    base = bits(run_decode(pa, d, b, 64))
    pi = np.random.default_rng(5).permutation(b.num_blocks)
    kp = np.empty_like(b.k_pool)
    vp = np.empty_like(b.v_pool)
    kp[pi], vp[pi] = b.k_pool, b.v_pool
    slots = b.slot_mapping
    b2 = dataclasses.replace(b, k_pool=kp, v_pool=vp,
                             block_tables=pi[b.block_tables].astype(np.int32),
                             slot_mapping=(pi[slots // 16] * 16 + slots % 16).astype(np.int32))
    d2 = DeviceBatch(b2)
    out = bits(run_decode(pa, d2, b2, 64))
    assert np.array_equal(out, base)


def test_shared_prefix_equals_duplicated_blocks(pa):
    """Tables pointing at one shared physical prefix give bit-identical
    output to tables pointing at private copies of it."""
    b, _ = prepared("long_small")
    d = DeviceBatch(b)
    base = bits(run_decode(pa, d, b, 256))
    shared = b.block_tables[0, :40]
    S = b.num_seqs
    extra = b.num_blocks + np.arange((S - 1) * 40).reshape(S - 1, 40)
    kp = np.concatenate([b.k_pool, np.tile(b.k_pool[shared], (S - 1, 1, 1, 1))])
    vp = np.concatenate([b.v_pool, np.tile(b.v_pool[shared], (S - 1, 1, 1, 1))])
    tables = b.block_tables.copy()
    tables[1:, :40] = extra
    b2 = dataclasses.replace(b, k_pool=kp, v_pool=vp, block_tables=tables.astype(np.int32))
    out = bits(run_decode(pa, DeviceBatch(b2), b2, 256))
    assert np.array_equal(out, base)


def test_batch_independence(pa):
    """A sequence's output does not depend on the rest of the batch."""
    b, _ = prepared("qwen3_small")
    d = DeviceBatch(b)
    full = bits(run_decode(pa, d, b, 64))
    idx = [3, 7, 8]
    o = pa.decode(d.q[idx].contiguous(), d.k_pool, d.v_pool, d.block_tables[idx].contiguous(),
                  d.context_lens[idx].contiguous(), b.max_context_len, partition_tokens=64)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), full[idx])


def test_non_default_stream(pa):
    b, ref = prepared("qwen25_small")
    d = DeviceBatch(b)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        pa.kv_write(d.new_k, d.new_v, d.slot_mapping, d.k_pool, d.v_pool)
        out = pa.decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens,
                        b.max_context_len, partition_tokens=0)
    s.synchronize()
    assert_close(f64(out), ref, b.dtype, "non-default stream")


def test_explicit_stream_keeps_its_allocations(pa):
    """stream= passed explicitly (not as the current stream): the workspace
    and the default output are allocated for that stream, so allocations that
    churn on the current stream meanwhile cannot take them over while the
    call's kernels still run.  A split call (partials in the workspace, then
    the merge) on a stream that first waits behind a long kernel."""
    b, ref = prepared("qwen25_small")
    d = DeviceBatch(b)
    pa.kv_write(d.new_k, d.new_v, d.slot_mapping, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    big = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    for trial in range(3):
        with torch.cuda.stream(s):
            torch.mul(big, 1.0001, out=big)  # keeps s busy while the call is enqueued behind it
        out = pa.decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.max_context_len,
                        scale=b.scale, partition_tokens=16, stream=s)
        # churn on the current stream: blocks freed by the call must not come back here
        junk = [torch.full((1 << 16,), float("nan"), device="cuda") for _ in range(64)]
        del junk
        s.synchronize()
        assert_close(f64(out), ref, b.dtype, f"explicit stream, trial {trial}")


def test_empty_contexts_with_partitions(pa):
    """Every context empty (max_context_len 0) with an explicit partition
    size gives zeros, as one pass does, instead of a launch error."""
    b = make_batch(51, name="empty", dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                   draw_lens=lambda rng: np.zeros(4, np.int64), draw_query_lens=lambda rng, L: L,
                   pool_blocks=4)
    d = DeviceBatch(b)
    q = dev(np.full((4, 4, 64), 0x3F80, np.uint16))
    for part in (16, 64, -1, 0):
        out = torch.full_like(q, 5.0)
        pa.decode(q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, 0, out=out, partition_tokens=part)
        torch.cuda.synchronize()
        assert not out.float().abs().sum().item(), part


def test_rejected_call_leaves_output(pa):
    b, _ = prepared("qwen25_small")
    d = DeviceBatch(b)
    out = torch.full_like(d.q, 3.0)
    with pytest.raises(pa.PAError):
        pa.decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.max_context_len,
                  out=out, partition_tokens=24)
    torch.cuda.synchronize()
    assert (out == 3.0).all()


def test_longest_first_order_is_bit_identical(pa):
    """A large batch is processed longest-first (an internal schedule); every
    row must come out bit-identical to decoding it in a small batch, which is
    processed in index order."""
    b, _ = prepared("qwen3_full")
    d = DeviceBatch(b)
    full = bits(run_decode(pa, d, b, -1))
    for lo in range(0, b.num_seqs, 64):
        idx = list(range(lo, min(lo + 8, b.num_seqs)))
        o = pa.decode(d.q[idx].contiguous(), d.k_pool, d.v_pool, d.block_tables[idx].contiguous(),
                      d.context_lens[idx].contiguous(), b.max_context_len, scale=b.scale,
                      partition_tokens=-1)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o), full[idx]), lo
