"""pa_decode_shared_prefix on the GPU: groups of sequences whose block tables
share their first blocks (a prefix-cache hit) decode to the oracle's result,
and to pa_decode's within rounding, for one group and for several groups of
different prefix lengths (0, not a multiple of 16, the whole context), large
groups (several 64-row tiles), block sizes 8/16/32, fp16, and every partition
choice."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, dev, ensure_built, f64
from workloads import long_context, make_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    ensure_built()
    import paged_kv_attention_22_amd as m
    return m


def share(b, groups, prefixes):
    """Tables where each group's members point their first ceil(P/B) entries
    at the group's first member's blocks; returns (tables, group_start)."""
    bs = b.k_pool.shape[1]
    t = b.block_tables.copy()
    start = [0]
    for members, p in zip(groups, prefixes):
        assert members[0] == start[-1] and all(int(b.context_lens[m]) >= p for m in members)
        nb = -(-p // bs)
        for m in members[1:]:
            t[m, :nb] = t[members[0], :nb]
        start.append(members[-1] + 1)
    assert start[-1] == b.num_seqs
    return t, np.asarray(start, np.int32)


def run_case(pa, b, tables, group_start, prefixes, parts=(-1, 0, 64)):
    kp, vp = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    ref = oracle.decode(b.q, kp, vp, tables, b.context_lens, b.scale, b.dtype)
    d_k, d_v, q = dev(kp), dev(vp), dev(b.q)
    d_t, lens = dev(tables), dev(b.context_lens)
    gs, pl = dev(group_start), dev(np.asarray(prefixes, np.int32))
    sizes = np.diff(group_start)
    for i, part in enumerate(parts):
        # the first partition choice also runs without a second stream (the
        # prefix phase first, on the call's stream)
        for aux in ((True, False) if i == 0 else (True,)):
            print(f"[shared prefix] {b.name} S={b.num_seqs} groups={len(prefixes)} prefixes={list(prefixes)[:6]} "
                  f"block={b.k_pool.shape[1]} part={part} aux={aux}", flush=True)
            out = pa.decode_shared_prefix(q, d_k, d_v, d_t, lens, b.max_context_len, gs, pl, int(sizes.max()),
                                          int(max(prefixes)), scale=b.scale, partition_tokens=part, aux=aux)
            plain = pa.decode(q, d_k, d_v, d_t, lens, b.max_context_len, scale=b.scale, partition_tokens=part)
            torch.cuda.synchronize()
            assert_close(f64(out), ref, b.dtype, f"{b.name} part={part} aux={aux} vs oracle")
            assert_close(f64(out), f64(plain), b.dtype, f"{b.name} part={part} aux={aux} vs pa_decode")


def test_one_group_long_prefix(pa):
    """The long-context shape (28/4/128, G = 7) with every sequence sharing 40 blocks."""
    b = long_context(batch=5, ctx=1500, shared_blocks=40)
    S = b.num_seqs
    run_case(pa, b, b.block_tables, np.array([0, S], np.int32), [40 * 16], parts=(-1, 0, 64, 256))


def test_long_context_full_size(pa):
    """The full long-context shape the benchmark times: 64 sequences of
    8,192 tokens, one group sharing a 4,096-token prefix, 28/4 heads (G = 7).
    The library's plan (one pass: 256 (sequence, kv head) units fill the
    chip) runs the prefix phase first in 8 key parts of 512 (seven 64-row
    tiles per kv head, key halves) and folds its partial states into the
    decode kernel's output; the explicit partitions (64, 512 tokens) run the
    prefix phase in 8 parts of 512 (128-row tiles) beside the split decode and
    merge the two."""
    b = long_context()
    S = b.num_seqs
    assert b.shared_prefix_tokens == 4096 and S == 64 and b.max_context_len == 8192
    run_case(pa, b, b.block_tables, np.array([0, S], np.int32), [b.shared_prefix_tokens],
             parts=(-1, 0, 64, 512))


def test_empty_contexts_with_partitions(pa):
    """Every context empty (max_context_len 0) with an explicit partition
    size: zeros, not a launch error."""
    b = make_batch(95, name="empty", dtype="bf16", num_q_heads=28, num_kv_heads=4, head_dim=128,
                   draw_lens=lambda rng: np.zeros(3, np.int64), draw_query_lens=lambda rng, L: L,
                   pool_blocks=4)
    q = dev(np.ones((3, 28, 128), np.uint16) * np.uint16(0x3F80))
    d_k, d_v, d_t, lens = dev(b.k_pool), dev(b.v_pool), dev(b.block_tables), dev(b.context_lens)
    gs, pl = dev(np.array([0, 3], np.int32)), dev(np.array([0], np.int32))
    for part in (16, 64, 0, -1):
        out = torch.full_like(q, 5.0)
        pa.decode_shared_prefix(q, d_k, d_v, d_t, lens, 0, gs, pl, 3, 0, out=out, partition_tokens=part)
        torch.cuda.synchronize()
        assert not out.float().abs().sum().item(), part


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_groups_of_different_prefixes(pa, bs):
    """Qwen3 shape (16/8/128, G = 2): a group of 3 with a 48-token prefix, a
    lone sequence without one, a group of 5 with a 200-token prefix (not a
    multiple of 16), and a group of 2 whose prefix is the whole context of
    one member."""
    lens = np.array([300, 90, 61, 450, 700, 205, 260, 333, 901, 128, 129], np.int64)
    b = make_batch(91, name=f"groups_bs{bs}", dtype="bf16", num_q_heads=16, num_kv_heads=8, head_dim=128,
                   block_size=bs, draw_lens=lambda rng: lens)
    groups = [[0, 1, 2], [3], [4, 5, 6, 7, 8], [9, 10]]
    prefixes = [48, 0, 200, 128]
    tables, gs = share(b, groups, prefixes)
    run_case(pa, b, tables, gs, prefixes)


def test_large_group_g7_d64_and_fp16(pa):
    """40 sequences in one group at G = 7 (280 rows per kv head: five 64-row
    tiles), head_dim 64; then fp16 pools at head_dim 128, G = 4."""
    b = make_batch(92, name="g7_d64_group40", dtype="bf16", num_q_heads=14, num_kv_heads=2, head_dim=64,
                   draw_lens=lambda rng: rng.integers(700, 1400, size=40))
    tables, gs = share(b, [list(range(40))], [640])
    run_case(pa, b, tables, gs, [640])
    b = make_batch(93, name="g4_d128_f16", dtype="f16", num_q_heads=16, num_kv_heads=4, head_dim=128,
                   draw_lens=lambda rng: rng.integers(300, 900, size=12))
    tables, gs = share(b, [list(range(6)), list(range(6, 12))], [256, 290])
    run_case(pa, b, tables, gs, [256, 290])


@pytest.mark.parametrize("S", [60, 72])
def test_many_small_groups(pa, S):
    """Thirty (or thirty-six) groups of two, prefixes from 16 to 576 tokens:
    the prefix phase has a 64-row tile per (group, kv head), 240 (or 288)
    of them, so the one-pass plan keeps the prefix in one key part (with
    288 even one part exceeds the small launch)."""
    b = make_batch(94, name=f"pairs{S}", dtype="bf16", num_q_heads=16, num_kv_heads=8, head_dim=128,
                   draw_lens=lambda rng: rng.integers(600, 1200, size=S))
    groups = [[2 * i, 2 * i + 1] for i in range(S // 2)]
    prefixes = [16 * (1 + i) for i in range(S // 2)]
    tables, gs = share(b, groups, prefixes)
    run_case(pa, b, tables, gs, prefixes, parts=(0,))


def test_large_batch_with_order_array(pa):
    """2,100 sequences in 30 groups of 70: more rows than the decode kernels
    rank themselves, so a sorting launch writes the longest-first order to
    the front of the workspace and the one-pass plan keeps the prefix's
    partial states after it.  G = 2 (the vector decode path)."""
    S, n = 2100, 70
    b = make_batch(96, name="order2100", dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                   draw_lens=lambda rng: rng.integers(130, 400, size=S))
    groups = [list(range(n * i, n * (i + 1))) for i in range(S // n)]
    prefixes = [32 + 3 * i for i in range(S // n)]   # not all multiples of 16
    tables, gs = share(b, groups, prefixes)
    run_case(pa, b, tables, gs, prefixes, parts=(-1, 0))


def test_no_group_has_a_prefix(pa):
    """max_prefix_len 0 (a batch with no prefix-cache hit): the one-pass plan
    is plain pa_decode (no prefix phase, no partial states, no workspace), the
    split plan keeps its partitions and merge."""
    b = make_batch(97, name="noprefix", dtype="bf16", num_q_heads=28, num_kv_heads=4, head_dim=128,
                   draw_lens=lambda rng: rng.integers(1, 1500, size=40))
    groups = [list(range(10 * i, 10 * (i + 1))) for i in range(4)]
    tables, gs = share(b, groups, [0, 0, 0, 0])
    assert pa.decode_shared_prefix_workspace_bytes(40, 28, 4, 128, b.max_context_len, 4, 10, 0, -1) == 0
    run_case(pa, b, tables, gs, [0, 0, 0, 0], parts=(-1, 0, 64))
