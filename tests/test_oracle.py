"""Pins for the fp64 oracle, independent of the oracle's own code.

Each ``pin_*`` takes the oracle module so that the mutation tests at the end
can run the same pins against copies of the oracle with a planted mistake and
check that some pin catches each one.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle.ref as ORACLE
from workloads import f32_to_bf16_bits, tiny_f32, qwen25_05b_decode, mixed_prefill

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")
B = 16  # block size


# ----------------------------------------------------------------- helpers
def scatter_dense(dense_list, num_blocks, rng, hkv, d, fill=np.nan, bs=B):
    """Independent pool builder: places each sequence's logical K (or V) rows
    [L, Hkv, D] into a fresh pool of bs-token blocks under a random
    physical-id permutation.  Returns (pool, tables)."""
    perm = rng.permutation(num_blocks)
    pool = np.full((num_blocks * bs, hkv, d), fill)
    maxb = max(1, max(-(-x.shape[0] // bs) for x in dense_list))
    tables = np.full((len(dense_list), maxb), perm[-1], np.int64)
    cur = 0
    for s, x in enumerate(dense_list):
        nb = -(-x.shape[0] // bs)
        tables[s, :nb] = perm[cur:cur + nb]
        cur += nb
        flat = np.repeat(tables[s, :nb], bs)[: x.shape[0]] * bs + np.tile(np.arange(bs), nb)[: x.shape[0]]
        pool[flat] = x
    return pool.reshape(num_blocks, bs, hkv, d), tables


def sdpa_f64(q, K, V, scale, mask=None):
    """torch's scaled_dot_product_attention on CPU float64 with repeated KV.
    q [n, Hq, D], K/V [L, Hkv, D]; mask [n, L] bool (True = visible)."""
    hq, hkv = q.shape[1], K.shape[1]
    rep = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).repeat_interleave(rep, dim=1).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(V).repeat_interleave(rep, dim=1).permute(1, 0, 2)[None].contiguous()
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def build_golden_pools(c):
    shape = (c["num_blocks"], B, c["num_kv_heads"], c["head_dim"])
    kp = np.full(shape, c["junk"])
    vp = np.full(shape, c["junk"])
    for blk, off, h, vec in c["k_entries"]:
        kp[blk, off, h] = vec
    for blk, off, h, vec in c["v_entries"]:
        vp[blk, off, h] = vec
    return kp, vp


# -------------------------------------------------------------------- pins
def pin_golden(ref):
    for c in load_golden():
        kp, vp = build_golden_pools(c)
        qsl = np.concatenate([[0], np.cumsum(c["query_lens"])])
        out = ref.attention(np.array(c["q"], np.float64), qsl, kp, vp,
                            np.array(c["block_tables"]), np.array(c["context_lens"]),
                            c["scale"], "f64")
        np.testing.assert_allclose(out, np.array(c["expected"]), rtol=0, atol=1e-12,
                                   err_msg=c["name"])


def pin_dense_vs_sdpa_decode(ref):
    rng = np.random.default_rng(11)
    for hq, hkv, d in [(2, 1, 64), (14, 2, 64), (4, 4, 16), (6, 2, 8)]:
        lens = [1, 5, 16, 17, 31, 32, 33, 70]
        Ks = [rng.standard_normal((L, hkv, d)) for L in lens]
        Vs = [rng.standard_normal((L, hkv, d)) for L in lens]
        q = rng.standard_normal((len(lens), hq, d))
        nb = sum(-(-L // B) for L in lens) + 3
        kp, tab = scatter_dense(Ks, nb, np.random.default_rng(5), hkv, d)
        vp, tab2 = scatter_dense(Vs, nb, np.random.default_rng(5), hkv, d)
        assert np.array_equal(tab, tab2)
        scale = 1 / math.sqrt(d)
        out = ref.decode(q, kp, vp, tab, np.array(lens), scale, "f64")
        for s, L in enumerate(lens):
            want = sdpa_f64(q[s:s + 1], Ks[s], Vs[s], scale)[0]
            np.testing.assert_allclose(out[s], want, rtol=0, atol=1e-12)


def pin_other_block_sizes(ref):
    """Pools of 8- and 32-token blocks (the pages leave the block size
    tunable): paged decode and prefill still equal dense attention."""
    rng = np.random.default_rng(13)
    hq, hkv, d = 4, 2, 16
    for bs in (8, 32):
        lens = [1, 7, 8, 9, 31, 32, 33, 65]
        Ks = [rng.standard_normal((L, hkv, d)) for L in lens]
        Vs = [rng.standard_normal((L, hkv, d)) for L in lens]
        q = rng.standard_normal((len(lens), hq, d))
        nb = sum(-(-L // bs) for L in lens) + 2
        kp, tab = scatter_dense(Ks, nb, np.random.default_rng(9), hkv, d, bs=bs)
        vp, _ = scatter_dense(Vs, nb, np.random.default_rng(9), hkv, d, bs=bs)
        scale = 1 / math.sqrt(d)
        out = ref.decode(q, kp, vp, tab, np.array(lens), scale, "f64")
        for s, L in enumerate(lens):
            np.testing.assert_allclose(out[s], sdpa_f64(q[s:s + 1], Ks[s], Vs[s], scale)[0], rtol=0, atol=1e-12)
        # a 5-row chunk at the end of each context
        n = 5
        rows = [rng.standard_normal((min(n, L), hq, d)) for L in lens]
        qsl = np.concatenate([[0], np.cumsum([r.shape[0] for r in rows])])
        out = ref.attention(np.concatenate(rows), qsl, kp, vp, tab, np.array(lens), scale, "f64")
        for s, L in enumerate(lens):
            m = rows[s].shape[0]
            mask = np.arange(L)[None, :] <= (L - m + np.arange(m))[:, None]
            np.testing.assert_allclose(out[qsl[s]:qsl[s + 1]], sdpa_f64(rows[s], Ks[s], Vs[s], scale, mask),
                                       rtol=0, atol=1e-12)


def pin_dense_vs_sdpa_prefill(ref):
    rng = np.random.default_rng(12)
    hq, hkv, d = 4, 2, 32
    cases = [(0, 5), (3, 4), (16, 16), (20, 13), (0, 40)]  # (prior context, chunk rows)
    Ks, Vs, qs = [], [], []
    for prior, n in cases:
        L = prior + n
        Ks.append(rng.standard_normal((L, hkv, d)))
        Vs.append(rng.standard_normal((L, hkv, d)))
        qs.append(rng.standard_normal((n, hq, d)))
    nb = sum(-(-(p + n) // B) for p, n in cases) + 2
    kp, tab = scatter_dense(Ks, nb, np.random.default_rng(7), hkv, d)
    vp, _ = scatter_dense(Vs, nb, np.random.default_rng(7), hkv, d)
    lens = np.array([p + n for p, n in cases])
    qsl = np.concatenate([[0], np.cumsum([n for _, n in cases])])
    out = ref.attention(np.concatenate(qs), qsl, kp, vp, tab, lens, 0.3, "f64")
    for s, (prior, n) in enumerate(cases):
        L = prior + n
        mask = np.arange(L)[None, :] <= (prior + np.arange(n))[:, None]
        want = sdpa_f64(qs[s], Ks[s], Vs[s], 0.3, mask)
        np.testing.assert_allclose(out[qsl[s]:qsl[s + 1]], want, rtol=0, atol=1e-12)
        if prior == 0:  # plain causal self-attention, torch's own is_causal path
            qt = torch.from_numpy(qs[s]).permute(1, 0, 2)[None]
            kt = torch.from_numpy(Ks[s]).repeat_interleave(hq // hkv, 1).permute(1, 0, 2)[None].contiguous()
            vt = torch.from_numpy(Vs[s]).repeat_interleave(hq // hkv, 1).permute(1, 0, 2)[None].contiguous()
            o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.3)
            np.testing.assert_allclose(out[qsl[s]:qsl[s + 1]], o[0].permute(1, 0, 2).numpy(), atol=1e-12)


def pin_permutation(ref):
    b = qwen25_05b_decode(seed=21, batch=6, lo=1, hi=120)
    kp, vp = ref.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    base = ref.decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, "bf16")
    pi = np.random.default_rng(3).permutation(b.num_blocks)   # old id -> new id
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[pi] = kp
    vp2[pi] = vp
    out = ref.decode(b.q, kp2, vp2, pi[b.block_tables], b.context_lens, b.scale, "bf16")
    assert np.array_equal(out, base)


def pin_single_token(ref):
    rng = np.random.default_rng(4)
    v = rng.standard_normal((3, 1, 2, 8))                     # 3 blocks, slot 0 used
    kp = rng.standard_normal((3, B, 2, 8))
    vp = np.full((3, B, 2, 8), np.nan)
    vp[:, 0] = v[:, 0]
    q = rng.standard_normal((3, 4, 8)) * 50
    out = ref.decode(q, kp, vp, np.array([[2], [0], [1]]), np.array([1, 1, 1]), 0.7, "f64")
    for s, blk in enumerate([2, 0, 1]):
        for h in range(4):
            assert np.array_equal(out[s, h], vp[blk, 0, h // 2])


def pin_uniform_keys(ref):
    rng = np.random.default_rng(5)
    L, d = 37, 16
    kp = np.zeros((3, B, 1, d))
    kp[:] = rng.standard_normal(d)            # every key identical
    vp = rng.standard_normal((3, B, 1, d))
    tab = np.array([[1, 2, 0]])
    out = ref.decode(rng.standard_normal((1, 3, d)), kp, vp, tab, np.array([L]), 0.25, "f64")
    rows = np.concatenate([vp[1], vp[2], vp[0]])[:L, 0]
    for h in range(3):
        np.testing.assert_allclose(out[0, h], rows.mean(0), rtol=0, atol=1e-14)
    # q = 0 also gives the mean, whatever the keys.
    kp = rng.standard_normal((3, B, 1, d))
    out = ref.decode(np.zeros((1, 1, d)), kp, vp, tab, np.array([L]), 0.25, "f64")
    np.testing.assert_allclose(out[0, 0], rows.mean(0), rtol=0, atol=1e-14)


def pin_two_token_sigmoid(ref):
    rng = np.random.default_rng(6)
    d = 5
    kp = rng.standard_normal((1, B, 1, d))
    vp = rng.standard_normal((1, B, 1, d))
    q = rng.standard_normal((1, 1, d))
    out = ref.decode(q, kp, vp, np.array([[0]]), np.array([2]), 0.9, "f64")[0, 0]
    s0 = 0.9 * float(q[0, 0] @ kp[0, 0, 0])
    s1 = 0.9 * float(q[0, 0] @ kp[0, 1, 0])
    sig = lambda x: 1 / (1 + math.exp(-x))
    want = sig(s0 - s1) * vp[0, 0, 0] + sig(s1 - s0) * vp[0, 1, 0]
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-14)


def pin_brute_force(ref):
    rng = np.random.default_rng(8)
    hq, hkv, d = 4, 2, 3
    for L in (1, 2, 3):
        kp = rng.standard_normal((2, B, hkv, d))
        vp = rng.standard_normal((2, B, hkv, d))
        q = rng.standard_normal((1, hq, d))
        out = ref.decode(q, kp, vp, np.array([[1]]), np.array([L]), 0.5, "f64")
        for h in range(hq):
            g = h // (hq // hkv)
            scores = [0.5 * sum(q[0, h, i] * kp[1, j, g, i] for i in range(d)) for j in range(L)]
            e = [math.exp(x) for x in scores]
            tot = sum(e)
            want = [sum(e[j] / tot * vp[1, j, g, i] for j in range(L)) for i in range(d)]
            np.testing.assert_allclose(out[0, h], want, rtol=0, atol=1e-14)


def pin_gqa_repeat(ref):
    b = qwen25_05b_decode(seed=22, batch=4, lo=20, hi=60)
    kp, vp = ref.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    gqa = ref.decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, "bf16")
    rep = b.num_q_heads // b.num_kv_heads
    mha = ref.decode(b.q, np.repeat(kp, rep, axis=2), np.repeat(vp, rep, axis=2),
                     b.block_tables, b.context_lens, b.scale, "bf16")
    assert np.array_equal(gqa, mha)


def pin_prefill_reductions(ref):
    b = mixed_prefill(seed=23, chunks=2, chunk_len=20, prior_hi=40, n_decode=3,
                      dec_lo=5, dec_hi=50)
    kp, vp = ref.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    full = ref.attention(b.q, b.query_start_loc, kp, vp, b.block_tables,
                         b.context_lens, b.scale, "bf16")
    # n = 1 rows are decode.
    dec = slice(b.num_prefill_seqs, b.num_seqs)
    rows = b.query_start_loc[b.num_prefill_seqs:-1]
    out = ref.decode(b.q[rows], kp, vp, b.block_tables[dec], b.context_lens[dec], b.scale, "bf16")
    assert np.array_equal(out, full[rows])
    # The last row of a chunk equals a decode of that token over the context.
    for s in range(b.num_prefill_seqs):
        last = b.query_start_loc[s + 1] - 1
        d1 = ref.decode(b.q[last:last + 1], kp, vp, b.block_tables[s:s + 1],
                        b.context_lens[s:s + 1], b.scale, "bf16")
        assert np.array_equal(d1[0], full[last])
    # Splitting a chunk into two chunks gives the same rows: rows of the first
    # half see the context truncated to their own end.
    s = 0
    n, L = int(b.query_lens[s]), int(b.context_lens[s])
    h = n // 2
    first = ref.attention(b.q[:h], np.array([0, h]), kp, vp, b.block_tables[:1],
                          np.array([L - n + h]), b.scale, "bf16")
    assert np.array_equal(first, full[:h])
    # P = 0, n = L: row 0 sees only key 0, so it equals V[0].
    rng = np.random.default_rng(9)
    kq = rng.standard_normal((1, B, 1, 4))
    vq = rng.standard_normal((1, B, 1, 4))
    o = ref.attention(rng.standard_normal((5, 2, 4)), np.array([0, 5]), kq, vq,
                      np.array([[0]]), np.array([5]), 0.5, "f64")
    assert np.array_equal(o[0, 0], vq[0, 0, 0]) and np.array_equal(o[0, 1], vq[0, 0, 0])


def pin_kv_write_roundtrip(ref):
    rng = np.random.default_rng(10)
    nb, hkv, d = 5, 2, 4
    kp = rng.integers(0, 2**16, size=(nb, B, hkv, d), dtype=np.uint16)
    vp = rng.integers(0, 2**16, size=(nb, B, hkv, d), dtype=np.uint16)
    slots = np.array([0, 17, -1, 79, 33, -5, 64])     # includes slot 0 and the last slot
    nk = rng.integers(0, 2**16, size=(len(slots), hkv, d), dtype=np.uint16)
    nv = rng.integers(0, 2**16, size=(len(slots), hkv, d), dtype=np.uint16)
    k2, v2 = ref.kv_write(kp, vp, nk, nv, slots)
    k_rows, v_rows = k2.reshape(-1, hkv, d), v2.reshape(-1, hkv, d)
    written = set()
    for t, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(k_rows[s], nk[t]) and np.array_equal(v_rows[s], nv[t])
            written.add(int(s))
    keep = [r for r in range(nb * B) if r not in written]
    assert np.array_equal(k_rows[keep], kp.reshape(-1, hkv, d)[keep])
    assert np.array_equal(v_rows[keep], vp.reshape(-1, hkv, d)[keep])
    # Gather after write returns the written rows: a table [b1, b2] reads
    # slots b1*16 .. b1*16+15, then b2*16 ...
    tab = np.array([4, 1])
    g = ref.gather(k2, tab, 18)
    assert np.array_equal(g[0], nk[6]) and np.array_equal(g[17], nk[1])


ALL_PINS = [pin_golden, pin_dense_vs_sdpa_decode, pin_other_block_sizes, pin_dense_vs_sdpa_prefill,
            pin_permutation, pin_single_token, pin_uniform_keys,
            pin_two_token_sigmoid, pin_brute_force, pin_gqa_repeat,
            pin_prefill_reductions, pin_kv_write_roundtrip]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ORACLE)


# ------------------------------------------------------- decode of storage
def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(1).integers(0, 2**16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]             # finite values only
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(ORACLE.to_f64(bits, "bf16"), want)


def test_f16_decode_matches_torch():
    vals = np.random.default_rng(2).standard_normal(4096).astype(np.float16)
    want = torch.from_numpy(vals).double().numpy()
    assert np.array_equal(ORACLE.to_f64(vals, "f16"), want)


def test_oracle_finite_on_poisoned_batches():
    """Generator batches carry NaN in every slot no sequence may read; a
    finite oracle result shows the oracle reads nothing past each length."""
    for b in (tiny_f32(), qwen25_05b_decode(batch=5, lo=1, hi=100),
              mixed_prefill(chunks=2, chunk_len=9, prior_hi=30, n_decode=4, dec_lo=1, dec_hi=40)):
        kp, vp = ORACLE.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
        out = ORACLE.attention(b.q, b.query_start_loc, kp, vp, b.block_tables,
                               b.context_lens, b.scale, b.dtype)
        assert np.isfinite(out).all(), b.name


# ---------------------------------------------------------------- mutants
MUTANTS = {
    "gqa_interleaved": ("g = h // group", "g = h % Hkv"),
    "causal_off_by_one": ("visible = L - n + i + 1", "visible = L - n + i"),
    "causal_top_left": ("visible = L - n + i + 1", "visible = i + 1"),
    "scale_dropped": ("scores = (keys @ q) * scale", "scores = (keys @ q)"),
    "score_sign": ("scores = (keys @ q) * scale", "scores = -(keys @ q) * scale"),
    "no_normalise": ("weights = weights / weights.sum()", "weights = weights"),
    "wrong_operand": ("return weights @ values", "return weights @ keys"),
    "gather_offset": ("offs = [j % bsz", "offs = [(j + 1) % bsz"),
    "gather_block": ("int(table_row[j // bsz])", "int(table_row[(j // bsz) % 1])"),
    "write_skips_slot0": ("if slot < 0:", "if slot <= 0:"),
    "write_transposed": ("block, offset = divmod(slot, bsz)",
                         "offset, block = divmod(slot, bsz)"),
    "write_k_into_v": ("v_out[block, offset] = new_v[t]", "v_out[block, offset] = new_k[t]"),
}


def make_mutant(old, new):
    with open(ORACLE.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mutant = make_mutant(*MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except Exception:       # an assertion or an indexing error both count
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
