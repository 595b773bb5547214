"""pa_decode_noalloc on the GPU, through the C ABI: the same output as
pa_decode with a workspace from the caller, bit for bit, and the oracle's
within the tolerance, over calls in a row that use the library's scratch array
for different things (a longest-first order plus split partials, then split
partials alone on smaller inputs), so that what one call leaves in the array
cannot leak into the next."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, bits, dev, ensure_built, f64
from workloads import make_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    ensure_built()
    import paged_kv_attention_22_amd as m
    return m


def batches():
    # more than 2048 sequences: the order array and split partials (64-token partitions)
    big = make_batch(301, name="noalloc_2100", dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                     draw_lens=lambda rng: rng.integers(1, 200, size=2100))
    # few long sequences at G = 7: the library splits them (partials only)
    mid = make_batch(302, name="noalloc_g7", dtype="bf16", num_q_heads=28, num_kv_heads=4, head_dim=128,
                     draw_lens=lambda rng: rng.integers(3000, 6000, size=8))
    small = make_batch(303, name="noalloc_g7_small", dtype="bf16", num_q_heads=28, num_kv_heads=4, head_dim=128,
                       draw_lens=lambda rng: rng.integers(500, 1500, size=3))
    return [(big, 64), (mid, 0), (small, 0), (small, 256)]


def test_noalloc_equals_decode_with_workspace(pa):
    L = pa.lib()
    stream = torch.cuda.current_stream().cuda_stream
    for b, part in batches():
        kp, vp = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
        ref = oracle.decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
        d_k, d_v, q = dev(kp), dev(vp), dev(b.q)
        t, lens = dev(b.block_tables), dev(b.context_lens)
        S, Hq, D = b.q.shape
        need = pa.decode_workspace_bytes(S, Hq, b.num_kv_heads, D, b.max_context_len, part)
        assert 0 < need <= 32 << 20, need  # the call uses the scratch array, within its size
        print(f"[noalloc] {b.name} S={S} part={part} scratch bytes {need}", flush=True)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        out_ws = torch.full_like(q, 7.0)
        out_na = torch.full_like(q, 9.0)
        pool = pa.pool_desc(d_k)
        st = L.pa_decode(q.data_ptr(), d_k.data_ptr(), d_v.data_ptr(), pool, t.data_ptr(), t.shape[1],
                         lens.data_ptr(), S, b.max_context_len, Hq, b.scale, out_ws.data_ptr(), part,
                         ws.data_ptr(), need, stream)
        assert st == 0, pa.status_str(st)
        st = L.pa_decode_noalloc(q.data_ptr(), d_k.data_ptr(), d_v.data_ptr(), pool, t.data_ptr(), t.shape[1],
                                 lens.data_ptr(), S, b.max_context_len, Hq, b.scale, out_na.data_ptr(), part,
                                 stream)
        assert st == 0, pa.status_str(st)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_na), bits(out_ws)), f"{b.name}: noalloc differs from pa_decode"
        assert_close(f64(out_na), ref, b.dtype, f"{b.name} part={part} noalloc vs oracle")
