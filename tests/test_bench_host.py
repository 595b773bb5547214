"""Host logic of bench.py (no GPU): the multi-GPU refusal, the algorithmic
byte and flop counts the roofline divides by, and the gate that reports the
committed HBM-traffic figure only for the kernel sources it was taken on."""
import json
import os
import subprocess
import sys

import numpy as np

from helpers import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
from workloads import long_context, mixed_prefill, qwen3_06b_decode  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def brute_unique_tokens(b) -> int:
    """Distinct (physical block, row) slots holding a token some sequence
    reads, counted slot by slot."""
    bs = b.k_pool.shape[1]
    slots = set()
    for s, L in enumerate(b.context_lens.tolist()):
        for j in range(L):
            slots.add((int(b.block_tables[s, j // bs]), j % bs))
    return len(slots)


def test_unique_tokens_count_shared_blocks_once():
    b = long_context(batch=5, ctx=300, shared_blocks=6)
    assert bench.unique_context_tokens(b) == brute_unique_tokens(b)
    # the shared 96 tokens are counted once, not five times
    assert bench.unique_context_tokens(b) == int(b.context_lens.sum()) - 4 * 6 * 16


def test_decode_bytes_formula():
    b = qwen3_06b_decode(batch=7, prompt=(1, 90), gen=(0, 40))
    es, hkv, d, hq = 2, b.num_kv_heads, b.head_dim, b.num_q_heads
    L = b.context_lens.astype(np.int64)
    expect = (int(L.sum()) * 2 * hkv * d * es          # K and V rows of every context token
              + 2 * b.num_seqs * hq * d * es           # q and out
              + 4 * int(np.sum(-(-L // 16)))           # table entries in use
              + 4 * b.num_seqs)                        # lengths
    assert bench.decode_bytes(b) == expect
    T = int((b.slot_mapping >= 0).sum())
    assert bench.kv_write_bytes(b) == 2 * 2 * T * hkv * d * es + 4 * b.slot_mapping.size


def test_chunk_flops_counts_visible_pairs():
    b = mixed_prefill(seed=9, chunks=2, chunk_len=20, prior_hi=50, n_decode=3, dec_lo=5, dec_hi=30)
    pairs = 0
    qsl, L = b.query_start_loc, b.context_lens
    for s in range(b.num_prefill_seqs):
        n = int(qsl[s + 1] - qsl[s])
        prior = int(L[s]) - n
        pairs += sum(prior + i + 1 for i in range(n))    # row i sees keys 0 .. prior + i
    assert bench.chunk_flops(b) == pairs * b.num_q_heads * 4 * b.head_dim


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    fresh = dict(t, kernel_source_hash=bench.kernel_source_hash())
    p = tmp_path / "fresh.json"
    p.write_text(json.dumps(fresh))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic(-1, 16, "qwen3_06b_decode") == t["hbm_bytes_per_decode"]
    assert bench.measured_traffic(64, 16, "qwen3_06b_decode") is None     # other partition
    assert bench.measured_traffic(-1, 8, "qwen3_06b_decode") is None      # other block size
    assert bench.measured_traffic(-1, 16, "long_context") is None         # other workload
    stale = dict(t, kernel_source_hash="0" * 16)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic(-1, 16, "qwen3_06b_decode") is None


def test_oracle_rows_of_a_subset_are_the_whole_batch_rows():
    """The all-cores baseline leg splits the batch by sequence: the oracle's
    rows for a subset of sequences (prefill chunks and decode rows) equal
    those rows of the whole batch's result."""
    import oracle
    b = mixed_prefill(seed=9, chunks=2, chunk_len=20, prior_hi=50, n_decode=3, dec_lo=5, dec_hi=30)
    kp, vp = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    whole = bench._oracle_rows(b, kp, vp)
    qsl = b.query_start_loc
    for seqs in ([0], [1, 3], [4, 0, 2]):
        rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs])
        assert np.array_equal(bench._oracle_rows(b, kp, vp, seqs), whole[rows])


def test_cpu_baseline_legs_on_a_mixed_batch():
    b = mixed_prefill(seed=9, chunks=2, chunk_len=20, prior_hi=50, n_decode=3, dec_lo=5, dec_hi=30)
    r = bench.cpu_baseline(b, min_seconds=0.0)
    assert r["kind"] == "oracle" and r["cores"] >= 1 and r["one_core"]["cores"] == 1
    assert r["seconds_per_pass"] > 0 and r["one_core"]["seconds_per_pass"] > 0
    assert r["affinity_cores"] == len(os.sched_getaffinity(0))


def test_traffic_record_scales_counters_by_the_copy(tmp_path):
    """FETCH_SIZE/WRITE_SIZE in KiB per dispatch, scaled by what each reads
    for the 1 GiB copy; only decode dispatches right after a KV write count."""
    cols = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"

    def write(path, name, copy_kib, dec_kib, other_kib):
        rows = [f"1,vectorized_elementwise_kernel<MulFunctor>,{name},{copy_kib}",
                f"2,kv_write_kernel,{name},10",
                f"3,rows_kernel<bf16>,{name},{dec_kib}",
                f"4,rows_kernel<bf16>,{name},{other_kib}",   # not after a KV write: ignored
                f"5,kv_write_kernel,{name},10",
                f"6,rows_kernel<bf16>,{name},{dec_kib}"]
        path.write_text(cols + "\n".join(rows) + "\n")

    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    write(f, "FETCH_SIZE", 524288, 500000, 1)     # reads half the copy's bytes: scale 2
    write(w, "WRITE_SIZE", 1048576, 1000, 1)      # reads them exactly: scale 1
    r = bench.traffic_record(str(f), str(w), alg=2 * 500000 * 1024)
    assert r["dispatches"] == 2
    assert r["calibration"]["fetch_scale"] == 2.0 and r["calibration"]["write_scale"] == 1.0
    assert r["hbm_read_bytes"] == 2 * 500000 * 1024 and r["hbm_write_bytes"] == 1000 * 1024
    assert r["traffic_over_algorithmic"] == round((2 * 500000 + 1000) / (2 * 500000), 4)
    assert r["kernel_source_hash"] == bench.kernel_source_hash()
