"""Benchmark: one decode step of the paged-KV attention hot path on one GPU.

A step is the KV write of every sequence's new token and batched GQA decode
attention over the paged pool (by default one pa_decode_append call, which
fuses the two; the two-call step, pa_kv_write then pa_decode, is timed beside
it and the pa_decode call alone gives the roofline), on the Qwen3-0.6B-shaped
workload
(16 q / 8 kv heads, head_dim 128, bf16, block size 16, 256 sequences with
context = U[100,1024] + U[0,1024] capped at 2048, pool 1.2x the blocks in use,
permuted block ids).  Inputs are synthetic and resident in HBM before timing.

Two copies of the pools alternate between steps, so no step finds the previous
step's K/V in the 256 MB last-level cache: every step streams its context from
HBM, as a real decode step over a large batch does.

Prints ONE JSON line (see the fields below).  --gpus N > 1 exits: this path runs
on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "pa_decode HBM GB/s (% of peak) + seq-steps/s, Qwen3-0.6B shape, batch 256"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, AMD published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_qwen3_06b_b256_traffic.json")
KERNEL_SOURCES = ["attn_rows.hip", "rows_body.hpp", "pa_device.hpp", "pa_internal.hpp", "pa_api.cpp"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_attention_22_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(partition: int, block_size: int, workload: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, when
    they were taken on the kernel sources, workload, block size and partition
    in use now."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel_source_hash") != kernel_source_hash() or t.get("partition_tokens") != partition
            or t.get("block_size", 16) != block_size or not str(t.get("workload", "")).startswith(workload)):
        return None
    return t.get("hbm_bytes_per_decode")


def traffic_record(fetch_csv: str, write_csv: str, alg: int | None = None) -> dict:
    """The traffic record of the headline decode kernel, from the counter CSVs
    of two rocprofv3 runs of `bench.py --no-cpu-baseline --copy-first --steps 5
    --warmup 1`, one with --pmc FETCH_SIZE and one with --pmc WRITE_SIZE (KiB
    per dispatch).  Each counter is scaled to bytes by what it reads for the
    1 GiB elementwise kernel the same process runs first (1 GiB read and
    1 GiB written per launch).  The decode dispatches are those of the
    two-call steps: each directly follows a kv_write dispatch."""
    import csv
    import statistics

    def pick(path):
        with open(path) as f:
            rs = list(csv.DictReader(f))
        copy = [float(r["Counter_Value"]) for r in rs if "MulFunctor" in r["Kernel_Name"]]
        dec = [float(r["Counter_Value"]) for i, r in enumerate(rs)
               if "rows_kernel" in r["Kernel_Name"] and i > 0 and "kv_write_kernel" in rs[i - 1]["Kernel_Name"]]
        if not copy or not dec:
            raise SystemExit(f"{path}: no calibration or decode dispatches found")
        return statistics.mean(copy), statistics.mean(dec), len(dec)

    copy_f, dec_f, n = pick(fetch_csv)
    copy_w, dec_w, _ = pick(write_csv)
    fs, ws = (1 << 30) / 1024 / copy_f, (1 << 30) / 1024 / copy_w
    rd, wr = dec_f * fs * 1024, dec_w * ws * 1024
    if alg is None:  # the headline batch's algorithmic bytes
        from workloads import qwen3_06b_decode
        alg = decode_bytes(qwen3_06b_decode())
    cmd = ("cd /tmp && timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d <out> -o run -- "
           "python3 /root/repo/bench.py --no-cpu-baseline --copy-first --steps 5 --warmup 1")
    return {
        "kernel": "rows_kernel<bf16, 128, 2> (pa_decode, one pass, longest first ranked in-kernel)",
        "workload": "qwen3_06b_decode (seed 3): 256 seqs, 16/8 heads, head_dim 128, bf16, block size 16",
        "block_size": 16,
        "kernel_source_hash": kernel_source_hash(),
        "partition_tokens": -1,
        "fetch_size_kib_per_dispatch": round(dec_f, 1),
        "write_size_kib_per_dispatch": round(dec_w, 1),
        "dispatches": n,
        "calibration": {
            "kernel": "torch.mul int32 over 1 GiB, three launches in the same process before the decode steps "
                      "(bench.py --copy-first): 1 GiB read + 1 GiB written per launch",
            "fetch_size_kib": round(copy_f, 1), "write_size_kib": round(copy_w, 1),
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
        "hbm_bytes_per_decode": int(rd + wr),
        "hbm_read_bytes": int(rd),
        "hbm_write_bytes": int(wr),
        "algorithmic_bytes": alg,
        "traffic_over_algorithmic": round((rd + wr) / alg, 4),
        "commands": [cmd.format(c="FETCH_SIZE"), cmd.format(c="WRITE_SIZE"),
                     "python3 bench.py --traffic-record <out>/fetch/run_counter_collection.csv "
                     "<out>/write/run_counter_collection.csv > profiles/decode_qwen3_06b_b256_traffic.json"],
        "dispatch_selection": "pa_decode dispatches of the two-call steps (each directly after a kv_write dispatch)",
    }


def unique_context_tokens(b) -> int:
    """Distinct pool slots the batch reads: a physical block shared by several
    tables (a common prefix) counts once."""
    import numpy as np
    bs = b.k_pool.shape[1]
    used = {}
    for s, L in enumerate(b.context_lens.tolist()):
        nb = -(-L // bs)
        for j, blk in enumerate(b.block_tables[s, :nb].tolist()):
            used[blk] = max(used.get(blk, 0), min(bs, L - bs * j))
    return int(np.sum(list(used.values()))) if used else 0


def decode_bytes(b) -> int:
    """Algorithmic bytes of one decode call: each distinct context token's K
    and V row once (shared prefix blocks once), q and out, the block-table
    entries in use and the lengths."""
    es = b.elem_bytes
    kv = unique_context_tokens(b) * 2 * b.num_kv_heads * b.head_dim * es
    qo = 2 * b.num_seqs * b.num_q_heads * b.head_dim * es
    bs = b.k_pool.shape[1]
    tables = 4 * int(sum(-(-int(L) // bs) for L in b.context_lens))
    return kv + qo + tables + 4 * b.num_seqs


def chunk_flops(b) -> int:
    """Algorithmic flops of the prefill chunks: every visible (row, key) pair
    costs 2*D for q.k and 2*D for the weighted V sum, per q head."""
    total = 0
    for s in range(b.num_prefill_seqs):
        n, L = int(b.query_lens[s]), int(b.context_lens[s])
        pairs = n * (L - n) + n * (n + 1) // 2
        total += pairs * b.num_q_heads * 4 * b.head_dim
    return total


def kv_write_bytes(b) -> int:
    T = int((b.slot_mapping >= 0).sum())
    return 2 * 2 * T * b.num_kv_heads * b.head_dim * b.elem_bytes + 4 * b.slot_mapping.size


class Timer:
    """HIP events created with hipEventDisableSystemFence, for timing only: an
    ordinary event record performs a system-scope release (cache write-back
    and invalidation) that stretches the interval it brackets and slows the
    work after it.  The events come from the HIP runtime torch has already
    loaded (same soname), so they take torch's stream handles."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import ctypes
        import torch
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            self._check(self._hip.hipEventCreateWithFlags(ctypes.byref(e),
                                                          ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)))
            self._ev.append(e)
        self._stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    @staticmethod
    def _check(rc: int) -> None:
        if rc != 0:
            raise RuntimeError(f"HIP event call failed with hipError {rc}")

    def start(self, i: int) -> None:
        self._check(self._hip.hipEventRecord(self._ev[2 * i], self._stream))

    def stop(self, i: int) -> None:
        self._check(self._hip.hipEventRecord(self._ev[2 * i + 1], self._stream))

    def us(self, i: int) -> float:
        import ctypes
        ms = ctypes.c_float()
        self._check(self._hip.hipEventSynchronize(self._ev[2 * i + 1]))
        self._check(self._hip.hipEventElapsedTime(ctypes.byref(ms), self._ev[2 * i], self._ev[2 * i + 1]))
        return ms.value * 1e3

    def close(self) -> None:
        for e in self._ev:
            self._hip.hipEventDestroy(e)
        self._ev = []


def time_calls(fn, steps: int, warmup: int):
    """Per-call durations (us) from fence-free HIP events on the current
    stream (the one the library launches on)."""
    import numpy as np
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    t = Timer(steps)
    for i in range(steps):
        t.start(i)
        fn(i)
        t.stop(i)
    torch.cuda.synchronize()
    us = np.array([t.us(i) for i in range(steps)])
    t.close()
    return us


def time_steps(fn, steps: int, warmup: int) -> float:
    """Mean wall time (us) of `steps` calls enqueued back to back between two
    synchronisations, with nothing else on the stream."""
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / steps


def bench_mixed(args, b, up, dev) -> dict:
    """Mixed chunked-prefill step: KV write of every new token, then
    pa_prefill_chunk over the chunks and the decode rows.  Also times the
    chunk rows alone (matrix cores) and the decode rows alone."""
    import numpy as np
    import torch

    import paged_kv_attention_22_amd as pa
    pools = [(up(b.k_pool), up(b.v_pool)) for _ in range(2)]
    q, new_k, new_v = up(b.q), up(b.new_k), up(b.new_v)
    slots, tables, lens = up(b.slot_mapping), up(b.block_tables), up(b.context_lens)
    qsl = up(b.query_start_loc)
    out = torch.empty_like(q)
    npre, S = b.num_prefill_seqs, b.num_seqs
    for kp, vp in pools:
        pa.kv_write(new_k, new_v, slots, kp, vp)
    rows_pre = int(b.query_start_loc[npre])
    sub = dict(q=q[:rows_pre], qsl=qsl[:npre + 1].contiguous(), tables=tables[:npre].contiguous(),
               lens=lens[:npre].contiguous())
    dec = dict(q=q[rows_pre:].contiguous(), tables=tables[npre:].contiguous(),
               lens=lens[npre:].contiguous())
    maxc = b.max_context_len

    def step(i):
        kp, vp = pools[i & 1]
        pa.kv_write(new_k, new_v, slots, kp, vp)
        pa.prefill_chunk(q, qsl, npre, b.max_query_len, kp, vp, tables, lens, maxc,
                         scale=b.scale, out=out)

    def chunks(i):
        kp, vp = pools[i & 1]
        pa.prefill_chunk(sub["q"], sub["qsl"], npre, b.max_query_len, kp, vp, sub["tables"],
                         sub["lens"], maxc, scale=b.scale)

    def decode_rows(i):
        kp, vp = pools[i & 1]
        pa.decode(dec["q"], kp, vp, dec["tables"], dec["lens"], maxc, scale=b.scale)

    log(f"[bench] timing {args.steps} mixed steps")
    step_mean_us = time_steps(step, args.steps, args.warmup)
    step_us = time_calls(step, args.steps, args.warmup)
    chunk_us = time_calls(chunks, args.steps, args.warmup)
    dec_us = time_calls(decode_rows, args.steps, args.warmup)
    flops = chunk_flops(b)
    es = b.elem_bytes
    dec_bytes = int(b.context_lens[npre:].sum()) * 2 * b.num_kv_heads * b.head_dim * es
    ms = step_mean_us * 1e-3
    return {
        "metric": "pa_prefill_chunk mixed batch step time (KV write + chunks + decode rows)",
        "value": round(ms * 1e3, 2), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": b.dtype, "data": "synthetic",
        "config": {"workload": b.name, "recipe": b.recipe, "seed": b.seed, "num_seqs": S,
                   "num_prefill_seqs": npre, "total_query_tokens": b.total_query_tokens},
        "step_us_events": {"median": round(float(np.median(step_us)), 2),
                           "p10": round(float(np.percentile(step_us, 10)), 2),
                           "p90": round(float(np.percentile(step_us, 90)), 2)},
        "chunks": {"us": round(float(np.median(chunk_us)), 2), "gflop": round(flops / 1e9, 3),
                   "tflops": round(flops / (float(np.median(chunk_us)) * 1e-6) / 1e12, 2),
                   "peak_tflops": 2500.0},
        "decode_rows": {"us": round(float(np.median(dec_us)), 2), "bytes": dec_bytes,
                        "gbs": round(dec_bytes / (float(np.median(dec_us)) * 1e-6) / 1e9, 1)},
    }


def fused_write_bytes(b) -> int:
    """Algorithmic bytes of pa_qkv_rope_write: each packed row read once, the
    rotated q written, one K and one V row written per token, the two norm
    weight vectors, and per token its slot out, its length and its table
    entry."""
    T = b.q.shape[0]
    es = b.elem_bytes
    hq, hkv, d = b.num_q_heads, b.num_kv_heads, b.head_dim
    return T * ((hq + 2 * hkv) * d + hq * d + 2 * hkv * d) * es + 2 * d * es + 12 * T


def bench_fused(args, b, up) -> dict:
    """The fused QKV split + rotary + KV write on the workload's new tokens
    (packed rows built from the batch's q and new K/V), alone and as the write
    half of a decode step (fused write + pa_decode) beside the plain step
    (pa_kv_write + pa_decode)."""
    import numpy as np
    import torch

    import paged_kv_attention_22_amd as pa
    from workloads import norm_weights, packed_qkv
    pools = [(up(b.k_pool), up(b.v_pool)) for _ in range(2)]
    qkv = up(packed_qkv(b))
    qn, kn = (up(w) for w in norm_weights(b, 77))
    tables, lens = up(b.block_tables), up(b.context_lens)
    qsl = up(b.query_start_loc) if b.num_prefill_seqs else None
    q_out = torch.empty_like(up(b.q))
    q, new_k, new_v, slots = up(b.q), up(b.new_k), up(b.new_v), up(b.slot_mapping)
    out = torch.empty_like(q)
    theta = 1e6

    def fused(i):
        kp, vp = pools[i & 1]
        pa.qkv_rope_write(qkv, b.num_q_heads, lens, tables, kp, vp, theta, query_start_loc=qsl,
                          q_norm=qn, k_norm=kn, q_out=q_out)

    def fused_step(i):
        kp, vp = pools[i & 1]
        fused(i)
        pa.decode(q_out, kp, vp, tables, lens, b.max_context_len, scale=b.scale, out=out)

    def plain_step(i):
        kp, vp = pools[i & 1]
        pa.kv_write(new_k, new_v, slots, kp, vp)
        pa.decode(q, kp, vp, tables, lens, b.max_context_len, scale=b.scale, out=out)

    log(f"[bench] timing the fused write ({args.steps} calls)")
    f_us = float(np.median(time_calls(fused, args.steps, args.warmup)))
    res = {"metric": "pa_qkv_rope_write GB/s (fused QKV split + rotary + KV write)",
           "value": round(fused_write_bytes(b) / (f_us * 1e-6) / 1e9, 1), "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(f_us * 1e-3, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": b.dtype,
           "data": "synthetic",
           "config": {"workload": b.name, "tokens": int(b.q.shape[0]), "rope_theta": theta,
                      "qk_norm": True, "bytes": fused_write_bytes(b)},
           "fused_write_us": round(f_us, 2)}
    if qsl is None:
        res["decode_step_us"] = {
            "fused_write_plus_decode": round(float(np.median(time_calls(fused_step, args.steps, args.warmup))), 2),
            "kv_write_plus_decode": round(float(np.median(time_calls(plain_step, args.steps, args.warmup))), 2)}
    return res


def bench_shared_prefix(args, b, up) -> dict:
    """A decode step on a batch whose sequences share a prompt prefix (one
    group, the generator's shared blocks): KV write + pa_decode_shared_prefix,
    beside KV write + pa_decode on the same inputs.  Both attention calls are
    timed with HIP events; the rate counts the shared blocks once."""
    import numpy as np
    import torch

    import paged_kv_attention_22_amd as pa
    if b.shared_prefix_tokens <= 0:
        raise SystemExit("bench.py: --op shared_prefix needs a workload with a shared prefix (long_context)")
    pools = [(up(b.k_pool), up(b.v_pool)) for _ in range(2)]
    q, new_k, new_v, slots = up(b.q), up(b.new_k), up(b.new_v), up(b.slot_mapping)
    tables, lens = up(b.block_tables), up(b.context_lens)
    S, P = b.num_seqs, b.shared_prefix_tokens
    gs = torch.tensor([0, S], dtype=torch.int32, device=q.device)
    pl = torch.tensor([P], dtype=torch.int32, device=q.device)
    out = torch.empty_like(q)
    need = pa.decode_shared_prefix_workspace_bytes(S, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                                   b.max_context_len, 1, S, P, args.partition)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dws = torch.empty(max(pa.decode_workspace_bytes(S, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                                    b.max_context_len, args.partition), 1),
                      dtype=torch.uint8, device=q.device)

    def shared(i):
        kp, vp = pools[i & 1]
        pa.decode_shared_prefix(q, kp, vp, tables, lens, b.max_context_len, gs, pl, S, P, scale=b.scale,
                                out=out, partition_tokens=args.partition, workspace=ws)

    def plain(i):
        kp, vp = pools[i & 1]
        pa.decode(q, kp, vp, tables, lens, b.max_context_len, scale=b.scale, out=out,
                  partition_tokens=args.partition, workspace=dws)

    def step(i):
        kp, vp = pools[i & 1]
        pa.kv_write(new_k, new_v, slots, kp, vp)
        shared(i)

    log(f"[bench] timing pa_decode_shared_prefix and pa_decode ({args.steps} calls each)")
    s_us = time_calls(shared, args.steps, args.warmup)
    p_us = time_calls(plain, args.steps, args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    dbytes, wbytes = decode_bytes(b), kv_write_bytes(b)
    mean_s = float(np.mean(s_us)) * 1e-6
    achieved = dbytes / mean_s / 1e9
    return {
        "metric": "pa_decode_shared_prefix HBM GB/s on unique K/V bytes (shared prefix read once)",
        "value": round((dbytes + wbytes) / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": b.dtype,
        "data": "synthetic",
        "config": {"workload": b.name, "recipe": b.recipe, "seed": b.seed, "num_seqs": S,
                   "num_q_heads": b.num_q_heads, "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                   "block_size": int(b.k_pool.shape[1]), "shared_prefix_tokens": P,
                   "max_context": b.max_context_len,
                   "step": "pa_kv_write + pa_decode_shared_prefix (one group of every sequence)"},
        "shared_prefix_us": {"mean": round(mean_s * 1e6, 2), "median": round(float(np.median(s_us)), 2),
                             "p10": round(float(np.percentile(s_us, 10)), 2),
                             "p90": round(float(np.percentile(s_us, 90)), 2)},
        "pa_decode_us": {"mean": round(float(np.mean(p_us)), 2), "median": round(float(np.median(p_us)), 2)},
        "roofline": {"kernel": "pa_decode_shared_prefix call: prefix chunk kernel, then the decode kernel folding its "
                                 "partial states in (with a split context: both side by side, then the merge)",
                     "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes": dbytes},
        "cpu_baseline": None,
    }


def copy_reference(steps: int) -> dict:
    """What a plain streaming kernel reaches on the same GPU in the same run:
    torch's elementwise int32 multiply over 1 GiB (1 GiB read + 1 GiB
    written), timed like the decode calls.  Context for the roofline fraction,
    not part of it (the fraction stays against the 8 TB/s published peak)."""
    import numpy as np
    import torch
    x = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    us = time_calls(lambda i: torch.mul(x, 1, out=y), max(steps, 10), 10)
    del x, y
    gbs = 2 * (1 << 30) / (float(np.mean(us)) * 1e-6) / 1e9
    return {"kernel": "torch.mul int32, 1 GiB read + 1 GiB written", "us": round(float(np.mean(us)), 2),
            "gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


# What the oracle workers read: the batch and the pools after the step's KV
# write (set before the pool forks, so each worker sees them without a copy).
_ORACLE_INPUT = None


def _oracle_rows(b, kp, vp, seqs=None):
    """The oracle's attention over the written pools for the given sequences
    (all of them by default): their query rows (one per decode sequence, a
    chunk's rows for a prefill sequence), their tables and lengths."""
    import numpy as np

    import oracle
    qsl = np.asarray(b.query_start_loc)
    if seqs is None:
        return oracle.attention(b.q, qsl, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
    rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs])
    sub_qsl = np.concatenate([[0], np.cumsum([qsl[s + 1] - qsl[s] for s in seqs])])
    return oracle.attention(b.q[rows], sub_qsl, kp, vp, b.block_tables[seqs], b.context_lens[seqs],
                            b.scale, b.dtype)


def _oracle_part(seqs):
    """Worker of the all-cores oracle leg: attention of the given sequences
    over the written pools (the oracle as it stands, one BLAS thread per
    worker)."""
    from threadpoolctl import threadpool_limits

    b, kp, vp = _ORACLE_INPUT
    with threadpool_limits(1):
        _oracle_rows(b, kp, vp, seqs)
    return len(seqs)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(b, min_seconds: float = 8.0) -> dict:
    """The fp64 oracle on the same step (KV write + attention of every
    sequence's query rows: one per decode sequence, a chunk's rows for a
    prefill sequence),
    timed on the host in two legs: one core (one BLAS thread), and every core
    this process may run on (the KV write in this process, then the decode on
    a pool of that many worker processes with the sequences dealt round-robin
    to them).  Each leg repeats whole passes over the batch until at least
    min_seconds have passed.  Runs before the GPU is touched, so the pool forks
    a process with no GPU state."""
    import multiprocessing

    from threadpoolctl import threadpool_limits

    import oracle
    global _ORACLE_INPUT
    nbytes = decode_bytes(b) + kv_write_bytes(b)
    passes, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            kp, vp = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
            _oracle_rows(b, kp, vp)
            passes += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    dt1 = (time.perf_counter() - t0) / passes
    ncores = len(os.sched_getaffinity(0))
    parts = [list(range(w, b.num_seqs, ncores)) for w in range(ncores)]
    parts = [p for p in parts if p]
    kp, vp = oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
    _ORACLE_INPUT = (b, kp, vp)
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(len(parts)) as pool:
        passes_n, t0 = 0, time.perf_counter()
        while True:
            # the write again (the workers read the copy made before they
            # forked, which holds the same values), then the parallel attention
            oracle.kv_write(b.k_pool, b.v_pool, b.new_k, b.new_v, b.slot_mapping)
            assert sum(pool.map(_oracle_part, parts, chunksize=1)) == b.num_seqs
            passes_n += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
        dtn = (time.perf_counter() - t0) / passes_n
    _ORACLE_INPUT = None
    del kp, vp
    model = cpu_model()
    return {"value": round(nbytes / dtn / 1e9, 4), "unit": "GB/s", "cores": len(parts), "kind": "oracle",
            "seq_steps_per_s": round(b.num_seqs / dtn, 2), "seconds_per_pass": round(dtn, 6),
            "cpu_model": model, "affinity_cores": ncores,
            "one_core": {"value": round(nbytes / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "seq_steps_per_s": round(b.num_seqs / dt1, 2), "seconds_per_pass": round(dt1, 6),
                         "passes": passes},
            "sample": f"whole batch ({b.num_seqs} seqs), KV write + attention, numpy fp64: {passes_n} pass(es) "
                      f"with the attention on {len(parts)} worker processes (sequences dealt round-robin, one BLAS "
                      f"thread each) after the write, and {passes} pass(es) on one core; CPU: {model}"}


# hipDeviceAttribute_t values (HIP 7 runtime): global memory bus width in
# bits, peak memory clock in kHz, peak core clock in kHz.
_HIP_ATTR_MEMORY_BUS_WIDTH, _HIP_ATTR_MEMORY_CLOCK_RATE, _HIP_ATTR_CLOCK_RATE = 59, 60, 5


def device_memory_props(dev_index: int) -> dict:
    """The device's reported memory bus width and clocks (from the HIP runtime
    torch has loaded), as context beside the published 8 TB/s the roofline
    uses.  No peak is derived from them: the runtime does not state how many
    transfers per pin it counts in one reported memory clock."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    out = {}
    for name, attr in (("memory_bus_width_bits", _HIP_ATTR_MEMORY_BUS_WIDTH),
                       ("memory_clock_khz", _HIP_ATTR_MEMORY_CLOCK_RATE), ("core_clock_khz", _HIP_ATTR_CLOCK_RATE)):
        v = ctypes.c_int(0)
        rc = hip.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(attr), ctypes.c_int(dev_index))
        out[name] = v.value if rc == 0 else None
    out["published_peak_gbs"] = HBM_PEAK_GBS
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 20 ms of untimed work by default: the clocks are still rising over
    # the first few milliseconds of load (measured: a timed loop right after 5
    # steps ran ~2% slower than the same loop later)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--partition", type=int, default=0,
                    help="partition_tokens for pa_decode (0 = library choice, -1 = one pass)")
    ap.add_argument("--workload", default="qwen3_06b_decode",
                    help="generator preset (default: the Qwen3-0.6B batch-256 decode step)")
    ap.add_argument("--op", default="step", choices=["step", "fused_write", "shared_prefix"],
                    help="step: the workload's attention step (default); fused_write: "
                         "pa_qkv_rope_write on the workload's new tokens; shared_prefix: "
                         "pa_decode_shared_prefix on a workload whose sequences share a prefix")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32],
                    help="tokens per pool block (16 is the pages' choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the headline decode's traffic record from two rocprofv3 --pmc counter CSVs "
                         "(FETCH_SIZE, WRITE_SIZE) and exit; uses no GPU")
    ap.add_argument("--copy-first", action="store_true",
                    help="run the plain 1 GiB copy three times before the benchmark, in the same process, "
                         "so one counter run reads both (the copy's bytes are known)")
    args = ap.parse_args()
    if args.traffic_record:
        print(json.dumps(traffic_record(*args.traffic_record), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(no multi-GPU path is built)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_attention_22_amd as pa
    from workloads import PRESETS

    if args.calibrate_copy or args.copy_first:
        # An elementwise kernel that reads 1 GiB and writes 1 GiB: the
        # counters' readings for it convert counter units to bytes.
        x = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1, out=y)
        torch.cuda.synchronize()
        del x, y
        if args.calibrate_copy:
            print(json.dumps({"calibration": "torch.mul int32, 1 GiB read + 1 GiB written per launch",
                              "launches": 3}))
            return 0

    if not os.path.exists(pa.LIB_PATH):
        from paged_kv_attention_22_amd import build as pa_build
        pa_build.build()

    log(f"[bench] generating {args.workload}")
    b = PRESETS[args.workload](**({} if args.block_size == 16 else {"block_size": args.block_size}))
    baseline = None
    if args.op == "step" and not args.no_cpu_baseline and not args.copy_first:
        # before anything touches the GPU: the oracle's worker pool forks
        log("[bench] timing the fp64 oracle on the host (one core, then every core)")
        baseline = cpu_baseline(b)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"[bench] device {props.name}, {props.multi_processor_count} CUs, "
        f"{props.total_memory / 2**30:.0f} GiB")

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    if args.op == "fused_write":
        print(json.dumps(bench_fused(args, b, up)), flush=True)
        return 0
    if args.op == "shared_prefix":
        print(json.dumps(bench_shared_prefix(args, b, up)), flush=True)
        return 0
    if b.num_prefill_seqs:
        res = bench_mixed(args, b, up, dev)
        if baseline is not None:
            # the mixed step's metric is a time: the oracle's, per whole pass
            baseline = dict(baseline, value=round(baseline["seconds_per_pass"] * 1e6, 1), unit="us",
                            higher_is_better=False,
                            one_core=dict(baseline["one_core"],
                                          value=round(baseline["one_core"]["seconds_per_pass"] * 1e6, 1),
                                          unit="us"))
        res["cpu_baseline"] = baseline
        print(json.dumps(res), flush=True)
        return 0

    pools = [(up(b.k_pool), up(b.v_pool)) for _ in range(2)]
    q, new_k, new_v = up(b.q), up(b.new_k), up(b.new_v)
    slots, tables, lens = up(b.slot_mapping), up(b.block_tables), up(b.context_lens)
    out = torch.empty_like(q)
    part = pa.decode_partition_tokens(b.num_seqs, b.num_kv_heads, b.head_dim, b.max_context_len, args.partition)
    ws_bytes = pa.decode_workspace_bytes(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                         b.max_context_len, args.partition)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step(i):
        # the step's KV write fused into the decode launch
        kp, vp = pools[i & 1]
        pa.decode_append(q, new_k, new_v, kp, vp, tables, lens, b.max_context_len, scale=b.scale, out=out,
                         partition_tokens=args.partition, workspace=ws)

    def two_call_step(i, t=None):
        kp, vp = pools[i & 1]
        pa.kv_write(new_k, new_v, slots, kp, vp)
        if t is not None:
            t.start(i)
        pa.decode(q, kp, vp, tables, lens, b.max_context_len, scale=b.scale, out=out,
                  partition_tokens=args.partition, workspace=ws)
        if t is not None:
            t.stop(i)

    log(f"[bench] warmup {args.warmup} steps (partition_tokens={part})")
    for i in range(args.warmup):
        step(i)
        two_call_step(i)
    torch.cuda.synchronize()
    # Whole steps, back to back between two synchronisations, nothing else on
    # the stream: first as two calls (pa_kv_write, then pa_decode), then
    # fused (the step throughput, value).
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        two_call_step(i)
    torch.cuda.synchronize()
    wall_two = time.perf_counter() - t0
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The two-call steps again with fence-free HIP events around each
    # pa_decode call: the decode duration (roofline).
    timer = Timer(args.steps)
    for i in range(args.steps):
        two_call_step(i, timer)
    torch.cuda.synchronize()
    dec_ms = [timer.us(i) * 1e-3 for i in range(args.steps)]
    timer.close()
    log(f"[bench] done: {wall * 1e3 / args.steps:.3f} ms/step ({wall_two * 1e3 / args.steps:.3f} as two calls), "
        f"decode median {float(np.median(dec_ms)) * 1e3:.1f} us")

    ms_per_step = wall * 1e3 / args.steps
    dbytes, wbytes = decode_bytes(b), kv_write_bytes(b)
    value = (dbytes + wbytes) / (ms_per_step * 1e-3) / 1e9
    dec_mean_s = float(np.mean(dec_ms)) * 1e-3
    achieved = dbytes / dec_mean_s / 1e9
    traffic = measured_traffic(part, int(b.k_pool.shape[1]), b.name)
    result = {
        "metric": METRIC if b.name == "qwen3_06b_decode" else f"pa_decode HBM GB/s (% of peak) + seq-steps/s, {b.name}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.dtype,
        "data": "synthetic",
        "config": {
            "workload": b.name, "recipe": b.recipe, "seed": b.seed, "num_seqs": b.num_seqs,
            "num_q_heads": b.num_q_heads, "num_kv_heads": b.num_kv_heads,
            "head_dim": b.head_dim, "block_size": int(b.k_pool.shape[1]), "num_blocks": b.num_blocks,
            "mean_context": round(float(b.context_lens.mean()), 2),
            "max_context": b.max_context_len, "partition_tokens": part,
            "step": "pa_decode_append: the KV write of one new token per sequence fused into pa_decode",
        },
        "two_call_step": {"ms_per_step": round(wall_two * 1e3 / args.steps, 5),
                          "value": round((dbytes + wbytes) / (wall_two / args.steps) / 1e9, 2),
                          "calls": "pa_kv_write + pa_decode"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(b.num_seqs / (ms_per_step * 1e-3), 1),
        "decode_us": {"mean": round(dec_mean_s * 1e6, 2),
                      "median": round(float(np.median(dec_ms)) * 1e3, 2),
                      "p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                      "p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2)},
        "roofline": {
            "kernel": ("pa_decode call: attention kernel (split partials) + merge kernel" if part > 0
                       else "pa_decode call: one attention kernel (one pass, longest first, ranked in-kernel)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": dbytes,
            "logical_kv_bytes": int(b.context_lens.sum()) * 2 * b.num_kv_heads * b.head_dim * b.elem_bytes,
        },
        "cpu_baseline": None,
    }
    result["copy_reference"] = copy_reference(args.steps)
    result["device_memory"] = device_memory_props(dev.index or 0)
    result["cpu_baseline"] = baseline
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
