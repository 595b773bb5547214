"""Paged-KV attention for MI355X (gfx950): Python binding of libpa.so.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/pa.h.  PyTorch supplies device memory and the current
stream.  If libpa.so is missing the calls raise; there is no fallback.

    import paged_kv_attention_22_amd as pa
    pa.kv_write(k, v, slot_mapping, k_pool, v_pool)
    out = pa.decode(q, k_pool, v_pool, block_tables, context_lens, max_context_len)
    out = pa.prefill_chunk(q, query_start_loc, num_prefill_seqs, max_query_len,
                           k_pool, v_pool, block_tables, context_lens, max_context_len)
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
BLOCK_SIZE = 16

PA_OK, PA_F32, PA_BF16, PA_F16 = 0, 0, 1, 2
PA_ERR_SHAPE, PA_ERR_WORKSPACE, PA_ERR_CAPACITY, PA_ERR_STREAM, PA_ERR_SCRATCH = 2, 5, 8, 9, 10

c_i32, c_i64, c_size, c_vp, c_f = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_float)


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", c_i32), ("block_size", c_i32), ("num_kv_heads", c_i32),
                ("head_dim", c_i32), ("dtype", c_i32)]


class AuxStream(ctypes.Structure):
    """pa_aux_stream: a second stream and fork/join events owned by the caller."""
    _fields_ = [("stream", c_vp), ("fork_event", c_vp), ("join_event", c_vp)]


class PAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


_SIGNATURES = {
    "pa_status_str": (ctypes.c_char_p, [c_i32]),
    "pa_kv_write": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_vp, c_i32, c_vp, c_vp, PoolDesc, c_vp]),
    "pa_decode_partition_tokens": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode": (c_i32, [c_vp, c_vp, c_vp, PoolDesc, c_vp, c_i32, c_vp, c_i32, c_i32, c_i32,
                          c_f, c_vp, c_i32, c_vp, c_size, c_vp]),
    "pa_decode_noalloc": (c_i32, [c_vp, c_vp, c_vp, PoolDesc, c_vp, c_i32, c_vp, c_i32, c_i32, c_i32,
                                  c_f, c_vp, c_i32, c_vp]),
    "pa_decode_append": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, PoolDesc, c_vp, c_i32, c_vp,
                                 c_i32, c_i32, c_i32, c_f, c_vp, c_i32, c_vp, c_size, c_vp]),
    "pa_decode_shared_prefix_workspace_bytes": (c_size, [c_i32] * 9),
    "pa_decode_shared_prefix": (c_i32, [c_vp, c_vp, c_vp, PoolDesc, c_vp, c_i32, c_vp, c_i32, c_i32,
                                        c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_f, c_vp, c_i32,
                                        c_vp, c_size, c_vp, ctypes.POINTER(AuxStream)]),
    "pa_qkv_rope_write": (c_i32, [c_vp, c_i64, c_vp, c_i32, c_i32, c_vp, c_vp, c_i32, c_i32, c_f,
                                  c_vp, c_vp, c_f, c_vp, c_vp, c_vp, PoolDesc, c_vp, c_vp]),
    "pa_prefill_workspace_bytes": (c_size, [c_i32] * 8),
    "pa_bm_create": (c_vp, [c_i32, c_i32, c_i32]),
    "pa_bm_destroy": (None, [c_vp]),
    "pa_bm_add_sequence": (c_i32, [c_vp, c_i64, c_vp, c_i32, c_vp]),
    "pa_bm_append": (c_i32, [c_vp, c_i64, c_vp, c_i32, c_vp]),
    "pa_bm_mark_computed": (c_i32, [c_vp, c_i64, c_i32]),
    "pa_bm_free_sequence": (c_i32, [c_vp, c_i64]),
    "pa_bm_block_table": (c_i32, [c_vp, c_i64, c_vp, c_i32, c_vp, c_vp]),
    "pa_bm_num_free_blocks": (c_i32, [c_vp]),
    "pa_bm_stats": (c_i32, [c_vp, c_vp, c_vp, c_vp]),
    "pa_bm_block_refcount": (c_i32, [c_vp, c_i32]),
    "pa_prefill_chunk": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, PoolDesc,
                                 c_vp, c_i32, c_vp, c_i32, c_i32, c_f, c_vp, c_i32, c_vp,
                                 c_size, c_vp, ctypes.POINTER(AuxStream)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libpa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m paged_kv_attention_22_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().pa_status_str(status).decode()


def _check(status: int, what: str) -> None:
    if status != PA_OK:
        raise PAError(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float16:
        return PA_F16
    if t.dtype == torch.float32:
        return PA_F32
    raise TypeError(f"unsupported element type {t.dtype} (bf16, fp16 or fp32)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _contig(t: torch.Tensor, name: str) -> int:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _dev(t, name)


def _i32(t: torch.Tensor, name: str) -> int:
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return _contig(t, name)


def pool_desc(k_pool: torch.Tensor) -> PoolDesc:
    nb, bs, hkv, d = k_pool.shape
    return PoolDesc(nb, bs, hkv, d, _dtype_code(k_pool))


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on(stream):
    """Allocations for a call made on `stream`: torch's allocator then keeps
    a block (workspace, default output) for that stream's work, instead of
    handing it back to the current stream while the call's kernels still use
    it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


class _AuxPerThread(threading.local):
    def __init__(self):
        self.by_device = {}


_aux = _AuxPerThread()


def aux_stream(device=None):
    """This host thread's second stream and fork/join events on `device`
    (created on first use, default priority), as the pa_aux_stream that
    prefill_chunk and decode_shared_prefix pass by default.  One per thread,
    so calls from several threads never share one.  Returns (stream,
    AuxStream)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    ent = _aux.by_device.get(idx)
    if ent is None:
        with torch.cuda.device(idx):
            s = torch.cuda.Stream()
            fork, join = torch.cuda.Event(), torch.cuda.Event()  # timing disabled
            fork.record(s)  # torch creates an event at its first record
            join.record(s)
        ent = (s, fork, join, AuxStream(s.cuda_stream, fork.cuda_event, join.cuda_event))
        _aux.by_device[idx] = ent
    return ent[0], ent[3]


def _aux_arg(aux, device):
    """aux: True = this thread's aux_stream(device), False/None = run on the
    call's stream alone, or an AuxStream."""
    if aux is True:
        return ctypes.pointer(aux_stream(device)[1])
    if aux is False or aux is None:
        return None
    if isinstance(aux, AuxStream):
        return ctypes.pointer(aux)
    raise TypeError("aux must be True, False, None or an AuxStream")


def kv_write(k, v, slot_mapping, k_pool, v_pool, stream=None) -> None:
    """Scatter rows k[t], v[t] ([T, Hkv, D], token stride free) to pool row
    slot_mapping[t]; negative slots are skipped."""
    for name, t in (("k", k), ("v", v)):
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{name} must be [T, Hkv, D] with contiguous token rows")
    if k.dtype != k_pool.dtype or v.dtype != v_pool.dtype:
        raise TypeError("k/v and pools must share an element type")
    st = lib().pa_kv_write(_dev(k, "k"), _dev(v, "v"), k.stride(0), v.stride(0),
                           _i32(slot_mapping, "slot_mapping"), slot_mapping.numel(),
                           _contig(k_pool, "k_pool"), _contig(v_pool, "v_pool"),
                           pool_desc(k_pool), _stream(stream))
    _check(st, "pa_kv_write")


def qkv_rope_write(qkv, num_q_heads, context_lens, block_tables, k_pool, v_pool, rope_theta,
                   query_start_loc=None, q_norm=None, k_norm=None, eps=1e-6, q_out=None,
                   slot_mapping_out=None, stream=None):
    """Packed projection rows qkv [T, >= (Hq + 2*Hkv) * D] -> rotated q [T, Hq, D];
    rotated k and v stored in the pools at slots derived from the tables.
    query_start_loc None: one token per sequence."""
    if qkv.dim() != 2 or qkv.stride(1) != 1:
        raise ValueError("qkv must be [T, width] with contiguous rows")
    if qkv.dtype != k_pool.dtype:
        raise TypeError("qkv and pools must share an element type")
    T = qkv.shape[0]
    S = context_lens.shape[0]
    D = k_pool.shape[3]
    if q_out is None:
        with _on(stream):
            q_out = torch.empty((T, num_q_heads, D), dtype=qkv.dtype, device=qkv.device)
    qsl = 0 if query_start_loc is None else _i32(query_start_loc, "query_start_loc")
    qn = 0 if q_norm is None else _contig(q_norm, "q_norm")
    kn = 0 if k_norm is None else _contig(k_norm, "k_norm")
    so = 0 if slot_mapping_out is None else _i32(slot_mapping_out, "slot_mapping_out")
    st = lib().pa_qkv_rope_write(_dev(qkv, "qkv"), qkv.stride(0), qsl, T, S,
                                 _i32(context_lens, "context_lens"), _i32(block_tables, "block_tables"),
                                 block_tables.shape[1], int(num_q_heads), float(rope_theta), qn, kn,
                                 float(eps), _contig(q_out, "q_out"), _contig(k_pool, "k_pool"),
                                 _contig(v_pool, "v_pool"), pool_desc(k_pool), so, _stream(stream))
    _check(st, "pa_qkv_rope_write")
    return q_out


def decode_partition_tokens(num_seqs, num_kv_heads, head_dim, max_context_len, partition_tokens=0) -> int:
    return lib().pa_decode_partition_tokens(num_seqs, num_kv_heads, head_dim, max_context_len,
                                            partition_tokens)


def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                           partition_tokens=0) -> int:
    return lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           max_context_len, partition_tokens)


def prefill_workspace_bytes(num_seqs, num_prefill_seqs, total_query_tokens, num_q_heads,
                            num_kv_heads, head_dim, max_context_len, partition_tokens=0) -> int:
    return lib().pa_prefill_workspace_bytes(num_seqs, num_prefill_seqs, total_query_tokens,
                                            num_q_heads, num_kv_heads, head_dim,
                                            max_context_len, partition_tokens)


def _workspace(nbytes: int, workspace, device):
    """The caller's workspace, or a new one of nbytes (None when none is
    needed); allocate under _on(stream)."""
    if nbytes == 0:
        return None
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace


def _ws_ptr(workspace) -> tuple[int, int]:
    if workspace is None:
        return 0, 0
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def decode(q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale=None,
           out=None, partition_tokens=0, workspace=None, stream=None):
    """Batched decode attention, q [S, Hq, D] -> out [S, Hq, D]."""
    S, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    hkv = k_pool.shape[2]
    need = decode_workspace_bytes(S, Hq, hkv, D, max_context_len, partition_tokens)
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        ws = _workspace(need, workspace, q.device)
    wp, wb = _ws_ptr(ws)
    st = lib().pa_decode(_contig(q, "q"), _contig(k_pool, "k_pool"), _contig(v_pool, "v_pool"),
                         pool_desc(k_pool), _i32(block_tables, "block_tables"),
                         block_tables.shape[1], _i32(context_lens, "context_lens"), S,
                         int(max_context_len), Hq, float(scale), _contig(out, "out"),
                         int(partition_tokens), wp, wb, _stream(stream))
    _check(st, "pa_decode")
    return out


def decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale=None,
                   out=None, partition_tokens=0, stream=None):
    """decode() through pa_decode_noalloc: the library's per-device scratch
    array instead of a workspace; `out` must be given by a caller that
    cannot allocate."""
    S, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        with _on(stream):
            out = torch.empty_like(q)
    st = lib().pa_decode_noalloc(_contig(q, "q"), _contig(k_pool, "k_pool"), _contig(v_pool, "v_pool"),
                                 pool_desc(k_pool), _i32(block_tables, "block_tables"), block_tables.shape[1],
                                 _i32(context_lens, "context_lens"), S, int(max_context_len), Hq, float(scale),
                                 _contig(out, "out"), int(partition_tokens), _stream(stream))
    _check(st, "pa_decode_noalloc")
    return out


def decode_append(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, max_context_len, scale=None,
                  out=None, partition_tokens=0, workspace=None, stream=None):
    """Decode step with the KV write fused in: sequence s's new K/V rows
    (k_new[s], v_new[s]: [S, Hkv, D], token stride free) are stored at the pool
    slot of position context_lens[s] - 1 and attended; same pools and output
    as kv_write (slots of those positions) followed by decode()."""
    S, Hq, D = q.shape
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dim() != 3 or t.shape[0] != S or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{name} must be [S, Hkv, D] with contiguous token rows")
    if k_new.dtype != k_pool.dtype or v_new.dtype != v_pool.dtype:
        raise TypeError("k_new/v_new and pools must share an element type")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    hkv = k_pool.shape[2]
    need = decode_workspace_bytes(S, Hq, hkv, D, max_context_len, partition_tokens)
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        ws = _workspace(need, workspace, q.device)
    wp, wb = _ws_ptr(ws)
    st = lib().pa_decode_append(_contig(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), k_new.stride(0),
                                v_new.stride(0), _contig(k_pool, "k_pool"), _contig(v_pool, "v_pool"),
                                pool_desc(k_pool), _i32(block_tables, "block_tables"), block_tables.shape[1],
                                _i32(context_lens, "context_lens"), S, int(max_context_len), Hq, float(scale),
                                _contig(out, "out"), int(partition_tokens), wp, wb, _stream(stream))
    _check(st, "pa_decode_append")
    return out


def decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                         num_groups, max_group_size, max_prefix_len,
                                         partition_tokens=0) -> int:
    return lib().pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                         max_context_len, num_groups, max_group_size,
                                                         max_prefix_len, partition_tokens)


def decode_shared_prefix(q, k_pool, v_pool, block_tables, context_lens, max_context_len, group_start,
                         prefix_lens, max_group_size, max_prefix_len, scale=None, out=None,
                         partition_tokens=0, workspace=None, stream=None, aux=True):
    """Decode attention for groups of sequences sharing a prompt prefix:
    group g is sequences group_start[g] .. group_start[g+1]-1 (int32 device
    tensor [G+1]) sharing their first prefix_lens[g] tokens (int32 device
    [G]).  Same result as decode() within rounding.  aux: see _aux_arg (by
    default the prefix phase runs on this thread's second stream)."""
    S, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    hkv = k_pool.shape[2]
    ng = group_start.shape[0] - 1
    need = decode_shared_prefix_workspace_bytes(S, Hq, hkv, D, max_context_len, ng, max_group_size,
                                                max_prefix_len, partition_tokens)
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        ws = _workspace(need, workspace, q.device)
    wp, wb = _ws_ptr(ws)
    st = lib().pa_decode_shared_prefix(_contig(q, "q"), _contig(k_pool, "k_pool"), _contig(v_pool, "v_pool"),
                                       pool_desc(k_pool), _i32(block_tables, "block_tables"),
                                       block_tables.shape[1], _i32(context_lens, "context_lens"), S,
                                       int(max_context_len), _i32(group_start, "group_start"),
                                       _i32(prefix_lens, "prefix_lens"), ng, int(max_group_size),
                                       int(max_prefix_len), Hq, float(scale), _contig(out, "out"),
                                       int(partition_tokens), wp, wb, _stream(stream), _aux_arg(aux, q.device))
    _check(st, "pa_decode_shared_prefix")
    return out


def prefill_chunk(q, query_start_loc, num_prefill_seqs, max_query_len, k_pool, v_pool,
                  block_tables, context_lens, max_context_len, scale=None, out=None,
                  partition_tokens=0, workspace=None, stream=None, aux=True):
    """Causal attention for a packed mixed batch, q [T, Hq, D] -> out [T, Hq, D].
    aux: see _aux_arg (by default the decode rows run on this thread's second
    stream beside the matrix-core chunks)."""
    T, Hq, D = q.shape
    S = context_lens.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    hkv = k_pool.shape[2]
    need = prefill_workspace_bytes(S, num_prefill_seqs, T, Hq, hkv, D, max_context_len,
                                   partition_tokens)
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        ws = _workspace(need, workspace, q.device)
    wp, wb = _ws_ptr(ws)
    st = lib().pa_prefill_chunk(_contig(q, "q"), _i32(query_start_loc, "query_start_loc"), T, S,
                                int(num_prefill_seqs), int(max_query_len),
                                _contig(k_pool, "k_pool"), _contig(v_pool, "v_pool"),
                                pool_desc(k_pool), _i32(block_tables, "block_tables"),
                                block_tables.shape[1], _i32(context_lens, "context_lens"),
                                int(max_context_len), Hq, float(scale), _contig(out, "out"),
                                int(partition_tokens), wp, wb, _stream(stream), _aux_arg(aux, q.device))
    _check(st, "pa_prefill_chunk")
    return out


class BlockManager:
    """Host-side block pool, block tables and prefix cache (pa_bm_* calls).

    Token ids and slots travel as int32 numpy arrays; nothing here touches the
    GPU.  The tables it hands out are what pa_decode / pa_prefill_chunk and
    pa_qkv_rope_write read (after a copy to the device)."""

    def __init__(self, num_blocks: int, block_size: int = 16, prefix_caching: bool = True):
        self._h = lib().pa_bm_create(int(num_blocks), int(block_size), int(bool(prefix_caching)))
        if not self._h:
            raise PAError(PA_ERR_SHAPE, "pa_bm_create")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self) -> None:
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _arr(tokens):
        import numpy as np
        a = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        return a, a.ctypes.data if a.size else 0

    def add_sequence(self, seq_id: int, prompt) -> int:
        """Register a sequence and its prompt; returns the prompt tokens found in the cache."""
        a, p = self._arr(prompt)
        cached = ctypes.c_int32(0)
        _check(lib().pa_bm_add_sequence(self._h, int(seq_id), p, a.size, ctypes.byref(cached)),
               "pa_bm_add_sequence")
        return cached.value

    def append(self, seq_id: int, tokens):
        """Add tokens; returns their flat slots (int32 numpy array)."""
        import numpy as np
        a, p = self._arr(tokens)
        slots = np.zeros(a.size, np.int32)
        _check(lib().pa_bm_append(self._h, int(seq_id), p, a.size, slots.ctypes.data if a.size else 0),
               "pa_bm_append")
        return slots

    def mark_computed(self, seq_id: int, num_tokens: int) -> None:
        _check(lib().pa_bm_mark_computed(self._h, int(seq_id), int(num_tokens)), "pa_bm_mark_computed")

    def free(self, seq_id: int) -> None:
        _check(lib().pa_bm_free_sequence(self._h, int(seq_id)), "pa_bm_free_sequence")

    def block_table(self, seq_id: int):
        """(block ids as an int32 numpy array, number of tokens)."""
        import numpy as np
        nb, nt = ctypes.c_int32(0), ctypes.c_int32(0)
        out = np.zeros(self.num_blocks, np.int32)
        _check(lib().pa_bm_block_table(self._h, int(seq_id), out.ctypes.data, out.size,
                                       ctypes.byref(nb), ctypes.byref(nt)), "pa_bm_block_table")
        return out[:nb.value].copy(), nt.value

    def num_free_blocks(self) -> int:
        return lib().pa_bm_num_free_blocks(self._h)

    def refcount(self, block_id: int) -> int:
        return lib().pa_bm_block_refcount(self._h, int(block_id))

    def stats(self) -> dict:
        h, q, c = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int32(0)
        _check(lib().pa_bm_stats(self._h, ctypes.byref(h), ctypes.byref(q), ctypes.byref(c)), "pa_bm_stats")
        return {"hit_blocks": h.value, "queried_blocks": q.value, "cached_blocks": c.value}
