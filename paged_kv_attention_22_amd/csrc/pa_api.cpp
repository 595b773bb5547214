// C ABI of the library: host-side validation, path choice and launch.
// Nothing here touches the GPU before every argument has been checked, and
// nothing reads device memory: sizes come in as host integers.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "pa_internal.hpp"

using namespace pa;

namespace {

// The caller's second stream for a call that runs two kernels side by side
// (pa_prefill_chunk: decode rows beside the matrix-core chunk kernel;
// pa_decode_shared_prefix: the prefix phase beside the decode kernel).  NULL
// means no second stream: the call then enqueues everything on its own
// stream, in an order that needs no second one.  The library keeps nothing:
// the stream and both events belong to the caller for as long as the caller
// likes.
int32_t check_aux(const pa_aux_stream* aux, hipStream_t s) {
    if (aux == nullptr) return PA_OK;
    if (aux->stream == nullptr || aux->fork_event == nullptr || aux->join_event == nullptr)
        return PA_ERR_STREAM;
    hipStream_t x = static_cast<hipStream_t>(aux->stream);
    if (x == s) return PA_ERR_STREAM;
    int dev_s = 0, dev_x = 0;
    if (s != nullptr) {
        if (hipStreamGetDevice(s, &dev_s) != hipSuccess) return PA_ERR_STREAM;
    } else if (hipGetDevice(&dev_s) != hipSuccess) {
        return PA_ERR_STREAM;
    }
    if (hipStreamGetDevice(x, &dev_x) != hipSuccess || dev_x != dev_s) return PA_ERR_STREAM;
    return PA_OK;
}

// Work enqueued on s before this point is also ordered before what is
// enqueued on the auxiliary stream after it.
int32_t fork_to(const pa_aux_stream& aux, hipStream_t s) {
    hipEvent_t e = static_cast<hipEvent_t>(aux.fork_event);
    if (hipEventRecord(e, s) != hipSuccess) return PA_ERR_LAUNCH;
    return hipStreamWaitEvent(static_cast<hipStream_t>(aux.stream), e, 0) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// Work enqueued on s after this point waits for what the auxiliary stream
// holds now.
int32_t join_from(const pa_aux_stream& aux, hipStream_t s) {
    hipEvent_t e = static_cast<hipEvent_t>(aux.join_event);
    if (hipEventRecord(e, static_cast<hipStream_t>(aux.stream)) != hipSuccess) return PA_ERR_LAUNCH;
    return hipStreamWaitEvent(s, e, 0) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int elem_size(int32_t dtype) {
    if (dtype == PA_BF16 || dtype == PA_F16) return 2;
    if (dtype == PA_F32) return 4;
    return 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// log2 of a supported pool block size (8, 16 or 32 tokens), else -1.
int32_t block_shift_of(int32_t block_size) {
    switch (block_size) {
        case 8: return 3;
        case 16: return 4;
        case 32: return 5;
        default: return -1;
    }
}

int32_t check_pool(const pa_pool_desc& p) {
    if (elem_size(p.dtype) == 0) return PA_ERR_DTYPE;
    if (p.num_blocks <= 0 || p.num_kv_heads <= 0 || p.head_dim <= 0 || p.block_size <= 0)
        return PA_ERR_SHAPE;
    if (block_shift_of(p.block_size) < 0) return PA_ERR_UNSUPPORTED;
    if (p.head_dim != 64 && p.head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (p.num_kv_heads > 65535) return PA_ERR_SHAPE;
    if ((int64_t)p.num_blocks * p.block_size > INT32_MAX) return PA_ERR_SHAPE;  // slots are int32
    return PA_OK;
}

int32_t check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
    if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
    const int32_t group = num_q_heads / num_kv_heads;
    if (group > kMaxGroup) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// Split-context choice.  One workgroup of the decode kernels per compute unit
// already streams at close to the chip's rate (measured: 256 (row, kv head)
// units of 4-8k tokens each in one pass beat every split of them), so a batch
// with at least 256 units runs in one pass.  Fewer units (few sequences, long
// contexts) are split into as many partitions as bring the launch to about 256
// workgroups; more partitions only add per-workgroup start-up, partial-state
// traffic and merge work (measured at 32-128 units: the best split always gave
// about 256 workgroups).  A split call costs about 15 us whatever its size (two
// launches and the partial states), while one pass costs about 5 us plus the
// longest unit's K/V at 35-50 GB/s per compute unit, so short units run in one
// pass too: those whose K/V (at two bytes an element) is at most
// kOnePassBytes.  (Measured, one pass against the split: head_dim 64, G = 7,
// 32 sequences up to 1,024 tokens 11.6 against 15.7 us, up to 2,048 14.6
// against 15.5; head_dim 128 up to 1,024 tokens at G = 2 20.5 against 16.6
// and at G = 4 16.3 against 15.5.)
constexpr int64_t kSplitTarget = 256;
constexpr int64_t kOnePassBytes = 384 << 10;
int32_t choose_partition(int64_t items, int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                         int32_t requested) {
    if (requested < 0) return -1;
    if (requested > 0) return requested;
    const int64_t units = items * num_kv_heads;
    if (units <= 0 || units >= kSplitTarget || (int64_t)max_context_len * head_dim * 4 <= kOnePassBytes)
        return -1;
    const int64_t parts = ceil_div(kSplitTarget, units);
    const int32_t part = std::max<int32_t>(64, (ceil_div(max_context_len, parts) + 15) / 16 * 16);
    return ceil_div(max_context_len, part) > 1 ? part : -1;
}

// Partial states of a split launch: items * Hq * slots * (acc[D], m, l) fp32,
// slots = the partitions of the context plus extra_slots in front (the key
// parts of a shared prefix).
size_t split_bytes(int64_t items, int32_t num_q_heads, int32_t head_dim,
                   int32_t max_context_len, int32_t part, int32_t extra_slots = 0) {
    if (part <= 0 || items <= 0) return 0;
    const int64_t nparts = ceil_div(max_context_len, part) + extra_slots;
    return (size_t)(items * num_q_heads * nparts * (int64_t)(head_dim + 2) * 4);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// A prefill chunk goes to the matrix cores when it gives at least one 16-row
// tile of (row, head) pairs per kv head; smaller chunks stay on the vector
// path, and have at most small_rows_for(group) rows.
constexpr int32_t kMfmaMinPairs = 16;
int32_t small_rows_for(int32_t group) { return group >= 1 ? (kMfmaMinPairs - 1) / group : 0; }

// Longest-first processing order for decode rows: with a ragged batch the
// workgroups of the longest sequences start first and the short ones fill the
// end, instead of a long sequence starting last and running alone.  Used once
// the batch spans several waves of workgroups.  Up to kRankMaxItems rows the
// attention kernels derive the order themselves; larger batches get it from a
// one-workgroup sorting launch (launch_plan) ahead of the attention kernel.
bool use_plan(int64_t items, int32_t num_kv_heads, int32_t max_context_len, int32_t part) {
    const int64_t units = items * num_kv_heads * (part > 0 ? ceil_div(max_context_len, part) : 1);
    return items >= 16 && units >= 1024;
}

size_t plan_bytes(int64_t items) { return align256((size_t)items * 4); }

// Workspace of one vector-path launch: [order (decode rows, when planned)]
// [split partials].
size_t rows_bytes(int64_t items, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t max_context_len, int32_t part, bool decode_rows, int32_t extra_slots = 0) {
    if (items <= 0) return 0;
    size_t n = 0;
    if (decode_rows && use_plan(items, num_kv_heads, max_context_len, part) && items > kRankMaxItems)
        n += plan_bytes(items);  // order array of launch_plan
    return n + split_bytes(items, num_q_heads, head_dim, max_context_len, part, extra_slots);
}

int32_t check_partition(int32_t requested) {
    if (requested > 0 && requested % kBlock != 0) return PA_ERR_SHAPE;
    return PA_OK;
}

// Fills the common part of a RowsArgs and checks the workspace.  Decode rows
// (no query_start_loc) may get a longest-first order in front of the partials.
int32_t prepare_rows(RowsArgs& a, int64_t items, int32_t part, void* workspace,
                     size_t workspace_bytes, int32_t extra_slots = 0) {
    // Every context empty: one pass, which writes the zero rows (a split
    // launch would have no partition to launch).  A shared prefix (extra
    // slots) needs a context of at least 16 tokens, so it never gets here.
    if (a.max_context_len == 0) part = -1;
    a.num_items = (int32_t)items;
    a.part_tokens = part;
    a.nparts = part > 0 ? ceil_div(a.max_context_len, part) + extra_slots : 1;
    a.prefix_slots = part > 0 ? extra_slots : 0;
    if (part > 0 && a.nparts > 65535) return PA_ERR_SHAPE;
    const bool decode_rows = a.query_start_loc == nullptr;
    const bool plan = decode_rows && use_plan(items, a.num_kv_heads, a.max_context_len, part);
    const size_t need = rows_bytes(items, a.num_q_heads, a.num_kv_heads, a.head_dim,
                                   a.max_context_len, part, decode_rows, extra_slots);
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < need) return PA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PA_ERR_ALIGN;
    }
    char* w = static_cast<char*>(workspace);
    // Up to kRankMaxItems decode rows the attention kernels rank themselves;
    // beyond that launch_plan writes the order into the workspace.
    const bool order_array = plan && items > kRankMaxItems;
    a.rank_shift = plan && !order_array ? rank_shift_for(a.max_context_len) : -1;
    a.order = order_array ? reinterpret_cast<int32_t*>(w) : nullptr;
    a.ws = part > 0 ? reinterpret_cast<float*>(w + (order_array ? plan_bytes(items) : 0)) : nullptr;
    return PA_OK;
}

// Plan (when chosen) and vector-path attention for one prepared launch.
int32_t run_rows(const RowsArgs& a, hipStream_t s) {
    if (a.num_items == 0) return PA_OK;
    if (a.order != nullptr) {
        if (int32_t st = launch_plan(a.context_lens, a.seq_begin, a.num_items, a.max_context_len,
                                     const_cast<int32_t*>(a.order), s))
            return st;
    }
    return launch_rows(a, s);
}

}  // namespace

int32_t pa::check_decode(const void* q, const void* k_pool, const void* v_pool, pa_pool_desc pool,
                         const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads, const void* out,
                         int32_t partition_tokens) {
    if (int32_t st = check_pool(pool)) return st;
    if (int32_t st = check_heads(num_q_heads, pool.num_kv_heads)) return st;
    if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
        (int64_t)max_context_len > (int64_t)max_blocks_per_seq * pool.block_size)
        return PA_ERR_SHAPE;
    if (int32_t st = check_partition(partition_tokens)) return st;
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_ALIGN;
    return PA_OK;
}

// pa_decode, and pa_decode_append when k_new is set (validated by the caller).
int32_t pa::decode_impl(const void* q, const void* k_new, const void* v_new, int64_t k_new_stride,
                    int64_t v_new_stride, const void* k_pool, const void* v_pool, pa_pool_desc pool,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads, float scale, void* out,
                    int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    if (int32_t st = check_decode(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens,
                                  num_seqs, max_context_len, num_q_heads, out, partition_tokens))
        return st;
    if (num_seqs == 0) return PA_OK;

    RowsArgs a = {};
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.max_blocks = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.query_start_loc = nullptr;
    a.seq_begin = 0;
    a.seq_end = num_seqs;
    a.row_begin = 0;
    a.mfma_min_pairs = 0;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = pool.num_kv_heads;
    a.head_dim = pool.head_dim;
    a.num_blocks = pool.num_blocks;
    a.block_shift = block_shift_of(pool.block_size);
    a.dtype = pool.dtype;
    a.max_context_len = max_context_len;
    a.scale = scale;
    a.out = out;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_new_stride = k_new_stride;
    a.v_new_stride = v_new_stride;
    const int32_t part = choose_partition(num_seqs, pool.num_kv_heads, pool.head_dim, max_context_len,
                                          partition_tokens);
    if (int32_t st = prepare_rows(a, num_seqs, part, workspace, workspace_bytes)) return st;
    return run_rows(a, static_cast<hipStream_t>(stream));
}

extern "C" {

const char* pa_status_str(int32_t status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "null pointer argument";
        case PA_ERR_SHAPE: return "size or count out of range or inconsistent";
        case PA_ERR_DTYPE: return "unknown element type";
        case PA_ERR_UNSUPPORTED: return "unsupported block size, head_dim or group size";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_LAUNCH: return "kernel launch failed";
        case PA_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
        case PA_ERR_CAPACITY: return "not enough free blocks";
        case PA_ERR_SCRATCH: return "needs more scratch than the library's per-device array holds (32 MiB)";
        case PA_ERR_STREAM: return "auxiliary stream or its events missing, equal to the call's stream, or on another device";
        default: return "unknown status";
    }
}

int32_t pa_kv_write(const void* k, const void* v, int64_t k_token_stride, int64_t v_token_stride,
                    const int32_t* slot_mapping, int32_t num_tokens, void* k_pool, void* v_pool,
                    pa_pool_desc pool, void* stream) {
    if (int32_t st = check_pool(pool)) return st;
    if (num_tokens < 0) return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if ((int64_t)pool.num_kv_heads * pool.head_dim * elem_size(pool.dtype) > INT32_MAX)
        return PA_ERR_SHAPE;
    if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PA_ERR_NULL;
    const int es = elem_size(pool.dtype);
    const int64_t row_elems = (int64_t)pool.num_kv_heads * pool.head_dim;
    if (k_token_stride < row_elems || v_token_stride < row_elems) return PA_ERR_SHAPE;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (k_token_stride * es) % 16 || (v_token_stride * es) % 16)
        return PA_ERR_ALIGN;
    KvWriteArgs a;
    a.k = k;
    a.v = v;
    a.k_stride = k_token_stride * es;
    a.v_stride = v_token_stride * es;
    a.slots = slot_mapping;
    a.num_tokens = num_tokens;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.pool_rows = (int64_t)pool.num_blocks * pool.block_size;
    a.row_bytes = (int32_t)(row_elems * es);
    return launch_kv_write(a, static_cast<hipStream_t>(stream));
}

int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t partition_tokens) {
    return choose_partition(num_seqs, num_kv_heads > 0 ? num_kv_heads : 1, head_dim > 0 ? head_dim : 0,
                            max_context_len, partition_tokens);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_tokens) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_context_len < 0 || check_partition(partition_tokens))
        return 0;
    const int32_t part = choose_partition(num_seqs, num_kv_heads, head_dim, max_context_len, partition_tokens);
    return rows_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, part, true);
}

int32_t pa_decode(const void* q, const void* k_pool, const void* v_pool, pa_pool_desc pool,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                  int32_t num_q_heads, float scale, void* out, int32_t partition_tokens,
                  void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(q, nullptr, nullptr, 0, 0, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, max_context_len, num_q_heads, scale, out, partition_tokens,
                       workspace, workspace_bytes, stream);
}

int32_t pa_decode_append(const void* q, const void* k_new, const void* v_new, int64_t k_new_stride,
                         int64_t v_new_stride, void* k_pool, void* v_pool, pa_pool_desc pool,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                         int32_t num_q_heads, float scale, void* out, int32_t partition_tokens,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (int32_t st = check_pool(pool)) return st;
    if (num_seqs > 0) {
        if (!k_new || !v_new) return PA_ERR_NULL;
        const int64_t row_elems = (int64_t)pool.num_kv_heads * pool.head_dim;
        if (k_new_stride < row_elems || v_new_stride < row_elems) return PA_ERR_SHAPE;
        const int es = elem_size(pool.dtype);
        if (!aligned16(k_new) || !aligned16(v_new) || (k_new_stride * es) % 16 || (v_new_stride * es) % 16)
            return PA_ERR_ALIGN;
    }
    return decode_impl(q, k_new, v_new, k_new_stride, v_new_stride, k_pool, v_pool, pool, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_q_heads, scale, out,
                       partition_tokens, workspace, workspace_bytes, stream);
}

int32_t pa_qkv_rope_write(const void* qkv, int64_t qkv_token_stride,
                          const int32_t* query_start_loc, int32_t num_tokens, int32_t num_seqs,
                          const int32_t* context_lens, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, int32_t num_q_heads, float rope_theta,
                          const void* q_norm_weight, const void* k_norm_weight, float norm_eps,
                          void* q_out, void* k_pool, void* v_pool, pa_pool_desc pool,
                          int32_t* slot_mapping_out, void* stream) {
    if (int32_t st = check_pool(pool)) return st;
    if (num_tokens < 0 || num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0)
        return PA_ERR_SHAPE;
    if (query_start_loc == nullptr && num_seqs != num_tokens) return PA_ERR_SHAPE;
    if (num_tokens > 0 && num_seqs == 0) return PA_ERR_SHAPE;
    const int64_t width = (int64_t)(num_q_heads + 2 * pool.num_kv_heads) * pool.head_dim;
    if (qkv_token_stride < width) return PA_ERR_SHAPE;
    if (!(rope_theta > 0.0f) || !isfinite(rope_theta) || !(norm_eps >= 0.0f) || !isfinite(norm_eps))
        return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if (!qkv || !context_lens || !block_tables || !q_out || !k_pool || !v_pool) return PA_ERR_NULL;
    const int es = elem_size(pool.dtype);
    if (!aligned16(qkv) || (qkv_token_stride * es) % 16 != 0 || !aligned16(k_pool) ||
        !aligned16(v_pool))
        return PA_ERR_ALIGN;
    QkvArgs a = {};
    a.qkv = qkv;
    a.qkv_stride = qkv_token_stride;
    a.query_start_loc = query_start_loc;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.context_lens = context_lens;
    a.block_tables = block_tables;
    a.max_blocks = max_blocks_per_seq;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = pool.num_kv_heads;
    a.head_dim = pool.head_dim;
    a.num_blocks = pool.num_blocks;
    a.block_shift = block_shift_of(pool.block_size);
    a.dtype = pool.dtype;
    a.log2_theta = log2((double)rope_theta);
    a.q_norm = q_norm_weight;
    a.k_norm = k_norm_weight;
    a.eps = norm_eps;
    a.q_out = q_out;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.slots_out = slot_mapping_out;
    return launch_qkv_write(a, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Launch plan of a shared-prefix decode.
struct CascadePlan {
    int32_t prefix_part;   // keys per part of the prefix phase (multiple of 64), 0: no prefix phase
    int32_t prefix_slots;  // key parts of the longest prefix
    int32_t part;          // partition of the keys after the prefix (multiple of 16); <= 0 with fold
    bool fold;             // one pass after the prefix phase, folding its partial states (no merge)
    size_t bytes;          // workspace
};

// Two plans, chosen by how pa_decode would split the whole context.
//
// When it would run one pass (enough (sequence, kv head) units to fill the
// chip, or units short enough that a split costs more than it saves), the
// prefix phase (if any group has a prefix) runs first, alone, on the call's
// stream, its key
// range split into as many parts as keep it a launch of 64-row tiles with key
// halves (row tiles x kv heads x groups x parts below kChunkSplitBelow; at
// least two 64-key tiles per part, one for each key half); then the decode
// kernel reads each sequence's keys after the prefix in one pass and folds
// the prefix's partial states into its own before writing the output.  No
// second stream, no merge launch.  (Measured on 64 sequences of 8,192 tokens
// sharing 4,096, G = 7: 8 parts in 224 workgroups 112 us for the call; 16
// parts in 256 workgroups of 128 rows 118 us; 6 parts 114 us.)
//
// Otherwise the keys after the prefix are split as pa_decode would split the
// whole context, always into partial states, and the prefix phase runs beside
// the decode kernel (on the caller's second stream when given): its key range
// is split into parts of at least 256 keys until it has about 128 workgroups,
// few enough parts to keep the merge short; the merge combines both.
CascadePlan cascade_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t max_context_len, int32_t num_groups, int32_t max_group_size,
                         int32_t prefix_cap, int32_t partition_tokens) {
    CascadePlan p = {};
    const int32_t group = num_q_heads / num_kv_heads;
    const int32_t plen = prefix_cap & ~15;
    int32_t part = choose_partition(num_seqs, num_kv_heads, head_dim, max_context_len, partition_tokens);
    p.fold = part <= 0;
    if (plen > 0) {
        const int64_t row_tiles = ceil_div((int64_t)max_group_size * group, 128);
        const int64_t tiles = ceil_div(plen, 64);
        const int64_t base = row_tiles * num_kv_heads * num_groups;
        int64_t parts;
        if (p.fold) {
            const int64_t small_base = ceil_div((int64_t)max_group_size * group, kChunkRowsSmall) *
                                       num_kv_heads * num_groups;
            parts = std::min<int64_t>((kChunkSplitBelow - 1) / small_base, tiles / 2);
        } else {
            parts = std::min<int64_t>(ceil_div(128, base), tiles / 4);
        }
        parts = std::max<int64_t>(1, parts);
        p.prefix_part = (int32_t)(64 * ceil_div(tiles, parts));
        p.prefix_slots = ceil_div(plen, p.prefix_part);
    }
    if (p.fold) {
        p.part = -1;
        p.bytes = rows_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, -1, true) +
                  (size_t)num_seqs * num_q_heads * p.prefix_slots * (size_t)(head_dim + 2) * 4;
        return p;
    }
    if (part <= 0) part = std::max(16, (max_context_len + 15) / 16 * 16);
    p.part = part;
    p.bytes = rows_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, part, true,
                         p.prefix_slots);
    return p;
}

}  // namespace

extern "C" {

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t max_context_len, int32_t num_groups,
                                               int32_t max_group_size, int32_t max_prefix_len,
                                               int32_t partition_tokens) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
        num_groups <= 0 || max_group_size <= 0 || max_prefix_len < 0 || max_prefix_len > max_context_len ||
        num_q_heads % num_kv_heads != 0 || check_partition(partition_tokens))
        return 0;
    return cascade_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, num_groups,
                        max_group_size, max_prefix_len, partition_tokens).bytes;
}

int32_t pa_decode_shared_prefix(const void* q, const void* k_pool, const void* v_pool, pa_pool_desc pool,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                const int32_t* group_start, const int32_t* prefix_lens, int32_t num_groups,
                                int32_t max_group_size, int32_t max_prefix_len, int32_t num_q_heads,
                                float scale, void* out, int32_t partition_tokens, void* workspace,
                                size_t workspace_bytes, void* stream, const pa_aux_stream* aux) {
    if (int32_t st = check_pool(pool)) return st;
    if (int32_t st = check_heads(num_q_heads, pool.num_kv_heads)) return st;
    if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
        (int64_t)max_context_len > (int64_t)max_blocks_per_seq * pool.block_size)
        return PA_ERR_SHAPE;
    if (int32_t st = check_partition(partition_tokens)) return st;
    if (num_seqs == 0) return PA_OK;
    if (num_groups <= 0 || num_groups > num_seqs || num_groups > 65535 || max_group_size <= 0 ||
        max_group_size > num_seqs || max_prefix_len < 0 || max_prefix_len > max_context_len)
        return PA_ERR_SHAPE;
    const int32_t group = num_q_heads / pool.num_kv_heads;
    if (!chunks_supported(pool.dtype, pool.head_dim, group)) return PA_ERR_UNSUPPORTED;
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out || !group_start || !prefix_lens)
        return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_ALIGN;
    if (int32_t st = check_aux(aux, static_cast<hipStream_t>(stream))) return st;

    const int32_t prefix_cap = (int32_t)std::min<int64_t>(max_prefix_len, (int64_t)max_blocks_per_seq * pool.block_size);
    const CascadePlan cp = cascade_plan(num_seqs, num_q_heads, pool.num_kv_heads, pool.head_dim, max_context_len,
                                        num_groups, max_group_size, prefix_cap, partition_tokens);
    RowsArgs a = {};
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.max_blocks = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.query_start_loc = nullptr;
    a.seq_begin = 0;
    a.seq_end = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = pool.num_kv_heads;
    a.head_dim = pool.head_dim;
    a.num_blocks = pool.num_blocks;
    a.block_shift = block_shift_of(pool.block_size);
    a.dtype = pool.dtype;
    a.max_context_len = max_context_len;
    a.scale = scale;
    a.out = out;
    a.group_start = group_start;
    a.prefix_lens = prefix_lens;
    a.num_groups = num_groups;
    a.prefix_cap = prefix_cap;
    a.prefix_part_tokens = cp.prefix_part > 0 ? cp.prefix_part : 64;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (cp.fold) {
        // one pass; the prefix's partial states follow the order array (if
        // any); with no prefix and no order array nothing is needed
        if (cp.bytes > 0 && (workspace == nullptr || workspace_bytes < cp.bytes)) return PA_ERR_WORKSPACE;
        if (workspace != nullptr && !aligned16(workspace)) return PA_ERR_ALIGN;
        if (int32_t st = prepare_rows(a, num_seqs, -1, workspace, workspace_bytes)) return st;
        const size_t order_bytes = rows_bytes(num_seqs, num_q_heads, pool.num_kv_heads, pool.head_dim,
                                              max_context_len, -1, true);
        a.ws = cp.prefix_slots > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + order_bytes)
                                   : nullptr;
        a.nparts = cp.prefix_slots;
        a.prefix_slots = cp.prefix_slots;
        a.fold_prefix = 1;
    } else if (int32_t st = prepare_rows(a, num_seqs, cp.part, workspace, workspace_bytes, cp.prefix_slots)) {
        return st;
    }
    if (cp.prefix_slots == 0) return run_rows(a, s);
    {
        // Prefix phase: each group's members are the rows of one "chunk" that
        // sees the whole prefix, read through the first member's table.
        ChunkArgs c = {};
        c.q = q;
        c.query_start_loc = group_start;
        c.num_seqs = num_groups;
        c.max_query_len = max_group_size;
        c.k_pool = k_pool;
        c.v_pool = v_pool;
        c.block_tables = block_tables;
        c.max_blocks = max_blocks_per_seq;
        c.context_lens = prefix_lens;
        c.max_context_len = prefix_cap;
        c.num_q_heads = num_q_heads;
        c.num_kv_heads = pool.num_kv_heads;
        c.head_dim = pool.head_dim;
        c.num_blocks = pool.num_blocks;
        c.block_shift = a.block_shift;
        c.dtype = pool.dtype;
        c.total_rows = num_seqs;
        c.scale = scale;
        c.out = out;
        c.min_pairs = 0;
        c.causal = 0;
        c.table_row_qsl = 1;
        c.key_parts = cp.prefix_slots;
        c.key_part_tokens = cp.prefix_part;
        c.partials = a.ws;
        c.part_slots = a.nparts;
        c.num_items = num_seqs;
        if (cp.fold) {
            // the prefix phase alone, then the decode kernel, which folds it in
            c.alone = 1;
            if (int32_t st = launch_chunks(c, s)) return st;
            return run_rows(a, s);
        }
        c.prefer_large = 1;
        // The prefix phase (matrix cores, LDS, cache-resident keys) runs on the
        // caller's auxiliary stream beside the decode kernel (HBM); they write
        // disjoint partial slots, and the merge waits for both.  Without an
        // auxiliary stream the two run one after the other on `stream`.
        if (aux == nullptr) {
            c.alone = 1;  // nothing beside it: the key-halves shape
            if (int32_t st = launch_chunks(c, s)) return st;
            return run_rows(a, s);
        }
        if (int32_t st = fork_to(*aux, s)) return st;
        // decode kernel first: its workgroups take one slot per compute unit,
        // the prefix workgroups fill in beside them
        a.defer_merge = 1;
        if (int32_t st = run_rows(a, s)) return st;
        if (int32_t st = launch_chunks(c, static_cast<hipStream_t>(aux->stream))) return st;
        if (int32_t st = join_from(*aux, s)) return st;
        return launch_merge(a, s);
    }
}

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_prefill_seqs,
                                  int32_t total_query_tokens, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                                  int32_t partition_tokens) {
    if (num_seqs <= 0 || num_prefill_seqs < 0 || num_prefill_seqs > num_seqs ||
        num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
        check_partition(partition_tokens))
        return 0;
    const int64_t num_decode = num_seqs - num_prefill_seqs;
    const int64_t prefill_rows = (int64_t)total_query_tokens - num_decode;
    // [decode rows' part, 256-byte aligned][prefill rows' part]: the two
    // vector-path launches may run at the same time on two streams.
    size_t pre = 0, dec = 0;
    if (prefill_rows > 0) {
        // The vector path covers either every prefill row or, when the matrix
        // cores take the large chunks, a few row slots per prefill sequence;
        // the element type decides which, so size for both.
        const int64_t slots = (int64_t)num_prefill_seqs * small_rows_for(num_q_heads / num_kv_heads);
        for (const int64_t items : {prefill_rows, slots}) {
            const int32_t part = choose_partition(items, num_kv_heads, head_dim, max_context_len, partition_tokens);
            const size_t p = rows_bytes(items, num_q_heads, num_kv_heads, head_dim, max_context_len, part, false);
            if (p > pre) pre = p;
        }
    }
    if (num_decode > 0) {
        const int32_t part = choose_partition(num_decode, num_kv_heads, head_dim, max_context_len, partition_tokens);
        dec = rows_bytes(num_decode, num_q_heads, num_kv_heads, head_dim, max_context_len, part, true);
    }
    return pre > 0 ? align256(dec) + pre : dec;
}

int32_t pa_prefill_chunk(const void* q, const int32_t* query_start_loc, int32_t total_query_tokens,
                         int32_t num_seqs, int32_t num_prefill_seqs, int32_t max_query_len,
                         const void* k_pool, const void* v_pool, pa_pool_desc pool,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t max_context_len, int32_t num_q_heads,
                         float scale, void* out, int32_t partition_tokens, void* workspace,
                         size_t workspace_bytes, void* stream, const pa_aux_stream* aux) {
    if (int32_t st = check_pool(pool)) return st;
    if (int32_t st = check_heads(num_q_heads, pool.num_kv_heads)) return st;
    if (num_seqs < 0 || num_prefill_seqs < 0 || num_prefill_seqs > num_seqs ||
        total_query_tokens < 0 || max_query_len < 0 || max_blocks_per_seq <= 0 ||
        max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * pool.block_size ||
        max_query_len > max_context_len)
        return PA_ERR_SHAPE;
    const int64_t num_decode = num_seqs - num_prefill_seqs;
    const int64_t prefill_rows = (int64_t)total_query_tokens - num_decode;
    if (prefill_rows < 0 || (num_prefill_seqs == 0 && prefill_rows != 0)) return PA_ERR_SHAPE;
    if (int32_t st = check_partition(partition_tokens)) return st;
    if (num_seqs == 0 || total_query_tokens == 0) return PA_OK;
    if (!q || !query_start_loc || !k_pool || !v_pool || !block_tables || !context_lens || !out)
        return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int32_t st = check_aux(aux, s)) return st;
    const int32_t group = num_q_heads / pool.num_kv_heads;

    RowsArgs base = {};
    base.q = q;
    base.k_pool = k_pool;
    base.v_pool = v_pool;
    base.block_tables = block_tables;
    base.max_blocks = max_blocks_per_seq;
    base.context_lens = context_lens;
    base.num_q_heads = num_q_heads;
    base.num_kv_heads = pool.num_kv_heads;
    base.head_dim = pool.head_dim;
    base.num_blocks = pool.num_blocks;
    base.block_shift = block_shift_of(pool.block_size);
    base.dtype = pool.dtype;
    base.max_context_len = max_context_len;
    base.scale = scale;
    base.out = out;

    // Check both vector-path launches before enqueuing anything.  Their
    // workspace parts are disjoint (decode rows first), so the two launches
    // need no ordering between them.
    RowsArgs pre = base, dec = base;
    pre.query_start_loc = query_start_loc;
    pre.seq_begin = 0;
    pre.seq_end = num_prefill_seqs;
    pre.row_begin = 0;
    const bool mfma = prefill_rows > 0 && chunks_supported(pool.dtype, pool.head_dim, group);
    pre.mfma_min_pairs = mfma ? kMfmaMinPairs : 0;
    pre.small_rows = mfma ? small_rows_for(group) : 0;
    // Every chunk has at most max_query_len rows, so the smallest has at least
    // prefill_rows - (num_prefill_seqs - 1) * max_query_len: when even that
    // many rows give a matrix-core tile, no chunk is left to the vector path
    // and its launch (all slots idle) is skipped.
    const int64_t min_chunk = prefill_rows - (int64_t)(num_prefill_seqs - 1) * max_query_len;
    const bool any_small = !mfma || min_chunk * group < kMfmaMinPairs;
    const int64_t pre_items = mfma ? (any_small ? (int64_t)num_prefill_seqs * pre.small_rows : 0) : prefill_rows;
    if (pre_items > INT32_MAX) return PA_ERR_SHAPE;
    dec.query_start_loc = nullptr;
    dec.seq_begin = num_prefill_seqs;
    dec.seq_end = num_seqs;
    dec.row_begin = (int32_t)prefill_rows;
    dec.mfma_min_pairs = 0;
    const int32_t dpart = choose_partition(num_decode, pool.num_kv_heads, pool.head_dim, max_context_len,
                                           partition_tokens);
    if (int32_t st = prepare_rows(dec, num_decode, dpart, workspace, workspace_bytes)) return st;
    const size_t dec_bytes = align256(rows_bytes(num_decode, num_q_heads, pool.num_kv_heads,
                                                 pool.head_dim, max_context_len, dpart, true));
    const int32_t ppart = choose_partition(pre_items, pool.num_kv_heads, pool.head_dim, max_context_len,
                                           partition_tokens);
    const bool pre_ws = rows_bytes(pre_items, num_q_heads, pool.num_kv_heads, pool.head_dim,
                                   max_context_len, ppart, false) > 0;
    if (pre_ws && workspace_bytes < dec_bytes) return PA_ERR_WORKSPACE;
    if (int32_t st = prepare_rows(pre, pre_items, ppart,
                                  pre_ws ? static_cast<char*>(workspace) + dec_bytes : nullptr,
                                  pre_ws ? workspace_bytes - dec_bytes : 0))
        return st;

    ChunkArgs c = {};
    if (mfma) {
        c.q = q;
        c.query_start_loc = query_start_loc;
        c.num_seqs = num_prefill_seqs;
        c.max_query_len = max_query_len;
        c.k_pool = k_pool;
        c.v_pool = v_pool;
        c.block_tables = block_tables;
        c.max_blocks = max_blocks_per_seq;
        c.context_lens = context_lens;
        c.max_context_len = max_context_len;
        c.num_q_heads = num_q_heads;
        c.num_kv_heads = pool.num_kv_heads;
        c.head_dim = pool.head_dim;
        c.num_blocks = pool.num_blocks;
        c.block_shift = block_shift_of(pool.block_size);
        c.dtype = pool.dtype;
        c.total_rows = total_query_tokens;
        c.scale = scale;
        c.out = out;
        c.min_pairs = kMfmaMinPairs;
        c.causal = 1;
        c.key_parts = 1;
        c.alone = num_decode == 0;  // nothing runs beside the chunk kernel
    }
    // The chunks (matrix cores, LDS) and the decode rows (HBM) use different
    // parts of the chip and run concurrently when the caller passes an
    // auxiliary stream: the chunk kernel on the caller's stream, the vector
    // path on the auxiliary stream.  They read the same
    // pools and write disjoint rows of out; the two vector-path launches use
    // disjoint parts of the workspace.  The order matters: a chunk workgroup
    // (4 waves of 256 registers, 96 KiB of LDS) fits on a compute unit beside
    // one decode workgroup but not beside the three the decode kernel places
    // on an idle one, so the chunks must reach the compute units first
    // (measured: with the decode rows first the chunk kernel waited for their
    // workgroups to drain and the mixed step took 10% longer).  A kernel on
    // the caller's stream starts about 1 us after the previous one ends, while
    // every wait across streams costs 8-14 us (measured on MI355X, whatever
    // the event flags), so the chunk kernel, launched right after the fork
    // mark, is on the compute units well before the decode rows pass their
    // fork wait, and the one cross-stream hop in front of the long decode
    // kernel is the fork itself.  (Chunks on the auxiliary stream behind the
    // fork, with the decode rows waiting for a `started` mark, put two hops in
    // front of the decode rows and measured 209 us per mixed step.  One fused
    // launch holding both kinds of workgroup avoids the waits but measured
    // slower: the decode loop compiled inside the larger kernel ran 12%
    // slower.)
    if (aux != nullptr && mfma && num_decode > 0) {
        hipStream_t x = static_cast<hipStream_t>(aux->stream);
        if (int32_t st = fork_to(*aux, s)) return st;
        if (int32_t st = launch_chunks(c, s)) return st;
        if (int32_t st = run_rows(pre, x)) return st;  // small chunks, if any
        if (int32_t st = run_rows(dec, x)) return st;
        return join_from(*aux, s);
    }
    // One stream: the chunk kernel runs before the vector path, alone.
    c.alone = 1;
    if (mfma)
        if (int32_t st = launch_chunks(c, s)) return st;
    if (int32_t st = run_rows(pre, s)) return st;
    if (num_decode > 0)
        if (int32_t st = run_rows(dec, s)) return st;
    return PA_OK;
}

}  // extern "C"
