// Internal interface between the C ABI layer (pa_api.cpp) and the kernel
// translation units.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

// The attention kernels work in chunks of 16 tokens (the pages' block size).
// A pool block holds 8, 16 or 32 tokens (block_shift 3, 4 or 5): a 16-token
// chunk lies inside one block of 16 or 32, and spans two blocks of 8.
constexpr int kBlock = 16;

// Where a 16-token chunk c lives, for pools of 1 << shift tokens per block:
// its table entries are lo = (c << mul) >> shr and hi = ((c << mul) + mul) >> shr
// (blocks of 8: entries 2c and 2c+1; of 16: c; of 32: c/2), its tokens 0-7
// start at row (c*16 & in_block) of entry lo, and its tokens 8-15 at row
// (c*16 & in_block) + hi_off of entry hi.
struct ChunkMap {
    int mul, shr, in_block, hi_off;
};
__host__ __device__ inline ChunkMap chunk_map(int shift) {
    return shift == 3 ? ChunkMap{1, 0, 0, 0} : ChunkMap{0, shift - 4, (1 << shift) - 1, 8};
}
constexpr int kMaxGroup = 8; // largest GQA group built
// Chunk-kernel launch shapes (chosen in launch_chunks): a launch with fewer
// than kChunkSplitBelow workgroups of kChunkRowsSmall rows runs them with key
// halves; larger launches take 128-row tiles.
constexpr int kChunkSplitBelow = 256;
constexpr int kChunkRowsSmall = 64;

// One launch of the vector-path attention over a set of query rows ("items").
struct RowsArgs {
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    int32_t max_blocks;
    const int32_t* context_lens;
    // NULL: item z is sequence seq_begin+z with one row (row_begin+z).
    // Otherwise item z is row row_begin+z, its sequence is found in
    // [seq_begin, seq_end) by binary search over query_start_loc.
    const int32_t* query_start_loc;
    int32_t seq_begin, seq_end;
    int32_t row_begin;
    int32_t num_items;
    // Without query_start_loc: optional processing order, item order[z] is
    // handled z-th (longest first, written by launch_plan); NULL = index order.
    const int32_t* order;
    // Without query_start_loc and order: rank_shift >= 0 makes each
    // workgroup derive the longest-first order itself from the lengths
    // (buckets min(L, max_context_len) >> rank_shift, at most kRankMaxItems
    // items); -1: no ranking.
    int32_t rank_shift;
    // With query_start_loc: items whose sequence gives at least this many
    // (row, head) pairs per kv head are left to the matrix-core kernel
    // (0 = handle every item here).
    int32_t mfma_min_pairs;
    // With query_start_loc and small_rows > 0: item z is row z % small_rows of
    // sequence seq_begin + z / small_rows (a slot past the sequence's rows, or
    // of a sequence left to the matrix cores, does nothing).  small_rows is the
    // most rows a sequence below mfma_min_pairs can have, so the launch covers
    // only the chunks that stay on the vector path, not every prefill row.
    int32_t small_rows;
    int32_t num_q_heads, num_kv_heads, head_dim, num_blocks, dtype;
    int32_t max_context_len;
    float scale;
    void* out;
    int32_t part_tokens;  // <= 0: one pass, else a multiple of 16
    int32_t nparts;       // partitions per item when split
    float* ws;            // split partials: acc [items,Hq,nparts,D], m, l [items,Hq,nparts]
    int32_t block_shift;  // log2 of the pool's block size
    // Shared-prefix mode (decode items, group_start != NULL): the sequences
    // group_start[g] .. group_start[g+1]-1 share their first prefix_lens[g]
    // tokens (clamped to prefix_cap, rounded down to a multiple of 16), which
    // the chunk kernel attended in parts of prefix_part_tokens keys, writing
    // partial slots 0.. of each (item, q head).  This launch covers the keys
    // after the prefix, always as partials, at slots prefix_slots + part; the
    // merge combines both.
    const int32_t* group_start;
    const int32_t* prefix_lens;
    int32_t num_groups;
    int32_t prefix_cap;
    int32_t prefix_part_tokens;
    int32_t prefix_slots;
    // Split launches: 1 leaves the merge to a later launch_merge call.
    int32_t defer_merge;
    // Shared-prefix mode in one pass (part_tokens <= 0): 1 = the prefix's
    // partial states (slots 0 .. of each (item, q head), nparts slots per
    // (item, q head)) are already in ws, and the attention kernel folds them
    // into its own state before writing the output (no merge launch).
    int32_t fold_prefix;
    // Append mode (decode items only, k_new != NULL): sequence s's new token
    // is the one at position len-1 (len = its clamped context length); its K
    // and V rows are at k_new + s*k_new_stride and v_new + s*v_new_stride
    // (elements, [Hkv, D] each).  The workgroup that attends position len-1
    // uses them in place of the pool's contents and stores them at that
    // position's pool slot when its table entry lies inside the pool.
    const void* k_new;
    const void* v_new;
    int64_t k_new_stride, v_new_stride;
};

int32_t launch_rows(const RowsArgs& a, hipStream_t stream);
// The log-sum-exp merge of a split launch (launch_rows does it itself unless
// defer_merge is set).
int32_t launch_merge(const RowsArgs& a, hipStream_t stream);

// Most decode items the attention kernels rank themselves (256 threads x 8);
// larger batches get their order from launch_plan.
constexpr int32_t kRankMaxItems = 2048;
// Bucket shift for in-kernel ranking: max_context_len >> shift < 256.
inline int32_t rank_shift_for(int32_t max_context_len) {
    int32_t shift = 0;
    while ((max_context_len >> shift) >= 256) ++shift;
    return shift;
}

// Counting sort of sequences seq_begin .. seq_begin+n-1 by context length,
// longest first, into order[0..n) (indices relative to seq_begin).
int32_t launch_plan(const int32_t* context_lens, int32_t seq_begin, int32_t n,
                    int32_t max_context_len, int32_t* order, hipStream_t stream);

struct KvWriteArgs {
    const void* k;
    const void* v;
    int64_t k_stride, v_stride;  // BYTES between consecutive tokens
    const int32_t* slots;
    int32_t num_tokens;
    void* k_pool;
    void* v_pool;
    int64_t pool_rows;           // num_blocks * 16
    int32_t row_bytes;           // num_kv_heads * head_dim * element size
};

int32_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);

// Fused QKV split + rotary embedding + KV write; one workgroup per token.
struct QkvArgs {
    const void* qkv;
    int64_t qkv_stride;                 // ELEMENTS between consecutive tokens
    const int32_t* query_start_loc;     // NULL: token t is sequence t
    int32_t num_seqs, num_tokens;
    const int32_t* context_lens;
    const int32_t* block_tables;
    int32_t max_blocks;
    int32_t num_q_heads, num_kv_heads, head_dim, num_blocks, dtype;
    double log2_theta;                  // log2 of the rotary base
    const void* q_norm;                 // [head_dim] or NULL (no norm)
    const void* k_norm;
    float eps;
    void* q_out;
    void* k_pool;
    void* v_pool;
    int32_t* slots_out;                 // [num_tokens] or NULL
    int32_t block_shift;                // log2 of the pool's block size
};

int32_t launch_qkv_write(const QkvArgs& a, hipStream_t stream);

// Matrix-core causal chunk attention for prefill sequences 0..num_seqs-1 whose
// rows give at least `min_pairs` (row, head) pairs per kv head.
struct ChunkArgs {
    const void* q;
    const int32_t* query_start_loc;
    int32_t num_seqs;
    int32_t max_query_len;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    int32_t max_blocks;
    const int32_t* context_lens;
    int32_t max_context_len;
    int32_t num_q_heads, num_kv_heads, head_dim, num_blocks, dtype;
    int32_t total_rows;
    float scale;
    void* out;
    int32_t min_pairs;
    int32_t block_shift;  // log2 of the pool's block size
    // 1: row i of an n-row chunk sees keys 0 .. L-n+i.  0 (a shared prefix):
    // every row sees keys 0 .. L-1, L rounded down to a multiple of 16.
    int32_t causal;
    // 1: sequence s reads its keys through table row query_start_loc[s] (a
    // group's first member) instead of row s.
    int32_t table_row_qsl;
    // key_parts > 1: the keys are split into parts of key_part_tokens (a
    // multiple of 64), one workgroup per (row tile, part).
    int32_t key_parts, key_part_tokens;
    // Non-NULL: each row leaves its partial state (acc, m, l) of its key part
    // kp at slot (row's item * Hq + q head) * part_slots + kp of the split
    // layout with num_items items, instead of writing out.
    float* partials;
    int32_t part_slots, num_items;
    // 1: always the 128-row, single-key-range launch shape (96 KiB of LDS,
    // leaving room on each compute unit for a concurrent decode kernel).
    int32_t prefer_large;
    // 1: nothing else runs beside this launch (a prefill batch without decode
    // rows): a large launch takes two key halves as well (8 waves, 144 KiB of
    // LDS per workgroup), which would crowd out a kernel sharing the chip.
    int32_t alone;
};

// Returns PA_ERR_UNSUPPORTED when no matrix-core kernel exists for the shape
// (the caller then sends every row down the vector path).
int32_t launch_chunks(const ChunkArgs& a, hipStream_t stream);
// Shapes the matrix-core chunk kernel is built for.
inline bool chunks_supported(int32_t dtype, int32_t head_dim, int32_t group) {
    return (dtype == PA_BF16 || dtype == PA_F16) && (head_dim == 64 || head_dim == 128) && group >= 1 &&
           group <= kMaxGroup;
}

// pa_decode's host-side argument checks (PA_OK for a valid call, including an
// empty batch).
int32_t check_decode(const void* q, const void* k_pool, const void* v_pool, pa_pool_desc pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads, const void* out,
                     int32_t partition_tokens);

// pa_decode (k_new == NULL) and pa_decode_append: validation, path choice and
// launch, with the workspace the caller provides.
int32_t decode_impl(const void* q, const void* k_new, const void* v_new, int64_t k_new_stride,
                    int64_t v_new_stride, const void* k_pool, const void* v_pool, pa_pool_desc pool,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads, float scale, void* out,
                    int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace pa
