/*
 * pa.h -- C ABI of the paged-KV attention library for MI355X (gfx950).
 *
 * The library has four operations, taken from how the pages frame the
 * problem:
 *
 *   pa_kv_write       append each step's new K/V rows into a shared block pool
 *                     at flat slots ("mini_engine", Next: fused kernels -- the
 *                     fused KV-cache write; "mini-vllm", Milestones item 7 --
 *                     GPU-side slot derivation).
 *   pa_qkv_rope_write the same write fed straight from the packed QKV
 *                     projection: q/k norm and rotary embedding applied, slots
 *                     derived on the device from the block tables.
 *   pa_decode         batched grouped-query decode attention over a ragged set
 *                     of sequences, reading K/V in place through per-sequence
 *                     block tables ("09 -- Mini Inference Engine (The
 *                     Capstone)", Week 4 -- Paged KV cache; "mini-vllm",
 *                     Milestones item 6; "mini_engine", What it does -- GQA).
 *   pa_prefill_chunk  causal attention for a mixed batch of prefill chunks and
 *                     decode rows under a token budget ("mini_engine", What it
 *                     does -- chunked prefill; Capstone page, Week 3 option B
 *                     and the design-decision table's chunked-prefill entry).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *   allocates no device memory, keeps no handle, stream, event or other
 *   global state between calls, and is reentrant.  Scratch memory is passed in
 *   as `workspace`, sized by the matching *_workspace_bytes.  The two calls
 *   that can run two kernels side by side (pa_prefill_chunk,
 *   pa_decode_shared_prefix) take a second stream and two events from the
 *   caller (pa_aux_stream); without one they run on `stream` alone.  (The
 *   block manager's state lives in the handle the caller creates and
 *   destroys.)
 * - Every call validates its host arguments first.  On failure it returns a
 *   non-zero pa_status, enqueues nothing and leaves every output untouched.
 * - On success the work is enqueued on `stream` (a hipStream_t; NULL means the
 *   default stream) and the call returns without synchronising.  The library
 *   never reads device memory from the host, so all sizes the launch needs come
 *   in as host integers.
 * - Layouts are row-major and contiguous unless a stride says otherwise:
 *     pools          [num_blocks, B, num_kv_heads, head_dim], B = block_size
 *     q, out         [rows, num_q_heads, head_dim]
 *     block_tables   int32 [num_seqs, max_blocks_per_seq]; entry i is the
 *                    physical block holding logical tokens B*i .. B*i+B-1
 *     context_lens   int32 [num_seqs]; tokens attended, including the ones
 *                    written in this step (write first, then attend)
 * - Query head h attends with kv head h / (num_q_heads / num_kv_heads).
 * - q, out and the pools share one element type: bf16 or fp16 (accumulation in
 *   fp32, output rounded to nearest even) or fp32.
 * - Device-side data is trusted for results but not for memory safety: slots
 *   outside [0, num_blocks*B) are skipped, block ids are clamped into
 *   [0, num_blocks), context lengths are clamped into [0, max_context_len] and
 *   to max_blocks_per_seq*B.  Such inputs give unspecified values, never an
 *   out-of-bounds access.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = 1,        /* a required pointer is NULL */
    PA_ERR_SHAPE = 2,       /* a size or count is out of range or inconsistent */
    PA_ERR_DTYPE = 3,       /* unknown element type */
    PA_ERR_UNSUPPORTED = 4, /* valid but not built: block size, head_dim, group */
    PA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
    PA_ERR_LAUNCH = 6,      /* the HIP runtime rejected a launch */
    PA_ERR_ALIGN = 7,       /* a pointer or stride breaks 16-byte alignment */
    PA_ERR_CAPACITY = 8,    /* block manager: not enough free blocks (nothing changed) */
    PA_ERR_STREAM = 9,      /* pa_aux_stream incomplete, equal to the call's stream,
                               or on another device */
    PA_ERR_SCRATCH = 10     /* pa_decode_noalloc: the call needs more scratch than the
                               library's fixed per-device array holds */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_F16 = 2 } pa_dtype;

/* Shape of one layer's K pool (the V pool has the same shape).
 * block_size 8, 16 or 32 tokens (16 is the pages' choice; the others serve a
 * block-size sweep, and a 16-token chunk then spans two blocks of 8 or half
 * a block of 32); head_dim 64 or 128; dtype a pa_dtype. */
typedef struct {
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;
} pa_pool_desc;

/* A second stream owned by the caller, for the calls that can run two
 * kernels at once (pa_prefill_chunk: decode rows beside matrix-core chunks;
 * pa_decode_shared_prefix: the prefix phase beside the decode kernel).
 *   stream      hipStream_t on the same device as the call's stream, and not
 *               that stream
 *   fork_event  hipEvent_t; the call records it on its stream and makes
 *               `stream` wait for it, so the auxiliary work follows everything
 *               enqueued on the call's stream before the call
 *   join_event  hipEvent_t; the call records it on `stream` and makes its own
 *               stream wait for it, so work enqueued on the call's stream after
 *               the call follows the auxiliary work
 * Create the events with hipEventDisableTiming (they only order work).  All
 * three stay the caller's; the library keeps no reference past the call.
 * Concurrent calls from several host threads must not share one
 * pa_aux_stream (their records and waits would interleave).  HIP graph capture
 * records the fork and the join like any other cross-stream dependency. */
typedef struct {
    void* stream;
    void* fork_event;
    void* join_event;
} pa_aux_stream;

/* Human-readable name of a status code (static string, never NULL). */
const char* pa_status_str(int32_t status);

/*
 * pa_kv_write -- scatter new tokens' K and V rows into the pools.
 *
 * k, v            [num_tokens, num_kv_heads, head_dim] rows; consecutive
 *                 tokens are k_token_stride / v_token_stride ELEMENTS apart
 *                 (so views into a packed QKV projection work); within a token
 *                 the [num_kv_heads, head_dim] row is contiguous.
 * slot_mapping    int32 [num_tokens]; token t goes to block slot/B, offset
 *                 slot%B, i.e. row `slot` of the pool seen as
 *                 [num_blocks*B, num_kv_heads*head_dim].  slot < 0 marks a
 *                 padding token: nothing is written for it.  Slots must be
 *                 distinct within one call (otherwise which row wins is
 *                 unspecified).
 * k_pool, v_pool  written in place; nothing else in them changes.
 * The copy is bit-exact.  Pointers and strides must be 16-byte aligned.
 * num_tokens == 0 returns PA_OK without enqueuing anything.
 */
int32_t pa_kv_write(const void* k, const void* v,
                    int64_t k_token_stride, int64_t v_token_stride,
                    const int32_t* slot_mapping, int32_t num_tokens,
                    void* k_pool, void* v_pool, pa_pool_desc pool,
                    void* stream);

/*
 * pa_qkv_rope_write -- split the packed QKV projection, apply the rotary
 * embedding (and optionally Qwen3's per-head RMSNorm) to q and k, store k and
 * v in the pools at slots derived on the device, and write the rotated q.
 * ("mini_engine", What it does: QKV packed into one GEMM, RoPE, RMSNorm; Next:
 * fused kernels -- fused RoPE, fused QKV split and KV-cache write; "mini-vllm",
 * Milestones item 7 -- GPU-side slot derivation.)
 *
 * qkv               [num_tokens, *] rows; consecutive tokens are
 *                   qkv_token_stride ELEMENTS apart (>= (Hq + 2*Hkv) * D); a row
 *                   holds the Hq q heads, then the Hkv k heads, then the Hkv v
 *                   heads, each head_dim elements.
 * query_start_loc   int32 [num_seqs + 1] as in pa_prefill_chunk (tokens of
 *                   sequence s are qsl[s] .. qsl[s+1]-1), or NULL: one token per
 *                   sequence, token t belongs to sequence t (num_seqs must equal
 *                   num_tokens).
 * context_lens      int32 [num_seqs]; lengths AFTER this step's tokens (write
 *                   first, then attend): token i of a sequence with n tokens
 *                   and length L is at position L - n + i.
 * block_tables      int32 [num_seqs, max_blocks_per_seq].
 * Slot of a token = block_tables[s][pos / B] * B + pos % B.  When the
 * position lies outside the table or the entry outside the pool, nothing is
 * written to the pools for that token (its q row is still written) and its
 * slot reads -1.
 * rope_theta        rotary base (> 0).  Rotate-half convention: dims i and
 *                   i + D/2 of every q and k head turn by pos * theta^(-2i/D);
 *                   the angle is formed and reduced to within half a turn in
 *                   fp64, its sine and cosine taken in fp32.
 * q_norm_weight, k_norm_weight
 *                   [head_dim] each, in the pool's element type, or NULL: with a
 *                   weight, each head is RMS-normalised (x / sqrt(mean(x^2) +
 *                   norm_eps) * w) before the rotation.
 * q_out             [num_tokens, Hq, D] rotated q, element type of the pool.
 * slot_mapping_out  int32 [num_tokens] or NULL: the derived slots.
 * Written K rows hold the rotated k rounded to the element type; V rows are the
 * input's bits.  Nothing else in the pools changes.  qkv, its token stride in
 * bytes and the pools must be 16-byte aligned.  num_tokens == 0 returns PA_OK
 * without enqueuing anything.
 */
int32_t pa_qkv_rope_write(const void* qkv, int64_t qkv_token_stride,
                          const int32_t* query_start_loc, int32_t num_tokens, int32_t num_seqs,
                          const int32_t* context_lens, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, int32_t num_q_heads, float rope_theta,
                          const void* q_norm_weight, const void* k_norm_weight, float norm_eps,
                          void* q_out, void* k_pool, void* v_pool, pa_pool_desc pool,
                          int32_t* slot_mapping_out, void* stream);

/*
 * Split-context choice shared by pa_decode and pa_prefill_chunk:
 *   partition_tokens < 0   one pass per (sequence, kv head); no workspace;
 *   partition_tokens == 0  the library picks (see pa_decode_partition_tokens);
 *   partition_tokens > 0   a multiple of 16: each (sequence, kv head) is split
 *                          into chunks of that many context tokens whose
 *                          partial softmax states are merged by a second
 *                          kernel (log-sum-exp), which needs the workspace.
 *
 * pa_decode_partition_tokens returns the partition size the library uses for
 * these arguments (-1 = one pass): one pass with at least 256 (sequence, kv
 * head) units, or when one unit's K and V at the longest context
 * (max_context_len x 2 x head_dim x 2 bytes) are at most 384 KiB (a split
 * then costs more than it saves); else partitions that bring the launch to
 * about 256 workgroups.
 * pa_decode_workspace_bytes returns the workspace pa_decode needs for the same
 * arguments: the longest-first processing order (num_seqs int32, 256-byte
 * aligned) when the batch has more than 2048 sequences and uses one, then the
 * split partials; 0 when neither is used.
 */
int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t partition_tokens);
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_tokens);

/*
 * pa_decode -- one query row per sequence.
 *
 * q, out          [num_seqs, num_q_heads, head_dim]
 * k_pool, v_pool  [num_blocks, B, num_kv_heads, head_dim] (read only)
 * block_tables    int32 [num_seqs, max_blocks_per_seq]; entries past
 *                 ceil(context_len/B) are never read
 * context_lens    int32 [num_seqs]; 0 gives an all-zero output row
 * max_context_len host-side upper bound of context_lens
 * scale           multiplies q.k before the softmax (normally 1/sqrt(head_dim))
 * Supported: num_q_heads % num_kv_heads == 0 with a group size of 1..8.
 * num_seqs == 0 returns PA_OK without enqueuing anything.
 */
int32_t pa_decode(const void* q, const void* k_pool, const void* v_pool,
                  pa_pool_desc pool,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t num_seqs,
                  int32_t max_context_len, int32_t num_q_heads, float scale,
                  void* out, int32_t partition_tokens,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Arguments, results and errors as pa_decode (same
 * kernels, bit-identical output), without the workspace: what pa_decode keeps
 * in its workspace (the longest-first order of batches over 2048 sequences,
 * split-context partials) goes to a fixed 32 MiB array in device memory that
 * the library holds for each device it runs on until the process ends.
 * PA_ERR_SCRATCH, with nothing enqueued, when the call needs more than that
 * (pa_decode_workspace_bytes > 32 MiB for the same arguments).  Nothing in the
 * array needs clearing between calls (every byte a call reads, it first
 * writes).  All calls on one device share its array: calls that overlap on one
 * device (two host threads, two streams without an ordering between them)
 * race and give unspecified values; calls ordered on one stream are safe.  The
 * first call on a device that needs scratch looks the array's address up
 * (hipGetSymbolAddress, with that device current): make that first call
 * outside graph capture.
 */
int32_t pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                          pa_pool_desc pool,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_context_len, int32_t num_q_heads, float scale,
                          void* out, int32_t partition_tokens, void* stream);

/*
 * pa_decode_append -- a decode step with the step's KV-cache write fused into
 * the attention launch: the mini_engine page names the fused KV-cache write
 * as a fusion target (Next: fused kernels) and mini-vllm derives slots on the
 * GPU (Milestones, item 7).  Sequence s's new token sits at position
 * L_s - 1 (L_s = context_lens[s], which counts it); its K and V rows are
 * stored at that position's pool slot,
 *     block_tables[s][(L_s - 1) / B] * B + (L_s - 1) % B,
 * and attended as pa_decode attends, in one launch and without a slot
 * mapping.  Pools and out are bit-identical to
 *     pa_kv_write(k_new, v_new, strides, slots of those positions) + pa_decode
 * (the same arithmetic in the same order; the new rows are used from
 * registers instead of being read back).
 *
 * q, out, block_tables, context_lens, max_context_len, scale, partition
 *                 as for pa_decode (same workspace: pa_decode_workspace_bytes)
 * k_new, v_new    [num_seqs, num_kv_heads, head_dim] device rows, token s at
 *                 k_new + s * k_new_stride elements (16-byte aligned strides
 *                 >= num_kv_heads * head_dim, so views into a packed QKV
 *                 buffer work)
 * k_pool, v_pool  written at the new tokens' slots only
 * A sequence with L_s = 0 has no new token (nothing written, zero output); a
 * table entry outside [0, num_blocks) means nothing is written for that
 * sequence (as pa_kv_write skips a slot outside the pool).  Precondition
 * (unchecked): the block receiving sequence s's new token is read by no other
 * sequence of the call (a block being filled is never a shared prefix block).
 * Errors as for pa_decode, plus PA_ERR_NULL for a missing k_new / v_new and
 * PA_ERR_ALIGN for misaligned rows or strides.
 */
int32_t pa_decode_append(const void* q, const void* k_new, const void* v_new,
                         int64_t k_new_stride, int64_t v_new_stride,
                         void* k_pool, void* v_pool, pa_pool_desc pool,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs,
                         int32_t max_context_len, int32_t num_q_heads, float scale,
                         void* out, int32_t partition_tokens,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_shared_prefix -- pa_decode for groups of sequences that share a
 * prompt prefix (the blocks a prefix-cache hit points several block tables
 * at: Capstone page, Week 5 -- Prefix caching; its acceptance criteria run
 * many sequences at 8k context).  The result equals pa_decode's (within
 * rounding: the sums are ordered differently), but each group's prefix is
 * read from memory once for all its members instead of once per member.
 *
 * Arguments as pa_decode, plus:
 * group_start     int32 device [num_groups + 1]: group g is sequences
 *                 group_start[g] .. group_start[g+1]-1; group_start[0] = 0,
 *                 nondecreasing, group_start[num_groups] = num_seqs (every
 *                 sequence in one group; a group may hold one sequence)
 * prefix_lens     int32 device [num_groups]: tokens of group g's shared
 *                 prefix, taken in whole 16-token chunks (rounded down) and
 *                 clamped to max_prefix_len; every member's first
 *                 ceil(prefix/B) table entries must equal the group's first
 *                 member's, and every member's context_len must be at least
 *                 the prefix (0 = no shared prefix)
 * max_group_size  host upper bound of the group sizes (1..num_seqs)
 * max_prefix_len  host upper bound of prefix_lens (0..max_context_len)
 * partition_tokens as pa_decode, for the keys after the prefix
 * workspace       pa_decode_shared_prefix_workspace_bytes(...) bytes,
 *                 16-byte aligned; when that is 0 (no group has a prefix and
 *                 the keys run in one pass) it may be NULL
 *
 * aux             NULL, or the caller's second stream (pa_aux_stream), used
 *                 only when the keys after the prefix are split (below)
 *
 * Work: the prefix of each group is attended on the matrix cores, the group's
 * members as rows of one block that sees all of the prefix (split into key
 * parts over workgroups, each leaving partial softmax states in the
 * workspace).  Then one of two plans, by what pa_decode would do with these
 * arguments (partition_tokens, or the library's choice):
 *   one pass   the prefix phase first on `stream`, then the decode kernel
 *              reads each context after its prefix in one pass and folds the
 *              prefix's partial states into its output (no merge launch; aux
 *              is not used);
 *   split      the keys after the prefix in partitions on the decode path on
 *              `stream`, the prefix phase beside it on aux->stream (forked
 *              from and joined back into `stream`) when aux is given, else
 *              first on `stream`; a log-sum-exp merge on `stream` combines
 *              the partial states.
 * Supported: bf16 or fp16 pools (the matrix cores), group size 1..8.
 * Preconditions on the group arrays are not checked beyond memory safety:
 * rows of groups larger than max_group_size, or groups that overlap, give
 * unspecified values.
 */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t num_groups,
                                               int32_t max_group_size, int32_t max_prefix_len,
                                               int32_t partition_tokens);

int32_t pa_decode_shared_prefix(const void* q, const void* k_pool, const void* v_pool,
                                pa_pool_desc pool,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_context_len,
                                const int32_t* group_start, const int32_t* prefix_lens,
                                int32_t num_groups, int32_t max_group_size,
                                int32_t max_prefix_len, int32_t num_q_heads, float scale,
                                void* out, int32_t partition_tokens,
                                void* workspace, size_t workspace_bytes, void* stream,
                                const pa_aux_stream* aux);

/*
 * pa_prefill_chunk -- causal attention for a packed mixed batch.
 *
 * q, out            [total_query_tokens, num_q_heads, head_dim]; the rows of
 *                   sequence s are query_start_loc[s] .. query_start_loc[s+1]-1
 * query_start_loc   int32 [num_seqs + 1], non-decreasing, [0] == 0,
 *                   [num_seqs] == total_query_tokens
 * num_prefill_seqs  sequences 0 .. num_prefill_seqs-1 may have any number of
 *                   rows n <= context_len (prefill chunks); the others must
 *                   have exactly one row (decode)
 * max_query_len     host-side upper bound of the rows of any sequence
 * Row i of a sequence with n rows and context length L sits at position
 * L-n+i and attends to keys 0 .. L-n+i (causal, aligned to the context end).
 * Chunks giving at least 16 (row, head) pairs per kv head run on the matrix
 * cores; the rest, and the decode rows, run on the vector path.  When
 * matrix-core chunks and decode rows are both present and `aux` is given, the
 * vector path runs on aux->stream, concurrently with the matrix-core kernel on
 * `stream`: it waits for the work enqueued on `stream` before the call, and
 * work enqueued on `stream` after the call waits for it (event fork/join,
 * which HIP graph capture records as well).  With aux NULL every kernel runs
 * on `stream`, the matrix-core chunks first.
 * The workspace (pa_prefill_workspace_bytes) holds the decode rows' processing
 * order and split-context partials, then, 256-byte aligned, the prefill rows'
 * split-context partials; the two parts never overlap.
 */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_prefill_seqs,
                                  int32_t total_query_tokens, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_tokens);

int32_t pa_prefill_chunk(const void* q, const int32_t* query_start_loc,
                         int32_t total_query_tokens, int32_t num_seqs,
                         int32_t num_prefill_seqs, int32_t max_query_len,
                         const void* k_pool, const void* v_pool, pa_pool_desc pool,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t max_context_len,
                         int32_t num_q_heads, float scale, void* out,
                         int32_t partition_tokens,
                         void* workspace, size_t workspace_bytes, void* stream,
                         const pa_aux_stream* aux);

/*
 * Host-side block manager (no GPU involved): the block pool's free list, the
 * per-sequence block tables that the attention calls read, and the prefix
 * cache.  ("09 -- Mini Inference Engine (The Capstone)": the engine diagram's
 * KV cache manager -- block pool with free list, prefix hash -> block ids,
 * block tables per sequence; Week 4 -- a block is allocated when a sequence's
 * last block fills and every block returns on completion; Week 5 -- rolling
 * hash(previous block hash, block tokens) per full block, a global hash ->
 * block map, shared prompt blocks, reference counts, a block freed only at
 * count zero.)
 *
 * A manager owns num_blocks physical block ids of block_size tokens each
 * (8, 16 or 32 for the attention calls).  All calls are host calls and
 * thread-safe (one lock per manager); each either succeeds or changes
 * nothing.  Sequence ids are the caller's.
 *
 * pa_bm_add_sequence   a new sequence with its prompt.  With prefix caching,
 *                      the prompt's leading full blocks whose exact token prefix
 *                      is already cached (and computed) are shared instead of
 *                      allocated; *num_cached_tokens (a multiple of block_size)
 *                      tells how many prompt tokens need no recomputation.  If
 *                      every prompt token would be cached, the last block is
 *                      allocated privately and recomputed.  Blocks for the rest
 *                      of the prompt come from the free list (least recently
 *                      freed first).  PA_ERR_CAPACITY when they do not fit.
 * pa_bm_append         adds tokens (generated ones) to a sequence, allocating a
 *                      block whenever the last one fills; slots_out (or NULL)
 *                      receives each new token's flat slot, block*block_size +
 *                      offset, the pa_kv_write slot convention.
 * pa_bm_mark_computed  the caller has written the K/V of the sequence's first
 *                      num_computed_tokens tokens: full blocks among them enter
 *                      the prefix cache (unless the same prefix is cached
 *                      already).
 * pa_bm_free_sequence  every block of the sequence loses one reference; a block
 *                      at zero returns to the free list (last block first) and,
 *                      if cached, stays findable until it is taken again.
 * pa_bm_block_table    copies the sequence's block table (capacity entries at
 *                      most) and its block and token counts.
 * pa_bm_num_free_blocks blocks that can be allocated now (-1 for a NULL manager).
 * pa_bm_stats          prompt blocks found in the cache / looked up, and the
 *                      number of cache entries.
 * pa_bm_block_refcount references to one block (-1 for a bad id).
 */
typedef struct pa_block_manager pa_block_manager;

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching);
void pa_bm_destroy(pa_block_manager* m);
int32_t pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* tokens,
                           int32_t num_tokens, int32_t* num_cached_tokens);
int32_t pa_bm_append(pa_block_manager* m, int64_t seq_id, const int32_t* tokens,
                     int32_t num_tokens, int32_t* slots_out);
int32_t pa_bm_mark_computed(pa_block_manager* m, int64_t seq_id, int32_t num_computed_tokens);
int32_t pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id);
int32_t pa_bm_block_table(pa_block_manager* m, int64_t seq_id, int32_t* table_out,
                          int32_t capacity, int32_t* num_blocks_out, int32_t* num_tokens_out);
int32_t pa_bm_num_free_blocks(pa_block_manager* m);
int32_t pa_bm_stats(pa_block_manager* m, int64_t* hit_blocks, int64_t* queried_blocks,
                    int32_t* cached_blocks);
int32_t pa_bm_block_refcount(pa_block_manager* m, int32_t block_id);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
