// Launchers of the matrix-core chunk attention (bf16 or fp16, gfx950 MFMA):
// the launch shape is chosen here; the device code is in chunk_body.hpp.
#include "chunk_body.hpp"

namespace pa {
namespace {

using namespace chunk_impl;

// The chip hands workgroups to its XCDs (each with its own L2) round-robin by
// linear index.  Every row tile and key part of one (sequence, kv head) reads
// the same keys, so a launch of at least kXcds such pairs is numbered to put
// all of them on one XCD: pair c runs on XCD c % kXcds, its `tiles`
// workgroups spread over that XCD's compute units (the grid holds tiles *
// (pairs rounded up to a multiple of kXcds) workgroups; the padding ones
// exit).  With fewer pairs that numbering would leave XCDs idle, so the
// workgroups are numbered plainly, pair-major.
constexpr int kXcds = 8;

template <typename T, int D, int NT, int DEPTH, int KSPLIT>
__global__ __launch_bounds__(kRowWaves * KSPLIT * 64) void chunk_kernel(const ChunkArgs a, int tiles) {
    const int id = blockIdx.x;
    const int npairs = a.num_kv_heads * a.num_seqs;
    int pair, k;
    if (npairs >= kXcds) {
        const int x = id % kXcds;
        k = id / kXcds;
        pair = k / tiles * kXcds + x;
    } else {
        pair = id / tiles;
        k = id;  // k % tiles below is the tile
    }
    if (pair >= npairs) return;
    if constexpr (KSPLIT == 1) {
        // the tile stages, one LDS array each (the loads into them go
        // straight from memory to LDS)
        __shared__ __align__(16) unsigned char k0[stage_bytes<D>()], k1[stage_bytes<D>()], k2[stage_bytes<D>()];
        __shared__ __align__(16) unsigned char v0[stage_bytes<D>()], v1[stage_bytes<D>()], v2[stage_bytes<D>()];
        static_assert(kStages == 3, "one array per stage");
        unsigned char* const kst[kStages] = {k0, k1, k2};
        unsigned char* const vst[kStages] = {v0, v1, v2};
        chunk_block<T, D, NT, DEPTH, KSPLIT>(a, k % tiles, pair % a.num_kv_heads, pair / a.num_kv_heads, nullptr,
                                             kst, vst);
    } else {
        __shared__ __align__(16) unsigned char lds[lds_bytes<D, KSPLIT>()];
        unsigned char* const none[kStages] = {nullptr, nullptr, nullptr};
        chunk_block<T, D, NT, DEPTH, KSPLIT>(a, k % tiles, pair % a.num_kv_heads, pair / a.num_kv_heads, lds,
                                             none, none);
    }
}

// Launch shapes: 64 rows with key halves (small launches), 128 rows in one
// key range (large launches sharing the chip), 128 rows with key halves (large
// launches that run alone).
enum Shape { kSmallHalves, kLargeRange, kLargeHalves };

template <typename T, int D>
void launch_shape(const ChunkArgs& a, Shape shape, int tiles, dim3 grid, dim3 block, hipStream_t stream) {
    if (shape == kSmallHalves) hipLaunchKernelGGL((chunk_kernel<T, D, 1, kDepth, 2>), grid, block, 0, stream, a, tiles);
    else if (shape == kLargeRange) hipLaunchKernelGGL((chunk_kernel<T, D, 2, kDepth, 1>), grid, block, 0, stream, a, tiles);
    else hipLaunchKernelGGL((chunk_kernel<T, D, 2, kDepth, 2>), grid, block, 0, stream, a, tiles);
}

template <typename T>
void launch_typed(const ChunkArgs& a, Shape shape, int tiles, dim3 grid, dim3 block, hipStream_t stream) {
    if (a.head_dim == 128) launch_shape<T, 128>(a, shape, tiles, grid, block, stream);
    else launch_shape<T, 64>(a, shape, tiles, grid, block, stream);
}

}  // namespace

int32_t launch_chunks(const ChunkArgs& a, hipStream_t stream) {
    const int group = a.num_q_heads / a.num_kv_heads;
    if (!chunks_supported(a.dtype, a.head_dim, group)) return PA_ERR_UNSUPPORTED;
    if (a.num_seqs == 0 || a.max_query_len == 0) return PA_OK;
    const int64_t rows = (int64_t)a.max_query_len * group;
    const int64_t kparts = a.key_parts > 1 ? a.key_parts : 1;
    const int64_t small_tiles = (rows + kRowsSmall - 1) / kRowsSmall * kparts;
    const bool small = !a.prefer_large && small_tiles * a.num_kv_heads * a.num_seqs < kSplitBelow;
    const int64_t tiles = small ? small_tiles : (rows + kRowsLarge - 1) / kRowsLarge * kparts;
    const Shape shape = small ? kSmallHalves : (a.alone ? kLargeHalves : kLargeRange);
    const int64_t pairs = (int64_t)a.num_kv_heads * a.num_seqs;
    const int64_t blocks = tiles * (pairs >= kXcds ? (pairs + kXcds - 1) / kXcds * kXcds : pairs);
    if (blocks > INT32_MAX) return PA_ERR_SHAPE;
    const dim3 grid((unsigned)blocks);
    const dim3 block(kRowWaves * (shape == kLargeRange ? 1 : 2) * 64);
    if (a.dtype == PA_BF16) launch_typed<uint16_t>(a, shape, (int)tiles, grid, block, stream);
    else launch_typed<_Float16>(a, shape, (int)tiles, grid, block, stream);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
