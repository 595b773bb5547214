// Device code of the vector-path and matrix-core decode attention: the
// workgroup bodies (rows_block, mfma_rows_block, which take their unit index
// and LDS from the caller) and their helpers.
#pragma once

#include "pa_device.hpp"
#include "pa_internal.hpp"
#include <type_traits>

// No implicit contraction of a*b+c in the decode bodies: each body is inlined
// into several code paths (the full-block loop, the tail block, the fused
// append), and a multiply-add the compiler fuses in one copy but not in
// another would round differently, so the same block of keys would give
// different bits depending on the path that read it.  Explicit fmaf calls are
// still fused.
#pragma clang fp contract(off)

namespace pa {
namespace rows_impl {


constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;      // waves of a vector-path workgroup
constexpr int kMaxWaves = 8;   // the most waves any decode workgroup has
// Smallest GQA group that takes the matrix-core decode path (bf16).
constexpr int kMfmaMinGroup = 4;
// Fewest full steps (of two 16-token chunks) per wave for which the
// matrix-core decode may run its steps backwards.
constexpr int kRevMinSteps = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// The 16x16x32 matrix-core product for each 16-bit element type.
template <typename T>
struct Mma;
template <>
struct Mma<uint16_t> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ floatx4 mfma(v8 a, v8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ floatx4 mfma(v8 a, v8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// 16-lane transposing LDS read: lane i of each group of 16 receives element
// i%4 of the 8-byte words addressed by lanes i/4 + 4k, k = 0..3.
__device__ __forceinline__ uint2 ld_tr16(const unsigned char* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p)));
}

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
    static constexpr int kPerChunk = 8;  // bf16 bit patterns
};
template <>
struct Elem<_Float16> {
    static constexpr int kPerChunk = 8;
};
template <>
struct Elem<float> {
    static constexpr int kPerChunk = 4;
};

template <typename T>
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k) {
    if constexpr (kIs16<T>) {
        float s = dot16<T>(q.x, k.x, 0.0f);
        s = dot16<T>(q.y, k.y, s);
        s = dot16<T>(q.z, k.z, s);
        return dot16<T>(q.w, k.w, s);
    } else {
        float s = __uint_as_float(q.x) * __uint_as_float(k.x);
        s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
        s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
        return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
    }
}

template <typename T>
__device__ __forceinline__ void unpack(const uint4& c, float* v) {
    if constexpr (kIs16<T>) {
        v[0] = lo16<T>(c.x); v[1] = hi16<T>(c.x);
        v[2] = lo16<T>(c.y); v[3] = hi16<T>(c.y);
        v[4] = lo16<T>(c.z); v[5] = hi16<T>(c.z);
        v[6] = lo16<T>(c.w); v[7] = hi16<T>(c.w);
    } else {
        v[0] = __uint_as_float(c.x); v[1] = __uint_as_float(c.y);
        v[2] = __uint_as_float(c.z); v[3] = __uint_as_float(c.w);
    }
}

// Store E fp32 values (already normalised) as one 16-byte chunk of T.
template <typename T>
__device__ __forceinline__ void store_chunk(T* dst, const float* o) {
    if constexpr (kIs16<T>) {
        st16(dst, make_uint4(pack16<T>(o[0], o[1]), pack16<T>(o[2], o[3]),
                             pack16<T>(o[4], o[5]), pack16<T>(o[6], o[7])));
    } else {
        st16(dst, make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]),
                             __float_as_uint(o[2]), __float_as_uint(o[3])));
    }
}

struct Item {
    int seq;
    int item;  // index of the item (its partial-state slots)
    int row;
    int n;     // query rows of the sequence
    int i;     // this row's index among them
    bool skip; // left to the matrix-core kernel
};

// Inclusive sum over the threads of a workgroup (at most kMaxWaves waves) of
// one value per thread.  `tmp` holds one int per wave; the caller
// synchronises before reusing it.
__device__ __forceinline__ int block_inclusive_sum(int v, int* tmp) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    if (lane == 63) tmp[w] = v;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < w; ++i) before += tmp[i];
    return v + before;
}

// Longest-first order computed by every workgroup itself: the decode items
// sorted by descending bucket min(L, max_context_len) >> rank_shift (kRank
// buckets), equal buckets in index order.  Returns the item handled z-th.
// The order is a function of the lengths alone, so all workgroups of a launch
// agree on it; each pays one pass over the lengths (kRankKeep per thread, in
// registers), a histogram in LDS and two workgroup-wide sums, instead of a
// separate sorting launch ahead of the attention kernel.  Called by every
// thread of the workgroup; in a workgroup of more than kWaves waves the
// threads past the first kRankBuckets hold no items.
constexpr int kRankBuckets = kWaves * 64;  // one bucket per thread of the first kWaves waves
constexpr int kRankKeep = 8;               // items per thread
constexpr int kRankLdsInts = kRankBuckets + kMaxWaves + 2;
__device__ __forceinline__ int rank_select(const RowsArgs& a, int z, int* rank_lds) {
    int* const hist = rank_lds;                    // [kRankBuckets]
    int* const tmp = rank_lds + kRankBuckets;      // [kMaxWaves]: one per wave of any decode workgroup
    int* const pick = tmp + kMaxWaves;             // [2], past every wave's tmp entry
    static_assert(kRankBuckets + kMaxWaves + 2 <= kRankLdsInts, "pick lies past tmp[kMaxWaves - 1]");
    const int t = threadIdx.x;
    const bool owner = t < kRankBuckets;  // holds a bucket and items
    const int n = a.num_items;
    const int32_t* lens = a.context_lens + a.seq_begin;
    // thread t owns items t*kRankKeep .. t*kRankKeep+kRankKeep-1: index order
    // within a bucket follows thread order, then j
    int pos[kRankKeep];  // position of the item's bucket, longest first; -1: no item
#pragma unroll
    for (int j = 0; j < kRankKeep; ++j) {
        const int i = t * kRankKeep + j;
        const bool has = owner && i < n;
        const int L = has ? lens[i] : 0;
        const int key = min(min(max(L, 0), a.max_context_len) >> a.rank_shift, kRankBuckets - 1);
        pos[j] = has ? kRankBuckets - 1 - key : -1;
    }
    if (owner) hist[t] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRankKeep; ++j)
        if (pos[j] >= 0) atomicAdd(&hist[pos[j]], 1);
    __syncthreads();
    const int c = owner ? hist[t] : 0;
    const int incl = block_inclusive_sum(c, tmp);
    if (incl - c <= z && z < incl) {  // bucket t holds rank z
        pick[0] = t;
        pick[1] = z - (incl - c);
    }
    __syncthreads();
    const int pb = pick[0], r = pick[1];
    int m = 0;
#pragma unroll
    for (int j = 0; j < kRankKeep; ++j) m += pos[j] == pb;
    const int incl2 = block_inclusive_sum(m, tmp);  // (every thread has read pick)
    if (incl2 - m <= r && r < incl2) {              // the r-th item of bucket pb is here
        int k = r - (incl2 - m);
#pragma unroll
        for (int j = 0; j < kRankKeep; ++j) {
            if (pos[j] == pb) {
                if (k == 0) pick[0] = t * kRankKeep + j;
                --k;
            }
        }
    }
    __syncthreads();
    return pick[0];
}

// Which sequence and q/out row grid index z stands for.  Decode items read
// nothing but the processing order (in-kernel ranking or an order array); the
// context length is loaded separately so that its latency overlaps the first
// q and block-id loads.
// rank_lds: kRankLdsInts ints of LDS, used only with in-kernel ranking.
__device__ __forceinline__ Item locate(const RowsArgs& a, int z, int group, int* rank_lds) {
    Item it;
    it.skip = false;
    it.item = z;
    if (a.query_start_loc == nullptr) {
        const int zz = a.rank_shift >= 0 ? rank_select(a, z, rank_lds) : (a.order != nullptr ? a.order[z] : z);
        it.item = zz;
        it.seq = a.seq_begin + zz;
        it.row = a.row_begin + zz;
        it.n = 1;
        it.i = 0;
        return it;
    }
    const int32_t* qsl = a.query_start_loc;
    if (a.small_rows > 0) {
        it.seq = a.seq_begin + z / a.small_rows;
        it.i = z % a.small_rows;
        const int q0 = qsl[it.seq];
        it.n = qsl[it.seq + 1] - q0;
        it.row = q0 + it.i;
        it.skip = it.i >= it.n || it.n * group >= a.mfma_min_pairs;
        return it;
    }
    const int row = a.row_begin + z;
    int lo = a.seq_begin, hi = a.seq_end - 1;  // last s with qsl[s] <= row
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qsl[mid] <= row) lo = mid; else hi = mid - 1;
    }
    it.seq = lo;
    it.row = row;
    it.n = qsl[lo + 1] - qsl[lo];
    it.i = row - qsl[lo];
    it.skip = a.mfma_min_pairs > 0 && it.n * group >= a.mfma_min_pairs;
    return it;
}

// Shared-prefix mode: 16-token chunks of the prefix of sequence seq's group
// (the last group g with group_start[g] <= seq), which the chunk kernel has
// attended; the decode kernels start after them.
__device__ __forceinline__ int prefix_chunks(const RowsArgs& a, int seq) {
    int lo = 0, hi = a.num_groups - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.group_start[mid] <= seq) lo = mid; else hi = mid - 1;
    }
    return min(max(a.prefix_lens[lo], 0), a.prefix_cap) >> 4;
}

// Keys visible to the row: 0 .. L-n+i, with L clamped to what the table holds.
__device__ __forceinline__ int visible_len(const RowsArgs& a, const Item& it, int L) {
    const int cap = (int)min((int64_t)a.max_context_len, (int64_t)a.max_blocks << a.block_shift);
    L = min(max(L, 0), cap);
    return min(max(L - it.n + it.i + 1, 0), L);
}

// Workgroups are numbered with the kv head fastest, then the partition, then
// the row: the kv heads of one row and partition read the same token rows of
// the pool (each head a 2*D-byte slice of every row) at about the same time.
__device__ __forceinline__ void unit_of(const RowsArgs& a, int id, int& z, int& g, int& part) {
    const int nparts = a.part_tokens > 0 ? a.nparts - a.prefix_slots : 1;  // partitions launched
    g = id % a.num_kv_heads;
    const int rest = id / a.num_kv_heads;
    part = rest % nparts;
    z = rest / nparts;
}

// Merge the per-wave softmax states W x (m, l, acc[D]) of the G heads of one
// (row, kv head, partition) left in LDS by the W waves of the workgroup, then
// write the normalised output (final_out) or the partition's partial state for
// merge_kernel.
template <typename T, int D, int G, int W = kWaves>
__device__ __forceinline__ void combine_waves(const RowsArgs& a, const Item& it, int z, int g, int part,
                                              bool final_out, const float (&s_acc)[W][G][D],
                                              const float (&s_m)[W][G], const float (&s_l)[W][G]) {
    constexpr int E = Elem<T>::kPerChunk;
    constexpr int CPR = D / E;  // 16-byte chunks per output row
    constexpr int kFold = 8;    // prefix slots read together
    static_assert(E % 4 == 0, "whole 16-byte accumulator chunks");
    const int Hq = a.num_q_heads;
    // With a folded prefix: the prefix's key parts of this (row, q head), in
    // the first slots of its partial states (as the merge would read them).
    int npre = 0;
    if (a.fold_prefix && final_out) {
        const int pch = prefix_chunks(a, it.seq);
        npre = min((pch * kBlock + a.prefix_part_tokens - 1) / a.prefix_part_tokens, a.nparts);
    }
    const int64_t nslots = (int64_t)a.num_items * a.num_q_heads * a.nparts;
    for (int t = threadIdx.x; t < G * CPR; t += W * 64) {
        const int h = t / CPR, cc = t % CPR;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < W; ++w) M = fmaxf(M, s_m[w][h]);
        const int64_t slot0 = ((int64_t)it.item * a.num_q_heads + g * G + h) * a.nparts;
        // The prefix's slots are read kFold at a time, the loads of a group
        // issued together (one memory round trip per group, not per slot);
        // past the last slot the index is clamped to it, which leaves the
        // maximum unchanged and is given no weight below.
        const float* const pm = a.ws + nslots * D + slot0;
        const float* const pl = pm + nslots;
        for (int p0 = 0; p0 < npre; p0 += kFold) {
            float mg[kFold];
#pragma unroll
            for (int j = 0; j < kFold; ++j) mg[j] = pm[min(p0 + j, npre - 1)];
#pragma unroll
            for (int j = 0; j < kFold; ++j) M = fmaxf(M, mg[j]);
        }
        const float mref = (M == kNegInf) ? 0.0f : M;
        float den = 0.0f, o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float wt = fast_exp2(s_m[w][h] - mref);
            den = fmaf(s_l[w][h], wt, den);
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = fmaf(s_acc[w][h][cc * E + e], wt, o[e]);
        }
        for (int p0 = 0; p0 < npre; p0 += kFold) {  // the prefix's partial states, folded in
            float mg[kFold], lg[kFold];
            uint4 ag[kFold][E / 4];
#pragma unroll
            for (int j = 0; j < kFold; ++j) {
                const int p = min(p0 + j, npre - 1);
                mg[j] = pm[p];
                lg[j] = pl[p];
                const float* ap = a.ws + (slot0 + p) * D + cc * E;
#pragma unroll
                for (int k = 0; k < E / 4; ++k) ag[j][k] = ld16(ap + 4 * k);
            }
#pragma unroll
            for (int j = 0; j < kFold; ++j) {
                const float wt = (p0 + j >= npre || mg[j] == kNegInf) ? 0.0f : fast_exp2(mg[j] - mref);
                den = fmaf(lg[j], wt, den);
#pragma unroll
                for (int k = 0; k < E / 4; ++k) {
                    o[4 * k] = fmaf(__uint_as_float(ag[j][k].x), wt, o[4 * k]);
                    o[4 * k + 1] = fmaf(__uint_as_float(ag[j][k].y), wt, o[4 * k + 1]);
                    o[4 * k + 2] = fmaf(__uint_as_float(ag[j][k].z), wt, o[4 * k + 2]);
                    o[4 * k + 3] = fmaf(__uint_as_float(ag[j][k].w), wt, o[4 * k + 3]);
                }
            }
        }
        const int hq = g * G + h;
        if (final_out) {
            const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] *= inv;
            store_chunk<T>(static_cast<T*>(a.out) + ((int64_t)it.row * Hq + hq) * D + cc * E, o);
        } else {
            const int64_t slot = ((int64_t)it.item * Hq + hq) * a.nparts + part;
            float* wa = a.ws + slot * D + cc * E;
#pragma unroll
            for (int e = 0; e < E; e += 4) st16(wa + e, make_uint4(__float_as_uint(o[e]), __float_as_uint(o[e + 1]),
                                                                   __float_as_uint(o[e + 2]), __float_as_uint(o[e + 3])));
            if (cc == 0) {
                a.ws[nslots * D + slot] = M;
                a.ws[nslots * D + nslots + slot] = den;
            }
        }
    }
}

// LDS of one rows_block workgroup (W waves): the wave merge's (acc, m, l) of
// each wave and head, then the ranking's ints.
template <int D, int G, int W = kWaves>
constexpr int rows_lds_bytes() {
    return W * G * (D + 2) * 4 + kRankLdsInts * 4;
}

// One workgroup of the vector-path attention: unit `bid` of the launch (see
// unit_of), with `lds` holding rows_lds_bytes<D, G>() bytes (16-byte
// aligned).  Called by every thread of the workgroup.
template <typename T, int D, int G>
__device__ __forceinline__ void rows_block(const RowsArgs& a, int bid, unsigned char* lds) {
    constexpr int E = Elem<T>::kPerChunk;
    constexpr int V = 1;                      // 16-byte chunks per lane per token
    constexpr int EL = V * E;                 // elements per lane per token
    constexpr int R = D / EL;                 // lanes per token row
    constexpr int TPW = 64 / R;               // token rows per wave
    constexpr int NT = kBlock / TPW;          // tokens of one chunk per lane
    static_assert(TPW >= 1 && NT >= 1 && R >= 4, "lane layout");
    static_assert(8 % TPW == 0, "each lane's rows split evenly between a chunk's two halves");
    constexpr float kLazy = 8.0f;             // log2 headroom before rescaling

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane % R;
    const int rg = lane / R;
    // LDS: [acc kWaves x G x D][m kWaves x G][l kWaves x G][ranking]
    float (&s_acc)[kWaves][G][D] = *reinterpret_cast<float (*)[kWaves][G][D]>(lds);
    float (&s_m)[kWaves][G] = *reinterpret_cast<float (*)[kWaves][G]>(lds + kWaves * G * D * 4);
    float (&s_l)[kWaves][G] = *reinterpret_cast<float (*)[kWaves][G]>(lds + kWaves * G * (D + 1) * 4);
    int* const rank_lds = reinterpret_cast<int*>(lds + kWaves * G * (D + 2) * 4);
    int z, g, part;
    unit_of(a, bid, z, g, part);

    const Item it = locate(a, z, G, rank_lds);
    if (it.skip) return;
    const bool split = a.part_tokens > 0;
    const int pb = split ? a.part_tokens / kBlock : 0;
    // shared-prefix mode: the chunks after the group's prefix (split, or one pass
    // that folds the prefix's partial states into its output)
    const bool cascade = a.group_start != nullptr;
    const int b0 = (cascade ? prefix_chunks(a, it.seq) : 0) + (split ? part * pb : 0);
    const int first = b0 + wave;  // this wave's blocks: first + k*kWaves

    // Issue the length, q and first block-id loads together.
    const int Lraw = a.context_lens[it.seq];
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    // Chunk u of this lane covers elements (u*R + c)*E .. +E of the row.
    const T* qp = static_cast<const T*>(a.q) + ((int64_t)it.row * Hq + g * G) * D + c * E;
    uint4 qv[G][V];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int u = 0; u < V; ++u) qv[h][u] = ld16(qp + h * D + u * R * E);
    const bool append = a.k_new != nullptr;
    // Block ids: lane i holds the table entry behind this wave's chunk
    // kbase + i (one load per 64 chunks): the block holding the chunk (blocks
    // of 16 or 32), or the first of its two blocks with the second in ids_hi
    // (blocks of 8).
    const int32_t* bt = a.block_tables + (int64_t)it.seq * a.max_blocks;
    const int bsh = a.block_shift;
    const ChunkMap cm = chunk_map(bsh);
    int ids = 0, ids_hi = 0;
    auto fetch_ids = [&](int kbase) {
        const int jj = first + (kbase + lane) * kWaves;
        ids = bt[min((jj << cm.mul) >> cm.shr, a.max_blocks - 1)];
        ids_hi = bt[min(((jj << cm.mul) + cm.mul) >> cm.shr, a.max_blocks - 1)];
    };
    fetch_ids(0);

    const int len = visible_len(a, it, Lraw);
    const int nblk = (len + kBlock - 1) / kBlock;
    int b1 = nblk;
    bool final_out = true;
    if (split) {
        b1 = min(nblk, b0 + pb);
        // the merge ignores missing partitions
        if (b0 >= b1 && (cascade || !(part == 0 && nblk == 0))) return;
        final_out = !cascade && nblk <= pb;  // a single partition writes the output itself
    }

    float m[G], l[G], acc[G][EL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegInf;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[h][e] = 0.0f;
    }

    // This wave's blocks are jb = first + k*kWaves, k < nk; blocks below
    // len/16 are full, and only the sequence's last block can be partial.  In
    // append mode the block holding position len-1 also takes the tail path,
    // which puts the new token in.
    const int nk = b1 > first ? (b1 - first + kWaves - 1) / kWaves : 0;
    const int nfull = (append ? max(len - 1, 0) : len) / kBlock;
    const int nkf = nfull > first ? min(nk, (nfull - first + kWaves - 1) / kWaves) : 0;
    // First pool rows of chunk k's tokens 0-7 (lo) and 8-15 (hi); ids are
    // clamped into the pool.
    auto chunk_rows = [&](int k, int64_t& lo, int64_t& hi) {  // ids of chunk k already fetched
        const int bl = min(max(__builtin_amdgcn_readlane(ids, k & 63), 0), a.num_blocks - 1);
        const int bh = min(max(__builtin_amdgcn_readlane(ids_hi, k & 63), 0), a.num_blocks - 1);
        const int off = ((first + k * kWaves) << 4) & cm.in_block;
        lo = ((int64_t)bl << bsh) + off;
        hi = ((int64_t)bh << bsh) + off + cm.hi_off;
    };
    auto rows_of = [&](int k, int64_t& lo, int64_t& hi) {
        if ((k & 63) == 0 && k != 0) fetch_ids(k);
        chunk_rows(k, lo, hi);
    };

    const int64_t tok_stride = (int64_t)Hkv * D;  // elements between tokens
    const T* kbase = static_cast<const T*>(a.k_pool) + (int64_t)g * D + c * E + rg * tok_stride;
    const T* vbase = static_cast<const T*>(a.v_pool) + (int64_t)g * D + c * E + rg * tok_stride;
    const float sl2 = a.scale * kLog2e;

    auto load = [&](uint4 (&kk)[NT][V], uint4 (&vv)[NT][V], int k) {
        int64_t lo, hi;
        rows_of(k, lo, hi);
        // element offsets of the chunk's rows 0 and 8 (wave-uniform)
        const int64_t o_lo = lo * tok_stride, o_hi = (hi - 8) * tok_stride;
        // rows of the chunk inside the visible context (wave-uniform): 16 or
        // more except in the sequence's last, partial block
        const int lim = len - (first + k * kWaves) * kBlock;
        if (lim >= kBlock) {
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    // this lane's row rg + i*TPW of the chunk is in its first half iff i*TPW < 8
                    const int64_t o = (i * TPW < 8 ? o_lo : o_hi) + (i * TPW) * tok_stride + u * R * E;
                    kk[i][u] = ld16_stream(kbase + o);
                    vv[i][u] = ld16_stream(vbase + o);
                }
        } else {
            // The partial last block: rows at or past the end of the context
            // are not loaded (they take no part in the result: compute()
            // masks their scores and zeroes their V rows), which saves their
            // bytes of memory traffic.
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    const int64_t o = (i * TPW < 8 ? o_lo : o_hi) + (i * TPW) * tok_stride + u * R * E;
                    uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
                    if (rg + i * TPW < lim) {
                        kx = ld16_stream(kbase + o);
                        vx = ld16_stream(vbase + o);
                    }
                    kk[i][u] = kx;
                    vv[i][u] = vx;
                }
        }
    };
    auto compute = [&](const uint4 (&kk)[NT][V], const uint4 (&vv)[NT][V], int k, bool masked) {
        bool valid[NT];
        const int tok0 = (first + k * kWaves) * kBlock + rg;
#pragma unroll
        for (int i = 0; i < NT; ++i) valid[i] = !masked || tok0 + i * TPW < len;
        float sc[NT][G];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = chunk_dot<T>(qv[h][0], kk[i][0]);
#pragma unroll
                for (int u = 1; u < V; ++u) d += chunk_dot<T>(qv[h][u], kk[i][u]);
                d = group_sum<R>(d) * sl2;
                // excluded, never weighted by zero: past-the-length slots may hold NaN
                sc[i][h] = valid[i] ? d : kNegInf;
            }
        float vf[NT][EL];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int u = 0; u < V; ++u) {
                const uint4 w = valid[i] ? vv[i][u] : make_uint4(0, 0, 0, 0);
                unpack<T>(w, &vf[i][u * E]);
            }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mb = sc[0][h];
#pragma unroll
            for (int i = 1; i < NT; ++i) mb = fmaxf(mb, sc[i][h]);
            if (mb > m[h] + kLazy) {  // raise the reference and rescale
                const float alpha = fast_exp2(m[h] - mb);
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < EL; ++e) acc[h][e] *= alpha;
                m[h] = mb;
            }
            const float mref = (m[h] == kNegInf) ? 0.0f : m[h];
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const float p = fast_exp2(sc[i][h] - mref);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < EL; ++e) acc[h][e] = fmaf(p, vf[i][e], acc[h][e]);
            }
        }
    };

    // Full blocks, two register buffers: the next block's loads are in flight
    // while the current one is computed.  The load at the end of the loop
    // fetches block k + 2 when this wave has one, which with an even number
    // of full blocks is the partial tail block, then in flight when the loop
    // ends.  (With an odd number the tail is loaded after the last full
    // block: a second live buffer for it costs registers, and with them
    // occupancy, on several shapes.)  A wave with nothing left to fetch loads
    // nothing: re-reading its last block instead (a load that is always
    // issued) cost about one 8 KiB block of HBM traffic per workgroup, 1.5%
    // of the headline batch's bytes, as the K and V loads are non-temporal.
    uint4 ka[NT][V], va[NT][V], kb[NT][V], vb[NT][V];
    const int last = nk - 1;
    int k = 0;
    if (nkf > 0) load(ka, va, 0);
    for (; k + 1 < nkf; k += 2) {
        load(kb, vb, k + 1);
        compute(ka, va, k, false);
        if (k + 2 <= last) load(ka, va, k + 2);
        compute(kb, vb, k + 1, false);
    }
    const bool tail_loaded = nkf > 0 && k == nkf;  // the loop's last load was block nkf
    if (k < nkf) {
        compute(ka, va, k, false);
        ++k;
    }
    if (k < nk && !tail_loaded) load(ka, va, k);
    if (k < nk) {  // the partial last block (or, appending, the one holding the new token), in ka
        if (append && ((len - 1) >> 4) == first + k * kWaves) {
            // The new token's K and V row (this lane's chunks) replace what
            // the pool holds at position len-1 and are stored there.  A table
            // entry outside the pool gets neither (the read stays clamped, as
            // pa_decode after a pa_kv_write that skipped the slot would see
            // it).  Only this wave of this workgroup touches that row's slice
            // of kv head g.
            const T* kn = static_cast<const T*>(a.k_new) + it.seq * a.k_new_stride + (int64_t)g * D + c * E;
            const T* vn = static_cast<const T*>(a.v_new) + it.seq * a.v_new_stride + (int64_t)g * D + c * E;
            uint4 knew[V], vnew[V];
#pragma unroll
            for (int u = 0; u < V; ++u) {
                knew[u] = ld16(kn + u * R * E);
                vnew[u] = ld16(vn + u * R * E);
            }
            const int row = (len - 1) & 15;  // row of the chunk
            const int raw = __builtin_amdgcn_readlane(row < 8 ? ids : ids_hi, k & 63);
            const bool in_pool = raw >= 0 && raw < a.num_blocks;
            int64_t lo, hi;
            chunk_rows(k, lo, hi);
            const int64_t o_lo = lo * tok_stride, o_hi = (hi - 8) * tok_stride;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                if (!in_pool || rg + i * TPW != row) continue;
                const int64_t o = (i * TPW < 8 ? o_lo : o_hi) + (i * TPW) * tok_stride;
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    ka[i][u] = knew[u];
                    va[i][u] = vnew[u];
                    st16(const_cast<T*>(kbase) + o + u * R * E, knew[u]);
                    st16(const_cast<T*>(vbase) + o + u * R * E, vnew[u]);
                }
            }
        }
        compute(ka, va, k, true);
    }

    // Merge the lane groups of this wave (they hold disjoint token subsets).
#pragma unroll
    for (int o = R; o < 64; o <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], o);
            const float lo = __shfl_xor(l[h], o);
            const float mn = fmaxf(m[h], mo);
            const float mref = (mn == kNegInf) ? 0.0f : mn;
            const float a1 = fast_exp2(m[h] - mref), a2 = fast_exp2(mo - mref);
            l[h] = l[h] * a1 + lo * a2;
#pragma unroll
            for (int e = 0; e < EL; ++e) {
                const float ao = __shfl_xor(acc[h][e], o);
                acc[h][e] = acc[h][e] * a1 + ao * a2;
            }
            m[h] = mn;
        }
    }

    // Merge the waves through LDS, then write the output or the partial state.
    if (rg == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < EL; ++e) s_acc[wave][h][((e / E) * R + c) * E + e % E] = acc[h][e];
            if (c == 0) {
                s_m[wave][h] = m[h];
                s_l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();
    combine_waves<T, D, G>(a, it, z, g, a.prefix_slots + part, final_out, s_acc, s_m, s_l);
}

// Decode rows on the matrix cores, for large GQA groups (bf16).  Same work
// unit, partitions, processing order and wave merge as rows_kernel; the
// per-token arithmetic moves to v_mfma_f32_16x16x32_bf16 so that the vector
// units no longer pay G dot products, reductions and FMAs per loaded byte.
// Each wave streams its own 32-token steps (two blocks):
//   S^T = K * Q^T    A = the K rows straight from memory (lane l: token l%16,
//                    dims 32*ks + 8*(l/16) .. +7), B = the group's q rows
//                    (heads padded to 16 with zeros) held in registers; lane
//                    l ends with head l%16's scores for tokens 16*mt +
//                    4*(l/16) + r.
//   O^T += V^T P^T   B = those probabilities (slot p < 4: token 4*(l/16)+p,
//                    p >= 4: 16+4*(l/16)+p-4), A = V^T read with
//                    ds_read_b64_tr_b16 from the wave's own row-major V tile in
//                    LDS (written with 16-byte stores; no barrier needed, the
//                    tile is private to the wave).
// LDS of one mfma_rows_block workgroup of W waves: each wave's V tile, then
// the wave merge's (acc, m, l) and the ranking's ints.
template <int D, int G, int W>
constexpr int mfma_rows_lds_bytes() {
    return W * 32 * (D * 2 + 32) + rows_lds_bytes<D, G, W>();
}

// One workgroup of W waves of the matrix-core decode path: unit `bid` of the
// launch, with `lds` holding mfma_rows_lds_bytes<D, G, W>() bytes (16-byte
// aligned).  Called
// by every thread of the workgroup.
template <typename T, int D, int G, int W>
__device__ __forceinline__ void mfma_rows_block(const RowsArgs& a, int bid, unsigned char* lds) {
    using V8 = typename Mma<T>::v8;
    constexpr int KS = D / 32;                // 32-dim slices (first product)
    constexpr int MT = D / 16;                // 16-dim output tiles (second product)
    constexpr int CPR = D / 8;                // 16-byte chunks per token row
    constexpr int VL = 32 * CPR / 64;         // V chunks per lane per step
    constexpr int VROW = D * 2 + 32;          // LDS bytes per V row (padded: the
                                              // transposing reads take 4 rows x 32 B)
    constexpr int VT = 32 * VROW;             // one wave's V tile
    constexpr float kLazy = 8.0f;
    static_assert(G <= 16, "group fits the 16 columns of one MFMA tile");
    static_assert(W <= kMaxWaves, "the ranking's LDS holds one partial sum per wave");
    // LDS: [V tiles W x VT][acc W x G x D][m][l][ranking]
    unsigned char* const s_v = lds;
    unsigned char* const rl = lds + W * VT;
    float (&s_acc)[W][G][D] = *reinterpret_cast<float (*)[W][G][D]>(rl);
    float (&s_m)[W][G] = *reinterpret_cast<float (*)[W][G]>(rl + W * G * D * 4);
    float (&s_l)[W][G] = *reinterpret_cast<float (*)[W][G]>(rl + W * G * (D + 1) * 4);
    int* const rank_lds = reinterpret_cast<int*>(rl + W * G * (D + 2) * 4);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, kg = lane >> 4;
    int z, g, part;
    unit_of(a, bid, z, g, part);
    const Item it = locate(a, z, G, rank_lds);
    if (it.skip) return;
    const bool split = a.part_tokens > 0;
    const int pb = split ? a.part_tokens / kBlock : 0;
    // shared-prefix mode: the chunks after the group's prefix (split, or one pass
    // that folds the prefix's partial states into its output)
    const bool cascade = a.group_start != nullptr;
    const int b0 = (cascade ? prefix_chunks(a, it.seq) : 0) + (split ? part * pb : 0);

    const int Lraw = a.context_lens[it.seq];
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    V8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (li < G)
            v = ld16(static_cast<const T*>(a.q) + ((int64_t)it.row * Hq + g * G + li) * D + ks * 32 + kg * 8);
        qf[ks] = __builtin_bit_cast(V8, v);
    }
    const bool append = a.k_new != nullptr;
    // Block ids: lane i holds the table entry behind chunk
    // b0 + 2*(wave + (kbase + i/2)*W) + i%2 (as in rows_kernel: blocks of
    // 8 keep the chunk's second block in ids_hi).
    const int32_t* bt = a.block_tables + (int64_t)it.seq * a.max_blocks;
    const int bsh = a.block_shift;
    const ChunkMap cm = chunk_map(bsh);
    int ids = 0, ids_hi = 0;
    // Step k of the loop attends step step_of(k) of this wave: the full steps
    // run backwards (last to first) in a long context whose table ends on an
    // odd physical block, forwards otherwise; the tail step always comes last.
    bool rev = false;
    int nkf_rev = 0;
    auto step_of = [&](int k) { return rev && k < nkf_rev ? nkf_rev - 1 - k : k; };
    auto fetch_ids = [&](int kbase) {
        const int jj = b0 + 2 * (wave + step_of(kbase + (lane >> 1)) * W) + (lane & 1);
        ids = bt[min((jj << cm.mul) >> cm.shr, a.max_blocks - 1)];
        ids_hi = bt[min(((jj << cm.mul) + cm.mul) >> cm.shr, a.max_blocks - 1)];
    };
    fetch_ids(0);

    const int len = visible_len(a, it, Lraw);
    const int nblk = (len + kBlock - 1) / kBlock;
    int b1 = nblk;
    bool final_out = true;
    if (split) {
        b1 = min(nblk, b0 + pb);
        if (b0 >= b1 && (cascade || !(part == 0 && nblk == 0))) return;
        final_out = !cascade && nblk <= pb;
    }
    // Steps of this wave: pair k covers blocks jb = b0 + 2*(wave + k*W)
    // and jb + 1; the steps with both blocks full come first, then at most one
    // step that needs masking.
    const int first = b0 + 2 * wave;
    const int nk = b1 > first ? (b1 - first + 2 * W - 1) / (2 * W) : 0;
    // blocks below this are full (appending, the block holding position len-1
    // takes the tail step, which puts the new token in)
    const int full_end = min(b1, (append ? max(len - 1, 0) : len) / kBlock);
    const int nkf = full_end >= first + 2 ? min(nk, (full_end - first - 2) / (2 * W) + 1) : 0;
    // Direction of the full steps.  In a batch whose sequences share a long
    // prefix, a unit reads the prefix (shared: from the caches, after the
    // first reader) and then its own blocks (from HBM); if every unit went in
    // the same direction, the whole chip would first read from the caches
    // and then stream from HBM.  Running about half of the long units
    // backwards (by the parity of the last table entry of the context, a
    // property of the sequence, so its result does not depend on the rest of
    // the batch) overlaps the two (measured: the long-context batch's
    // pa_decode 130 -> 127 us).  Short contexts keep the forward order, whose
    // first ids are already on their way.
    if (nkf >= kRevMinSteps) {
        const int last_id = bt[min(((nblk - 1) << cm.mul) >> cm.shr, a.max_blocks - 1)];
        rev = (__builtin_amdgcn_readfirstlane(last_id) & 1) != 0;
        nkf_rev = nkf;
        if (rev) fetch_ids(0);
    }
    // First pool rows of the step's chunk `half`, tokens 0-7 (lo) and 8-15 (hi).
    auto chunk_rows = [&](int k, int half, int64_t& lo, int64_t& hi) {  // ids already fetched
        const int ln = ((k & 31) << 1) | half;
        const int bl = min(max(__builtin_amdgcn_readlane(ids, ln), 0), a.num_blocks - 1);
        const int bh = min(max(__builtin_amdgcn_readlane(ids_hi, ln), 0), a.num_blocks - 1);
        const int off = ((first + 2 * W * step_of(k) + half) << 4) & cm.in_block;
        lo = ((int64_t)bl << bsh) + off;
        hi = ((int64_t)bh << bsh) + off + cm.hi_off;
    };
    auto rows_of = [&](int k, int half, int64_t& lo, int64_t& hi) {
        if ((k & 31) == 0 && k != 0 && half == 0) fetch_ids(k);
        chunk_rows(k, half, lo, hi);
    };

    const int64_t tok_stride = (int64_t)Hkv * D;
    const T* kpool = static_cast<const T*>(a.k_pool) + (int64_t)g * D;
    const T* vpool = static_cast<const T*>(a.v_pool) + (int64_t)g * D;
    constexpr int TPS = 64 / CPR;  // V rows one 64-lane slice covers
    static_assert(8 % TPS == 0, "a V slice stays inside half a chunk");
    const int k_lane = li * (int)tok_stride + kg * 8;                             // K row li, column
    const int v_lane = (lane / CPR) * (int)tok_stride + (lane % CPR) * 8;          // V row, column
    unsigned char* vt = s_v + wave * VT;
    const float sl2 = a.scale * kLog2e;

    float m = kNegInf, lsum = 0.0f;
    floatx4 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    auto load = [&](uint4 (&kf)[2][KS], uint4 (&vr)[VL], int k) {
        const int jb = first + 2 * W * step_of(k);
        int64_t lo0, hi0, lo1, hi1;
        rows_of(k, 0, lo0, hi0);
        if (jb + 1 < b1) {
            rows_of(k, 1, lo1, hi1);
        } else {
            lo1 = lo0;
            hi1 = hi0;
        }
        // Wave-uniform element offsets of rows 0 and 8 of both chunks; the
        // lanes add their own (loop-invariant) row and column offsets.
        const int64_t o_lo0 = lo0 * tok_stride, o_hi0 = (hi0 - 8) * tok_stride;
        const int64_t o_lo1 = lo1 * tok_stride, o_hi1 = (hi1 - 8) * tok_stride;
        // K: lane row li of chunk mt lies in the chunk's first half iff li < 8.
        // One K load takes 64 bytes of each of 16 rows (half a 128-byte line);
        // the next slice takes the other half, so these loads are ordinary
        // (cached) loads: measured 7-10% faster than non-temporal ones, with
        // which the second half went back to memory.  V loads take whole rows
        // and stay non-temporal (cached V measured slower).
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const T* kp = kpool + (mt ? (li < 8 ? o_lo1 : o_hi1) : (li < 8 ? o_lo0 : o_hi0));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kf[mt][ks] = ld16(kp + k_lane + ks * 32);
        }
        // V: slice u covers step tokens u*TPS .. u*TPS+TPS-1, all in one half
        // of one chunk (known at compile time)
#pragma unroll
        for (int u = 0; u < VL; ++u) {
            const int t0 = u * TPS;
            const int64_t o = (t0 >> 4) ? ((t0 & 15) < 8 ? o_lo1 : o_hi1) : ((t0 & 15) < 8 ? o_lo0 : o_hi0);
            vr[u] = ld16_stream(vpool + o + (int64_t)(t0 & 15) * tok_stride + v_lane);
        }
    };
    auto compute = [&](const uint4 (&kf)[2][KS], const uint4 (&vr)[VL], int k, bool masked) {
        const int pos0 = (first + 2 * W * step_of(k)) * kBlock;  // first token of the step
        const int pend = min(len, b1 * kBlock);              // tokens at or past this are excluded
#pragma unroll
        for (int u = 0; u < VL; ++u) {
            const int c = lane + 64 * u, tk = c / CPR, piece = c % CPR;
            // excluded tokens are zeroed, never weighted by zero (their slots may hold NaN)
            const uint4 w = (!masked || pos0 + tk < pend) ? vr[u] : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(vt + tk * VROW + piece * 16) = w;
        }
        floatx4 st[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            floatx4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) c = Mma<T>::mfma(__builtin_bit_cast(V8, kf[mt][ks]), qf[ks], c);
            st[mt] = c;
        }
        float sc[8];
        float mx = kNegInf;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = st[mt][r] * sl2;
                const bool ok = !masked || pos0 + mt * 16 + kg * 4 + r < pend;
                sc[mt * 4 + r] = ok ? v : kNegInf;
                mx = fmaxf(mx, sc[mt * 4 + r]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (mx > m + kLazy) {  // raise the reference and rescale
            const float alpha = fast_exp2(m - mx);
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[i] *= alpha;
            m = mx;
        }
        const float mref = (m == kNegInf) ? 0.0f : m;
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // the sum takes the probabilities as rounded for the product
            const uint32_t lo = to16<T>(fast_exp2(sc[2 * i] - mref));
            const uint32_t hi = to16<T>(fast_exp2(sc[2 * i + 1] - mref));
            lsum += lo16<T>(lo) + lo16<T>(hi);
            pk[i] = lo | (hi << 16);
        }
        const V8 pb = __builtin_bit_cast(V8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's V tile is in LDS
        const unsigned char* v0 = vt + (4 * kg + ((lane >> 2) & 3)) * VROW + (lane & 3) * 8;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint2 lo = ld_tr16(v0 + mt * 32);
            const uint2 hi = ld_tr16(v0 + 16 * VROW + mt * 32);
            acc[mt] = Mma<T>::mfma(__builtin_bit_cast(V8, make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, acc[mt]);
        }
    };

    // Two register buffers, as in rows_block: the load at the end of the loop
    // fetches step k + 2 when this wave has one, so with an even number of
    // full steps the tail step is in flight when the loop ends, and a wave
    // with nothing left loads nothing.  (With an odd number the tail is
    // loaded after the last full step: a second live buffer for it would push
    // this kernel past 256 registers.)
    uint4 ka[2][KS], va[VL], kb[2][KS], vb[VL];
    const int last = nk - 1;
    int k = 0;
    if (nkf > 0) load(ka, va, 0);
    for (; k + 1 < nkf; k += 2) {
        load(kb, vb, k + 1);
        compute(ka, va, k, false);
        if (k + 2 <= last) load(ka, va, k + 2);
        compute(kb, vb, k + 1, false);
    }
    const bool tail_loaded = nkf > 0 && k == nkf;  // the loop's last load was step nkf
    if (k < nkf) {
        compute(ka, va, k, false);
        ++k;
    }
    if (k < nk && !tail_loaded) load(ka, va, k);
    if (k < nk) {  // the step holding the partial block and/or the partition end, in ka
        const int jb = first + 2 * W * k, tc = (len - 1) >> 4;
        if (append && (tc == jb || (tc == jb + 1 && jb + 1 < b1))) {
            // The new token's K and V row replace what the pool holds at
            // position len-1 and are stored there; a table entry outside the
            // pool gets neither (as in the vector path).  K: lanes of row
            // `row` of chunk mt hold columns ks*32 + kg*8; V: the lanes whose
            // step token is mt*16 + row hold piece lane % CPR.  (Requested
            // here: kept in registers from the start, they push this kernel
            // past 256 registers.)
            const T* kn = static_cast<const T*>(a.k_new) + it.seq * a.k_new_stride + (int64_t)g * D;
            const T* vn = static_cast<const T*>(a.v_new) + it.seq * a.v_new_stride + (int64_t)g * D;
            uint4 knew[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) knew[ks] = ld16(kn + ks * 32 + kg * 8);
            const uint4 vnew = ld16(vn + (lane % CPR) * 8);
            const int mt = tc - jb, row = (len - 1) & 15;
            const int raw = __builtin_amdgcn_readlane(row < 8 ? ids : ids_hi, ((k & 31) << 1) | mt);
            const bool in_pool = raw >= 0 && raw < a.num_blocks;
            int64_t lo, hi;
            chunk_rows(k, mt, lo, hi);
            const int64_t orow = (row < 8 ? lo * tok_stride : (hi - 8) * tok_stride) + (int64_t)row * tok_stride;
            if (in_pool && li == row) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (mt == 0) ka[0][ks] = knew[ks];
                    else ka[1][ks] = knew[ks];
                    st16(const_cast<T*>(kpool) + orow + kg * 8 + ks * 32, knew[ks]);
                }
            }
#pragma unroll
            for (int u = 0; u < VL; ++u) {
                if (!in_pool || (lane + 64 * u) / CPR != mt * 16 + row) continue;
                va[u] = vnew;
                st16(const_cast<T*>(vpool) + orow + (lane % CPR) * 8, vnew);
            }
        }
        compute(ka, va, k, true);
    }

    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (li < G) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_acc[wave][li][mt * 16 + kg * 4 + r] = acc[mt][r];
        if (kg == 0) {
            s_m[wave][li] = m;
            s_l[wave][li] = lsum;
        }
    }
    __syncthreads();
    combine_waves<T, D, G, W>(a, it, z, g, a.prefix_slots + part, final_out, s_acc, s_m, s_l);
}

}  // namespace rows_impl
}  // namespace pa
