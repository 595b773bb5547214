// Vector-path attention over a paged KV pool: decode rows, and prefill rows
// too short for the matrix cores.
//
// Work unit: one workgroup per (query row, kv head, context partition).  The
// G = Hq/Hkv query heads of the kv head share every K/V row the workgroup
// loads, so each K/V byte crosses HBM once per (row, kv head).  Context
// partitions (split-context, flash-decoding style) give a long or ragged batch
// enough workgroups; their partial softmax states are merged by merge_kernel.
//
// Lane layout inside a wave: a token's [head_dim] row of K (or V) is R
// 16-byte chunks, so R consecutive lanes hold one token and a wave covers
// 64/R tokens per load.  A block of 16 tokens is NT = 16*R/64 loads per lane.
// Each lane group of R lanes keeps its own running max / sum / accumulator
// (fp32 online softmax); the groups, then the waves, are merged at the end.
// q.k partial sums are reduced across the R lanes with DPP row operations.
#include "pa_device.hpp"
#include "pa_internal.hpp"

#include <type_traits>

namespace pa {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
    static constexpr int kPerChunk = 8;  // bf16 bit patterns
};
template <>
struct Elem<float> {
    static constexpr int kPerChunk = 4;
};

template <typename T>
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k) {
    if constexpr (std::is_same_v<T, uint16_t>) {
        float s = dot2_bf16(q.x, k.x, 0.0f);
        s = dot2_bf16(q.y, k.y, s);
        s = dot2_bf16(q.z, k.z, s);
        return dot2_bf16(q.w, k.w, s);
    } else {
        float s = __uint_as_float(q.x) * __uint_as_float(k.x);
        s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
        s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
        return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
    }
}

template <typename T>
__device__ __forceinline__ void unpack(const uint4& c, float* v) {
    if constexpr (std::is_same_v<T, uint16_t>) {
        v[0] = bf_lo(c.x); v[1] = bf_hi(c.x);
        v[2] = bf_lo(c.y); v[3] = bf_hi(c.y);
        v[4] = bf_lo(c.z); v[5] = bf_hi(c.z);
        v[6] = bf_lo(c.w); v[7] = bf_hi(c.w);
    } else {
        v[0] = __uint_as_float(c.x); v[1] = __uint_as_float(c.y);
        v[2] = __uint_as_float(c.z); v[3] = __uint_as_float(c.w);
    }
}

// Store E fp32 values (already normalised) as one 16-byte chunk of T.
template <typename T>
__device__ __forceinline__ void store_chunk(T* dst, const float* o) {
    if constexpr (std::is_same_v<T, uint16_t>) {
        st16(dst, make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                             pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])));
    } else {
        st16(dst, make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]),
                             __float_as_uint(o[2]), __float_as_uint(o[3])));
    }
}

struct Item {
    int seq;
    int row;
    int len;   // keys visible to this row
    bool skip; // left to the matrix-core kernel
};

__device__ __forceinline__ Item resolve(const RowsArgs& a, int z, int group) {
    Item it;
    it.skip = false;
    const int cap = min(a.max_context_len, a.max_blocks * kBlock);
    if (a.query_start_loc == nullptr) {
        it.seq = a.seq_begin + z;
        it.row = a.row_begin + z;
        it.len = min(max(a.context_lens[it.seq], 0), cap);
        return it;
    }
    const int row = a.row_begin + z;
    const int32_t* qsl = a.query_start_loc;
    int lo = a.seq_begin, hi = a.seq_end - 1;  // last s with qsl[s] <= row
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qsl[mid] <= row) lo = mid; else hi = mid - 1;
    }
    const int n = qsl[lo + 1] - qsl[lo];
    const int i = row - qsl[lo];
    const int L = min(max(a.context_lens[lo], 0), cap);
    it.seq = lo;
    it.row = row;
    it.len = min(max(L - n + i + 1, 0), L);
    it.skip = a.mfma_min_pairs > 0 && n * group >= a.mfma_min_pairs;
    return it;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kWaves * 64) void rows_kernel(const RowsArgs a) {
    constexpr int E = Elem<T>::kPerChunk;
    constexpr int R = D / E;          // lanes per token row
    constexpr int TPW = 64 / R;       // token rows per wave load
    constexpr int NT = kBlock / TPW;  // tokens of one block per lane
    static_assert(TPW >= 1 && NT >= 1, "lane layout");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane % R;
    const int rg = lane / R;
    const int z = blockIdx.x, g = blockIdx.y, part = blockIdx.z;

    const Item it = resolve(a, z, G);
    if (it.skip) return;
    const int nblk = (it.len + kBlock - 1) / kBlock;
    const bool split = a.part_tokens > 0;
    int b0 = 0, b1 = nblk;
    if (split) {
        const int pb = a.part_tokens / kBlock;
        b0 = part * pb;
        b1 = min(nblk, b0 + pb);
        if (b0 >= b1) return;  // the merge kernel ignores missing partitions
    }

    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const T* qp = static_cast<const T*>(a.q) + ((int64_t)it.row * Hq + g * G) * D + c * E;
    uint4 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = ld16(qp + h * D);

    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegInf;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
    }

    const int32_t* bt = a.block_tables + (int64_t)it.seq * a.max_blocks;
    const int64_t tok_stride = (int64_t)Hkv * D;  // elements between tokens
    const T* kbase = static_cast<const T*>(a.k_pool) + (int64_t)g * D + c * E + rg * tok_stride;
    const T* vbase = static_cast<const T*>(a.v_pool) + (int64_t)g * D + c * E + rg * tok_stride;
    const float sl2 = a.scale * kLog2e;

    for (int jb = b0 + wave; jb < b1; jb += kWaves) {
        const int blk = min(max(bt[jb], 0), a.num_blocks - 1);
        const int64_t off = (int64_t)blk * kBlock * tok_stride;
        uint4 kc[NT], vc[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            kc[i] = ld16(kbase + off + (int64_t)(i * TPW) * tok_stride);
            vc[i] = ld16(vbase + off + (int64_t)(i * TPW) * tok_stride);
        }
        float sc[NT][G];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int h = 0; h < G; ++h) sc[i][h] = group_sum<R>(chunk_dot<T>(qv[h], kc[i])) * sl2;

        if ((jb + 1) * kBlock > it.len) {  // last block: mask tokens past the length
            const int tok0 = jb * kBlock + rg;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const bool valid = tok0 + i * TPW < it.len;
#pragma unroll
                for (int h = 0; h < G; ++h) sc[i][h] = valid ? sc[i][h] : kNegInf;
                vc[i] = valid ? vc[i] : make_uint4(0, 0, 0, 0);
            }
        }
        float vf[NT][E];
#pragma unroll
        for (int i = 0; i < NT; ++i) unpack<T>(vc[i], vf[i]);

#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mb = sc[0][h];
#pragma unroll
            for (int i = 1; i < NT; ++i) mb = fmaxf(mb, sc[i][h]);
            const float mn = fmaxf(m[h], mb);
            const float mref = (mn == kNegInf) ? 0.0f : mn;
            const float alpha = fast_exp2(m[h] - mref);
            l[h] *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const float p = fast_exp2(sc[i][h] - mref);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, vf[i][e], acc[h][e]);
            }
            m[h] = mn;
        }
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
            for (int e = 0; e < E; ++e) {
                const float ao = __shfl_xor(acc[h][e], o);
                acc[h][e] = acc[h][e] * a1 + ao * a2;
            }
            m[h] = mn;
        }
    }

    // Merge the waves through LDS, then write the output or the partial state.
    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];
    if (rg == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < E; ++e) s_acc[wave][h][c * E + e] = acc[h][e];
            if (c == 0) {
                s_m[wave][h] = m[h];
                s_l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < G * R; t += kWaves * 64) {
        const int h = t / R, cc = t % R;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
        const float mref = (M == kNegInf) ? 0.0f : M;
        float den = 0.0f, o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float wt = fast_exp2(s_m[w][h] - mref);
            den = fmaf(s_l[w][h], wt, den);
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = fmaf(s_acc[w][h][cc * E + e], wt, o[e]);
        }
        const int hq = g * G + h;
        if (!split) {
            const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] *= inv;
            store_chunk<T>(static_cast<T*>(a.out) + ((int64_t)it.row * Hq + hq) * D + cc * E, o);
        } else {
            const int64_t slot = ((int64_t)z * Hq + hq) * a.nparts + part;
            float* wa = a.ws + slot * D + cc * E;
#pragma unroll
            for (int e = 0; e < E; e += 4) st16(wa + e, make_uint4(__float_as_uint(o[e]), __float_as_uint(o[e + 1]),
                                                                   __float_as_uint(o[e + 2]), __float_as_uint(o[e + 3])));
            if (cc == 0) {
                const int64_t nslots = (int64_t)a.num_items * Hq * a.nparts;
                a.ws[nslots * D + slot] = M;
                a.ws[nslots * D + nslots + slot] = den;
            }
        }
    }
}

// Log-sum-exp merge of the partitions of one (row, q head):
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
template <typename T, int D>
__global__ __launch_bounds__(64) void merge_kernel(const RowsArgs a, int group) {
    const int z = blockIdx.x, hq = blockIdx.y;
    const Item it = resolve(a, z, group);
    if (it.skip) return;
    const int pb = a.part_tokens / kBlock;
    const int nblk = (it.len + kBlock - 1) / kBlock;
    const int np = (nblk + pb - 1) / pb;
    const int Hq = a.num_q_heads;
    const int64_t slot0 = ((int64_t)z * Hq + hq) * a.nparts;
    const int64_t nslots = (int64_t)a.num_items * Hq * a.nparts;
    const float* ms = a.ws + nslots * D + slot0;
    const float* ls = ms + nslots;
    const float* acc = a.ws + slot0 * D;

    float M = kNegInf;
    for (int p = 0; p < np; ++p) M = fmaxf(M, ms[p]);
    const float mref = (M == kNegInf) ? 0.0f : M;
    float den = 0.0f;
    for (int p = 0; p < np; ++p) den = fmaf(ls[p], fast_exp2(ms[p] - mref), den);
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;

    const int d = threadIdx.x * 2;
    if (d >= D) return;
    float o0 = 0.0f, o1 = 0.0f;
    for (int p = 0; p < np; ++p) {
        const float wt = fast_exp2(ms[p] - mref);
        const float2 v = *reinterpret_cast<const float2*>(acc + (int64_t)p * D + d);
        o0 = fmaf(v.x, wt, o0);
        o1 = fmaf(v.y, wt, o1);
    }
    o0 *= inv;
    o1 *= inv;
    T* dst = static_cast<T*>(a.out) + ((int64_t)it.row * Hq + hq) * D + d;
    if constexpr (std::is_same_v<T, uint16_t>) {
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(o0, o1);
    } else {
        *reinterpret_cast<float2*>(dst) = make_float2(o0, o1);
    }
}

template <typename T, int D, int G>
int32_t launch_typed(const RowsArgs& a, hipStream_t stream) {
    const bool split = a.part_tokens > 0;
    dim3 grid(a.num_items, a.num_kv_heads, split ? a.nparts : 1);
    hipLaunchKernelGGL((rows_kernel<T, D, G>), grid, dim3(kWaves * 64), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
    if (split) {
        hipLaunchKernelGGL((merge_kernel<T, D>), dim3(a.num_items, a.num_q_heads), dim3(64), 0,
                           stream, a, G);
        if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
    }
    return PA_OK;
}

template <typename T, int D>
int32_t launch_group(const RowsArgs& a, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_typed<T, D, 1>(a, stream);
        case 2: return launch_typed<T, D, 2>(a, stream);
        case 3: return launch_typed<T, D, 3>(a, stream);
        case 4: return launch_typed<T, D, 4>(a, stream);
        case 5: return launch_typed<T, D, 5>(a, stream);
        case 6: return launch_typed<T, D, 6>(a, stream);
        case 7: return launch_typed<T, D, 7>(a, stream);
        case 8: return launch_typed<T, D, 8>(a, stream);
        default: return PA_ERR_UNSUPPORTED;
    }
}

}  // namespace

int32_t launch_rows(const RowsArgs& a, hipStream_t stream) {
    if (a.num_items == 0) return PA_OK;
    const int group = a.num_q_heads / a.num_kv_heads;
    if (a.dtype == PA_BF16) {
        if (a.head_dim == 64) return launch_group<uint16_t, 64>(a, group, stream);
        if (a.head_dim == 128) return launch_group<uint16_t, 128>(a, group, stream);
    } else if (a.dtype == PA_F32) {
        if (a.head_dim == 64) return launch_group<float, 64>(a, group, stream);
        if (a.head_dim == 128) return launch_group<float, 128>(a, group, stream);
    }
    return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
