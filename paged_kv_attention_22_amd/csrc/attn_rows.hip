// Vector-path attention over a paged KV pool: decode rows, and prefill rows
// too short for the matrix cores.
//
// Work unit: one workgroup per (query row, kv head, context partition).  The
// G = Hq/Hkv query heads of the kv head share every K/V row the workgroup
// loads, so each K/V byte crosses HBM once per (row, kv head).  Context
// partitions (split-context, flash-decoding style) give a long or ragged batch
// enough workgroups; their partial softmax states are merged by merge_kernel.
//
// Lane layout inside a wave: a token's [head_dim] row of K (or V) is split
// over R consecutive lanes, each holding V 16-byte chunks (V = 1: one load
// instruction covers 64/R whole rows; two chunks per lane cut the DPP steps
// but measured slower through the higher register count), and a wave covers
// 64/R tokens at once.  A block of 16 tokens is
// NT = 16*R/64 tokens per lane.  Each lane group of R lanes keeps its own
// running max / sum / accumulator (fp32 online softmax); the groups, then the
// waves, are merged at the end.  q.k partial sums are reduced across the R
// lanes with DPP row operations.  The running max is only raised when a score
// exceeds it by more than 2^8 (lazy rescaling): the exponentials stay below
// 256, and the accumulator is rescaled rarely instead of every block.
#include "rows_body.hpp"

namespace pa {
namespace {

using namespace rows_impl;

template <typename T, int D, int G>
__global__ __launch_bounds__(kWaves * 64) void rows_kernel(const RowsArgs a) {
    __shared__ __align__(16) unsigned char lds[rows_lds_bytes<D, G>()];
    rows_block<T, D, G>(a, blockIdx.x, lds);
}

template <typename T, int D, int G, int W>
__global__ __launch_bounds__(W * 64) void mfma_rows_kernel(const RowsArgs a) {
    __shared__ __align__(16) unsigned char lds[mfma_rows_lds_bytes<D, G, W>()];
    mfma_rows_block<T, D, G, W>(a, blockIdx.x, lds);
}

// Log-sum-exp merge of the partitions of one (row, q head):
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
// Rows whose context fits one partition were written by rows_kernel.  The
// first eight partials are loaded before any reduction so that the loads
// overlap instead of forming a chain.  Partials are indexed by item, so the
// merge runs in index order (its arguments carry no processing order).
template <typename T, int D>
__global__ __launch_bounds__(64) void merge_kernel(const RowsArgs a, int group) {
    constexpr int kPre = 8;
    const int z = blockIdx.x, hq = blockIdx.y;
    const Item it = locate(a, z, group, nullptr);  // index order: no ranking
    if (it.skip) return;
    const int len = visible_len(a, it, a.context_lens[it.seq]);
    const int pb = a.part_tokens / kBlock;
    const int nblk = (len + kBlock - 1) / kBlock;
    // Partials: npre of the shared prefix (slots 0..npre-1, shared-prefix mode
    // only), then nsuf of the rest (slots prefix_slots..).
    int npre = 0, c0 = 0;
    if (a.group_start != nullptr) {
        const int pch = prefix_chunks(a, it.seq);
        npre = (pch * kBlock + a.prefix_part_tokens - 1) / a.prefix_part_tokens;
        c0 = min(pch, nblk);
    }
    const int nsuf = (nblk - c0 + pb - 1) / pb;
    const int np = npre + nsuf;
    if (a.group_start == nullptr && np <= 1) return;  // written by the attention kernel
    auto slot_of = [&](int p) { return p < npre ? p : a.prefix_slots + p - npre; };
    const int Hq = a.num_q_heads;
    const int lane = threadIdx.x;
    const int64_t slot0 = ((int64_t)z * Hq + hq) * a.nparts;
    const int64_t nslots = (int64_t)a.num_items * Hq * a.nparts;
    const float* ms = a.ws + nslots * D + slot0;
    const float* ls = ms + nslots;
    const float* acc = a.ws + slot0 * D;
    const int d = min(lane * 2, D - 2);

    float2 v[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u)
        v[u] = u < np ? *reinterpret_cast<const float2*>(acc + (int64_t)slot_of(u) * D + d) : make_float2(0.0f, 0.0f);
    float M = kNegInf;
    for (int p = lane; p < np; p += 64) M = fmaxf(M, ms[slot_of(p)]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float mref = (M == kNegInf) ? 0.0f : M;
    float den = 0.0f, wl = 0.0f;
    for (int p = lane; p < np; p += 64) den = fmaf(ls[slot_of(p)], fast_exp2(ms[slot_of(p)] - mref), den);
    if (lane < np) wl = fast_exp2(ms[slot_of(lane)] - mref);  // weight of partial `lane`
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;

    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const float wt = __shfl(wl, u);
        o0 = fmaf(v[u].x, wt, o0);
        o1 = fmaf(v[u].y, wt, o1);
    }
    for (int p = kPre; p < np; ++p) {
        const float wt = fast_exp2(ms[slot_of(p)] - mref);
        const float2 w = *reinterpret_cast<const float2*>(acc + (int64_t)slot_of(p) * D + d);
        o0 = fmaf(w.x, wt, o0);
        o1 = fmaf(w.y, wt, o1);
    }
    if (lane * 2 >= D) return;
    o0 *= inv;
    o1 *= inv;
    T* dst = static_cast<T*>(a.out) + ((int64_t)it.row * Hq + hq) * D + d;
    if constexpr (kIs16<T>) {
        *reinterpret_cast<uint32_t*>(dst) = pack16<T>(o0, o1);
    } else {
        *reinterpret_cast<float2*>(dst) = make_float2(o0, o1);
    }
}

// Counting sort of the sequences by context length, longest first, in one
// workgroup: histogram of (length >> shift) in LDS, exclusive scan in
// descending key order, then each sequence takes the next slot of its key.
// Each length is read from memory once (kept in registers for up to
// kPlanKeep items per thread).  Equal keys come out in no particular order
// (every order is correct; only the scheduling changes).
constexpr int kPlanThreads = 256;
constexpr int kPlanBuckets = 1024;
constexpr int kPlanKeep = 8;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* context_lens, int seq_begin,
                                                            int n, int cap, int shift, int32_t* order) {
    __shared__ int start[kPlanBuckets];
    __shared__ int wave_sum[kPlanThreads / 64];
    const int t = threadIdx.x;
    auto key_of = [&](int i) {
        const int L = min(max(context_lens[seq_begin + i], 0), cap);
        return min(L >> shift, kPlanBuckets - 1);
    };
    int key[kPlanKeep];
#pragma unroll
    for (int j = 0; j < kPlanKeep; ++j) {
        const int i = t + j * kPlanThreads;
        key[j] = i < n ? key_of(i) : -1;
    }
    for (int b = t; b < kPlanBuckets; b += kPlanThreads) start[b] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPlanKeep; ++j)
        if (key[j] >= 0) atomicAdd(&start[key[j]], 1);
    for (int i = t + kPlanKeep * kPlanThreads; i < n; i += kPlanThreads) atomicAdd(&start[key_of(i)], 1);
    __syncthreads();
    // Thread t owns descending positions r = kPer*t .. kPer*t+kPer-1, i.e.
    // keys kPlanBuckets-1-r.
    constexpr int kPer = kPlanBuckets / kPlanThreads;
    int cnt[kPer], sum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        cnt[j] = start[kPlanBuckets - 1 - (t * kPer + j)];
        sum += cnt[j];
    }
    int incl = sum;  // inclusive scan over threads: within the wave, then across waves
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if ((t & 63) >= o) incl += y;
    }
    if ((t & 63) == 63) wave_sum[t >> 6] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < (t >> 6); ++w) before += wave_sum[w];
    int excl = before + incl - sum;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        start[kPlanBuckets - 1 - (t * kPer + j)] = excl;
        excl += cnt[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPlanKeep; ++j)
        if (key[j] >= 0) order[atomicAdd(&start[key[j]], 1)] = t + j * kPlanThreads;
    for (int i = t + kPlanKeep * kPlanThreads; i < n; i += kPlanThreads)
        order[atomicAdd(&start[key_of(i)], 1)] = i;
}

template <typename T, int D>
int32_t launch_merge_typed(const RowsArgs& a, int group, hipStream_t stream) {
    RowsArgs m = a;  // index order
    m.order = nullptr;
    m.rank_shift = -1;
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3(a.num_items, a.num_q_heads), dim3(64), 0, stream, m, group);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <typename T, int D, int G>
int32_t launch_typed(const RowsArgs& a, hipStream_t stream) {
    const bool split = a.part_tokens > 0;
    const int64_t units = (int64_t)a.num_items * a.num_kv_heads * (split ? a.nparts - a.prefix_slots : 1);
    if (units > INT32_MAX) return PA_ERR_SHAPE;
    if constexpr (kIs16<T> && G >= kMfmaMinGroup) {
        // Eight waves per workgroup (two per SIMD) keep twice the loads in
        // flight of four; a decode beside the shared-prefix tiles keeps four,
        // which leave room on each compute unit for a prefix workgroup.
        if (a.group_start != nullptr && !a.fold_prefix)
            hipLaunchKernelGGL((mfma_rows_kernel<T, D, G, kWaves>), dim3((unsigned)units), dim3(kWaves * 64), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((mfma_rows_kernel<T, D, G, kMaxWaves>), dim3((unsigned)units), dim3(kMaxWaves * 64),
                               0, stream, a);
    } else
        hipLaunchKernelGGL((rows_kernel<T, D, G>), dim3((unsigned)units), dim3(kWaves * 64), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
    if (split && !a.defer_merge) return launch_merge_typed<T, D>(a, G, stream);
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

int32_t launch_plan(const int32_t* context_lens, int32_t seq_begin, int32_t n,
                    int32_t max_context_len, int32_t* order, hipStream_t stream) {
    if (n <= 0) return PA_OK;
    int shift = 0;
    while ((max_context_len >> shift) >= kPlanBuckets) ++shift;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, context_lens, seq_begin, n,
                       max_context_len, shift, order);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int32_t launch_merge(const RowsArgs& a, hipStream_t stream) {
    if (a.num_items == 0 || a.part_tokens <= 0) return PA_OK;
    const int group = a.num_q_heads / a.num_kv_heads;
    if (a.dtype == PA_BF16) {
        if (a.head_dim == 64) return launch_merge_typed<uint16_t, 64>(a, group, stream);
        if (a.head_dim == 128) return launch_merge_typed<uint16_t, 128>(a, group, stream);
    } else if (a.dtype == PA_F16) {
        if (a.head_dim == 64) return launch_merge_typed<_Float16, 64>(a, group, stream);
        if (a.head_dim == 128) return launch_merge_typed<_Float16, 128>(a, group, stream);
    } else if (a.dtype == PA_F32) {
        if (a.head_dim == 64) return launch_merge_typed<float, 64>(a, group, stream);
        if (a.head_dim == 128) return launch_merge_typed<float, 128>(a, group, stream);
    }
    return PA_ERR_UNSUPPORTED;
}

int32_t launch_rows(const RowsArgs& a, hipStream_t stream) {
    if (a.num_items == 0) return PA_OK;
    const int group = a.num_q_heads / a.num_kv_heads;
    if (a.dtype == PA_BF16) {
        if (a.head_dim == 64) return launch_group<uint16_t, 64>(a, group, stream);
        if (a.head_dim == 128) return launch_group<uint16_t, 128>(a, group, stream);
    } else if (a.dtype == PA_F16) {
        if (a.head_dim == 64) return launch_group<_Float16, 64>(a, group, stream);
        if (a.head_dim == 128) return launch_group<_Float16, 128>(a, group, stream);
    } else if (a.dtype == PA_F32) {
        if (a.head_dim == 64) return launch_group<float, 64>(a, group, stream);
        if (a.head_dim == 128) return launch_group<float, 128>(a, group, stream);
    }
    return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
