// Fused QKV split + rotary embedding + KV-cache write, with each token's slot
// derived on the device from its sequence's block table and its position.
//
// The model's packed projection gives one row per token, [q heads | k heads |
// v heads] ("mini_engine", What it does: QKV packed into one GEMM); this
// kernel is the "fused RoPE" and "fused QKV split and KV-cache write" of
// "mini_engine", Next: fused kernels, with the GPU-side slot derivation of
// "mini-vllm", Milestones item 7.  One workgroup per token:
//   - sequence of the token: the last s with query_start_loc[s] <= t, found by
//     a wave-wide search that narrows the range 64-fold per round (no
//     query_start_loc: token t is sequence t);
//   - position L - n + i (the attention call's causal alignment), slot =
//     table[s][pos / 16] * 16 + pos % 16, or none when the position is past
//     the table or the entry is outside the pool (nothing is written then);
//   - q and k heads: optional per-head RMSNorm, then the rotate-half rotation:
//     lane j of a head holds dims j and j + D/2 and turns them by
//     pos * theta^(-2j/D) (fp32, precise sine and cosine); q goes to q_out, k to
//     the pool row;
//   - v heads: copied unchanged, 16 bytes per lane.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float load_elem(const T* p) {
    if constexpr (std::is_same_v<T, uint16_t>) return bf_lo(*p);
    else return *p;
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, float x) {
    if constexpr (std::is_same_v<T, uint16_t>) *p = (uint16_t)bf16_rne(x);
    else *p = x;
}

// Last s in [0, num_seqs) with qsl[s] <= t (qsl is non-decreasing, qsl[0] = 0).
// Each round the 64 lanes sample the range at a stride and the highest lane
// whose sample is <= t narrows it; wave-uniform result.
__device__ __forceinline__ int find_seq(const int32_t* qsl, int num_seqs, int t) {
    const int lane = threadIdx.x & 63;
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int span = hi - lo + 1;
        const int step = (span + 63) / 64;
        const int idx = lo + lane * step;
        const bool ok = idx <= hi && qsl[idx] <= t;
        const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
        const int last = m ? 63 - __builtin_clzll(m) : 0;
        lo = lo + last * step;
        hi = min(hi, lo + step - 1);
        if (step == 1) break;
    }
    return __builtin_amdgcn_readfirstlane(lo);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void qkv_write_kernel(const QkvArgs a) {
    constexpr int HALF = D / 2;
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    const int t = blockIdx.x;
    int s, n, i;
    if (a.query_start_loc == nullptr) {
        s = t;
        n = 1;
        i = 0;
    } else {
        s = find_seq(a.query_start_loc, a.num_seqs, t);
        const int q0 = a.query_start_loc[s];
        n = a.query_start_loc[s + 1] - q0;
        i = t - q0;
    }
    const int L = a.context_lens[s];
    const int pos = L - n + i;
    int64_t slot = -1;
    if (pos >= 0 && pos < a.max_blocks * kBlock) {
        const int blk = a.block_tables[(int64_t)s * a.max_blocks + pos / kBlock];
        if (blk >= 0 && blk < a.num_blocks) slot = (int64_t)blk * kBlock + pos % kBlock;
    }
    if (threadIdx.x == 0 && a.slots_out != nullptr) a.slots_out[t] = (int32_t)slot;

    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const T* row = static_cast<const T*>(a.qkv) + (int64_t)t * a.qkv_stride;
    T* qo = static_cast<T*>(a.q_out) + (int64_t)t * Hq * D;
    const int64_t srow = slot >= 0 ? slot : 0;  // rows are only written when slot >= 0
    T* kp = static_cast<T*>(a.k_pool) + srow * Hkv * D;
    T* vp = static_cast<T*>(a.v_pool) + srow * Hkv * D;
    const T* qn = static_cast<const T*>(a.q_norm);
    const T* kn = static_cast<const T*>(a.k_norm);

    // Rotated heads: item = head * HALF + j; a wave covers 64 / HALF whole heads,
    // so the per-head norm is a reduction over HALF consecutive lanes.
    const int items = (Hq + Hkv) * HALF;
    for (int it = threadIdx.x; it - (int)(threadIdx.x & 63) < items; it += kThreads) {
        const bool active = it < items;
        const int head = active ? it / HALF : 0;
        const int j = it % HALF;
        const bool is_q = head < Hq;
        float x1 = active ? load_elem(row + head * D + j) : 0.0f;
        float x2 = active ? load_elem(row + head * D + j + HALF) : 0.0f;
        const T* w = is_q ? qn : kn;
        if (w != nullptr) {  // uniform across the head's lanes
            const float ss = group_sum<HALF>(x1 * x1 + x2 * x2);
            const float r = 1.0f / sqrtf(ss / D + a.eps);
            x1 = x1 * r * load_elem(w + j);
            x2 = x2 * r * load_elem(w + j + HALF);
        }
        const float inv_freq = exp2f(-(2.0f * j / D) * a.log2_theta);
        float sn, cs;
        sincosf((float)pos * inv_freq, &sn, &cs);
        const float o1 = x1 * cs - x2 * sn;
        const float o2 = x2 * cs + x1 * sn;
        if (!active) continue;
        if (is_q) {
            store_elem(qo + head * D + j, o1);
            store_elem(qo + head * D + j + HALF, o2);
        } else if (slot >= 0) {
            const int kh = head - Hq;
            store_elem(kp + kh * D + j, o1);
            store_elem(kp + kh * D + j + HALF, o2);
        }
    }

    // V heads: bits copied unchanged.
    if (slot >= 0) {
        const T* vin = row + (Hq + Hkv) * D;
        for (int c = threadIdx.x; c < Hkv * D / EPC; c += kThreads) st16(vp + c * EPC, ld16(vin + c * EPC));
    }
}

}  // namespace

int32_t launch_qkv_write(const QkvArgs& a, hipStream_t stream) {
    if (a.num_tokens == 0) return PA_OK;
    const dim3 grid((unsigned)a.num_tokens), block(kThreads);
    if (a.dtype == PA_BF16) {
        if (a.head_dim == 128) hipLaunchKernelGGL((qkv_write_kernel<uint16_t, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((qkv_write_kernel<uint16_t, 64>), grid, block, 0, stream, a);
    } else {
        if (a.head_dim == 128) hipLaunchKernelGGL((qkv_write_kernel<float, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((qkv_write_kernel<float, 64>), grid, block, 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
