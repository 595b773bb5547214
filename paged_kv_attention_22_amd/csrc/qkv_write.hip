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
//     pos * theta^(-2j/D) (angle formed and reduced in fp64, sine and cosine
//     in fp32); q goes to q_out, k to the pool row;
//   - v heads: copied unchanged, 16 bytes per lane.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kThreads = 256;

// T: uint16_t (bf16 bits), _Float16 or float.
template <typename T>
__device__ __forceinline__ float load_elem(const T* p) {
    if constexpr (std::is_same_v<T, uint16_t>) return bf_lo(*p);
    else return (float)*p;
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, float x) {
    if constexpr (std::is_same_v<T, uint16_t>) *p = (uint16_t)bf16_rne(x);
    else *p = (T)x;
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
    constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte chunk
    constexpr int HPT = kThreads / HALF;  // rotated heads per pass
    constexpr int KB = 8;                 // passes whose loads are in flight together
    constexpr int VB = 2;                 // V chunks per thread loaded up front
    const int t = blockIdx.x;
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const int nh = Hq + Hkv;
    const T* row = static_cast<const T*>(a.qkv) + (int64_t)t * a.qkv_stride;

    // Everything the token's row provides is requested first: the first KB
    // passes of rotated pairs and the first V chunks.  Thread tid always holds
    // pair j = tid % HALF of heads tid / HALF + k * HPT (a wave covers whole
    // heads, so the per-head norm is a reduction over HALF consecutive lanes).
    const int j = threadIdx.x % HALF;
    const int h0 = threadIdx.x / HALF;
    // Every lane loads (heads past the last one re-read it, unused): loads
    // without a branch around them are all in flight at once.
    float x1[KB], x2[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int head = min(h0 + k * HPT, nh - 1);
        x1[k] = load_elem(row + head * D + j);
        x2[k] = load_elem(row + head * D + j + HALF);
    }
    const T* vin = row + nh * D;
    const int vchunks = Hkv * D / EPC;
    uint4 vv[VB];
#pragma unroll
    for (int k = 0; k < VB; ++k) vv[k] = ld16(vin + min((int)threadIdx.x + k * kThreads, vchunks - 1) * EPC);

    // Sequence, position and slot (scalar loads).
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
    const int pos = a.context_lens[s] - n + i;
    int64_t slot = -1;
    const int bsh = a.block_shift;  // pool blocks of 1 << bsh tokens
    if (pos >= 0 && (int64_t)pos < ((int64_t)a.max_blocks << bsh)) {
        const int blk = a.block_tables[(int64_t)s * a.max_blocks + (pos >> bsh)];
        if (blk >= 0 && blk < a.num_blocks) slot = ((int64_t)blk << bsh) + (pos & ((1 << bsh) - 1));
    }
    if (threadIdx.x == 0 && a.slots_out != nullptr) a.slots_out[t] = (int32_t)slot;

    T* qo = static_cast<T*>(a.q_out) + (int64_t)t * Hq * D;
    const int64_t srow = slot >= 0 ? slot : 0;  // rows are only written when slot >= 0
    T* kp = static_cast<T*>(a.k_pool) + srow * Hkv * D;
    T* vp = static_cast<T*>(a.v_pool) + srow * Hkv * D;
    const T* qn = static_cast<const T*>(a.q_norm);
    const T* kn = static_cast<const T*>(a.k_norm);

    // The rotation angle of pair j is the same for every head: one sine and
    // cosine per thread.  The angle pos * theta^(-2j/D) is formed in fp64 and
    // reduced to a fraction of a turn in [-1/2, 1/2] there, so the fp32 sine
    // and cosine (the hardware ones, which take turns) see a small argument
    // and no precision is lost to large positions.
    const double turns = (double)pos * exp2(-(2.0 * j / D) * a.log2_theta) * 0.15915494309189535;
    const float f = (float)(turns - rint(turns));
    const float sn = __builtin_amdgcn_sinf(f);
    const float cs = __builtin_amdgcn_cosf(f);
    const T* qw = qn != nullptr ? qn : row;  // a valid address either way; unused without a norm
    const T* kw = kn != nullptr ? kn : row;
    const float wq1 = load_elem(qw + j), wq2 = load_elem(qw + j + HALF);
    const float wk1 = load_elem(kw + j), wk2 = load_elem(kw + j + HALF);

    for (int hb = 0; hb < nh; hb += HPT * KB) {
        if (hb > 0) {  // later passes (many heads): load them the same way
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int head = min(hb + h0 + k * HPT, nh - 1);
                x1[k] = load_elem(row + head * D + j);
                x2[k] = load_elem(row + head * D + j + HALF);
            }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int head = hb + h0 + k * HPT;  // the same for the HALF lanes of a head
            if (head >= nh) continue;
            const bool is_q = head < Hq;
            float y1 = x1[k], y2 = x2[k];
            if (is_q ? qn != nullptr : kn != nullptr) {
                const float ss = group_sum<HALF>(y1 * y1 + y2 * y2);
                const float r = 1.0f / sqrtf(ss / D + a.eps);
                y1 *= r * (is_q ? wq1 : wk1);
                y2 *= r * (is_q ? wq2 : wk2);
            }
            const float o1 = y1 * cs - y2 * sn;
            const float o2 = y2 * cs + y1 * sn;
            if (is_q) {
                store_elem(qo + head * D + j, o1);
                store_elem(qo + head * D + j + HALF, o2);
            } else if (slot >= 0) {
                const int kh = head - Hq;
                store_elem(kp + kh * D + j, o1);
                store_elem(kp + kh * D + j + HALF, o2);
            }
        }
    }

    // V heads: bits copied unchanged.
    if (slot >= 0) {
#pragma unroll
        for (int k = 0; k < VB; ++k) {
            const int c = threadIdx.x + k * kThreads;
            if (c < vchunks) st16(vp + c * EPC, vv[k]);
        }
        for (int c = threadIdx.x + VB * kThreads; c < vchunks; c += kThreads)
            st16(vp + c * EPC, ld16(vin + c * EPC));
    }
}

}  // namespace

int32_t launch_qkv_write(const QkvArgs& a, hipStream_t stream) {
    if (a.num_tokens == 0) return PA_OK;
    const dim3 grid((unsigned)a.num_tokens), block(kThreads);
    if (a.dtype == PA_BF16) {
        if (a.head_dim == 128) hipLaunchKernelGGL((qkv_write_kernel<uint16_t, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((qkv_write_kernel<uint16_t, 64>), grid, block, 0, stream, a);
    } else if (a.dtype == PA_F16) {
        if (a.head_dim == 128) hipLaunchKernelGGL((qkv_write_kernel<_Float16, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((qkv_write_kernel<_Float16, 64>), grid, block, 0, stream, a);
    } else {
        if (a.head_dim == 128) hipLaunchKernelGGL((qkv_write_kernel<float, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((qkv_write_kernel<float, 64>), grid, block, 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
