// Matrix-core causal attention for prefill chunks (bf16, gfx950 MFMA).
//
// A chunk of n new query tokens of a sequence with context length L holds
// rows (token t, head hh) of the kv head's GQA group, n*G rows in all; row
// (t, hh) sees keys 0 .. L-n+t.  One workgroup of 4 waves owns 128 rows of
// one (sequence, kv head); each wave owns two tiles of 16 rows, so every K and
// V fragment it reads from LDS feeds two MFMAs.  Keys arrive in tiles of 64 (four
// 16-token blocks, gathered through the block table into LDS, K and V both
// row-major); the tile is shared by all four waves.
//
// Per tile and wave (v_mfma_f32_16x16x32_bf16, D = A*B + C, lane l holds
// A[l%16][k-slice l/16], B[k-slice l/16][l%16], D[4*(l/16)+r][l%16]):
//   S^T = K * Q^T      A = K rows from LDS, B = the wave's Q rows (registers);
//                      lane l ends with row l%16's scores for keys
//                      16*mt + 4*(l/16) + r, mt = 0..3, r = 0..3.
//   online softmax     in that layout: max across the 4 lanes sharing a row,
//                      the row sum kept per lane and added up at the end;
//                      the reference max moves only by more than 2^8 (lazy
//                      rescaling).
//   O^T += V^T * P^T   per 32 keys: B = the probabilities exactly as the S^T
//                      step left them (contraction slot p < 4: key
//                      4*(l/16)+p, p >= 4: key 16+4*(l/16)+p-4), A = V^T read
//                      from the row-major V tile with ds_read_b64_tr_b16, whose
//                      16-lane transpose hands lane i element i%4 of lanes
//                      i/4 + 4k: lanes 4k..4k+3 of a group point at key row k
//                      (dims 4 apart), and every lane receives one dim of four
//                      consecutive keys.
// Two LDS buffers: the next tile is written while the current one is read,
// one barrier per tile; the tile after that is already loading from memory.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKeys = 64;   // keys per tile
constexpr int kWaves = 4;
// Shape of the launch: 16-row tiles per wave (register blocking) and tiles of
// keys in flight from memory (register buffers) while one is computed.
constexpr int kNT = 2;
constexpr int kDepth = 1;
constexpr int kRowsPerGroup = 16 * kNT * kWaves;

__device__ __forceinline__ floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint2 ld_tr(const unsigned char* p) {
    const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
    return __builtin_bit_cast(uint2, v);
}

// Max over the four lanes l, l^16, l^32, l^48 (the lanes holding one row's
// scores): the gfx950 swaps exchange the upper 32 lanes of one operand with the
// lower 32 of the other (and odd 16-lane rows with even ones), so with both
// operands equal to x the two results are x and its partner lanes; no LDS trip.
__device__ __forceinline__ float max_across_row_lanes(float x) {
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    const auto s32 = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    x = fmaxf(__builtin_bit_cast(float, s32[0]), __builtin_bit_cast(float, s32[1]));
    const uint32_t c = __builtin_bit_cast(uint32_t, x);
    const auto s16 = __builtin_amdgcn_permlane16_swap(c, c, false, false);
    return fmaxf(__builtin_bit_cast(float, s16[0]), __builtin_bit_cast(float, s16[1]));
}

template <int D, int NT, int DEPTH>
__global__ __launch_bounds__(kWaves * 64) void chunk_kernel(const ChunkArgs a) {
    constexpr int kNT = NT;
    constexpr int kRowsPerWave = 16 * NT;
    constexpr int kRowsPerGroup = kRowsPerWave * kWaves;
    constexpr int KS = D / 32;           // 32-wide slices of head_dim (first product)
    constexpr int MT = D / 16;           // 16-dim tiles of the output (second product)
    constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
    constexpr int LOADS = kKeys * CPR / (kWaves * 64);  // chunks per thread per tile
    // LDS row strides: K rows are read 16 lanes x 16 bytes down a column, a
    // 16-byte pad spreads those rows over the banks; V rows are read by the
    // transposing loads as 4 rows x 32 bytes per 16 lanes, which a 32-byte pad
    // keeps apart.
    constexpr int KROW = D * 2 + 16;
    constexpr int VROW = D * 2 + 32;
    constexpr int KTILE = kKeys * KROW;
    constexpr int VTILE = kKeys * VROW;
    constexpr int KEYS_PER_WAVE_LOAD = 64 / CPR;  // keys one wave covers per load slot
    static_assert(LOADS >= 1 && kBlock % KEYS_PER_WAVE_LOAD == 0, "tile loader");
    __shared__ __align__(16) unsigned char lds_k[2 * KTILE];
    __shared__ __align__(16) unsigned char lds_v[2 * VTILE];

    const int s = blockIdx.z, g = blockIdx.y;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int qs = a.query_start_loc[s];
    const int n = a.query_start_loc[s + 1] - qs;
    const int rows = n * G;
    if (rows < a.min_pairs) return;  // the vector path handles this sequence
    const int row0 = blockIdx.x * kRowsPerGroup;
    if (row0 >= rows) return;
    const int cap = min(a.max_context_len, a.max_blocks * kBlock);
    const int L = min(max(a.context_lens[s], 0), cap);
    const int prior = L - n;  // keys before the chunk

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform branches below
    const int li = lane & 15, kg = lane >> 4;
    const int wrow0 = row0 + wave * kRowsPerWave;
    // This lane's rows: wrow0 + 16*nt + li, nt = 0..kNT-1.
    bool row_ok[kNT];
    int trow[kNT], hh[kNT], lim[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int R = wrow0 + nt * 16 + li;
        row_ok[nt] = R < rows;
        trow[nt] = R / G;
        hh[nt] = R - trow[nt] * G;
        lim[nt] = prior + trow[nt];  // last visible key of the row
    }

    // Keys this workgroup / this wave needs.
    const int last_row = min(row0 + kRowsPerGroup, rows) - 1;
    const int kend = min(prior + last_row / G + 1, L);
    const int ntiles = kend > 0 ? (kend + kKeys - 1) / kKeys : 0;
    const int wkend = wrow0 < rows ? min(prior + (min(wrow0 + kRowsPerWave, rows) - 1) / G + 1, L) : 0;
    const int wlim_min = prior + wrow0 / G;  // smallest last-visible key among the wave's rows

    // The block table is read-only for the whole kernel: reading it through
    // the constant address space makes the (wave-uniform) id loads scalar, so
    // they do not queue behind the K/V loads.
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    const const_i32* bt = (const const_i32*)(a.block_tables + (int64_t)s * a.max_blocks);

    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    // q rows: every lane loads (rows past the chunk read its last row and are
    // zeroed after), so the loads are issued together and waited for once.
    uint4 qraw[kNT][KS];
    bf16x8 qf[kNT][KS];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int R = min(wrow0 + nt * 16 + li, rows - 1);
        const int t = R / G, h = R - t * G;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qraw[nt][ks] = ld16(q + ((int64_t)(qs + t) * Hq + g * G + h) * D + ks * 32 + kg * 8);
    }
    const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
    const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
    const int64_t tok_stride = (int64_t)Hkv * D;

    // Loader: thread tid moves chunks ci = tid + 256*u of a tile (key ci/CPR,
    // 16-byte piece ci%CPR) from the pool into registers.  For one u the 64
    // lanes of a wave cover 64/CPR consecutive keys inside one block, so the
    // block id is wave-uniform: one scalar load per (wave, u).  Every lane
    // loads, and every step loads a tile (past the last tile it reloads the
    // last one; the clamped ids keep each address inside the pool): loads that
    // are never skipped are counted exactly by the memory counter, so the wait
    // before storing one register buffer leaves the later buffers in flight.
    // Keys at or past kend (no row of this workgroup sees them) are masked out
    // of the scores; their V rows, whatever the slots hold (NaN included), are
    // stored as zeros so that a zero probability times them stays zero.
    uint4 kreg[DEPTH][LOADS], vreg[DEPTH][LOADS];
    auto load_tile = [&](int tile, uint4 (&kr)[LOADS], uint4 (&vr)[LOADS]) {
        const int j0 = min(tile, ntiles - 1) * kKeys;
        int blk[LOADS];
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {  // scalar loads first, one wait for all
            const int key0 = (wave * 64 + u * kWaves * 64) / CPR;  // wave-uniform
            const int bi = min((j0 + key0) / kBlock, a.max_blocks - 1);
            blk[u] = min(max(bt[bi], 0), a.num_blocks - 1);
        }
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int ci = tid + u * kWaves * 64;
            const int key = ci / CPR, c = ci % CPR;
            const int64_t off = ((int64_t)blk[u] * kBlock + ((j0 + key) % kBlock)) * tok_stride + (int64_t)g * D + c * 8;
            kr[u] = ld16(kpool + off);
            vr[u] = ld16(vpool + off);
        }
    };
    auto store_tile = [&](int buf, int j0, const uint4 (&kr)[LOADS], const uint4 (&vr)[LOADS]) {
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int ci = tid + u * kWaves * 64;
            const int key = ci / CPR, c = ci % CPR;
            const uint32_t keep = 0u - (uint32_t)(j0 + key < kend);  // all ones or zero
            const uint4 v = make_uint4(vr[u].x & keep, vr[u].y & keep, vr[u].z & keep, vr[u].w & keep);
            *reinterpret_cast<uint4*>(lds_k + buf * KTILE + key * KROW + c * 16) = kr[u];
            *reinterpret_cast<uint4*>(lds_v + buf * VTILE + key * VROW + c * 16) = v;
        }
    };

    const float sl2 = a.scale * kLog2e;
    float m[kNT], lsum[kNT];
    floatx4 acc[kNT][MT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        m[nt] = kNegInf;
        lsum[nt] = 0.0f;
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[nt][i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // One tile of math on LDS buffer `buf` (keys j0 .. j0+63).
    auto compute_tile = [&](int j0, int buf) {
        if (j0 < wkend) {
            const unsigned char* kt = lds_k + buf * KTILE;
            const unsigned char* vt = lds_v + buf * VTILE;
            // S^T for keys j0 .. j0+63.  Every K fragment is read first and
            // the products follow, so the LDS reads overlap one another
            // instead of each waiting in front of its product; each fragment
            // feeds the kNT row tiles.
            uint4 kf[4][KS];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[mt][ks] = *reinterpret_cast<const uint4*>(kt + (mt * 16 + li) * KROW + (ks * 32 + kg * 8) * 2);
            __builtin_amdgcn_sched_barrier(0);
            floatx4 st[kNT][4];
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) st[nt][mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt) st[nt][mt] = mfma(as_bf16x8(kf[mt][ks]), qf[nt][ks], st[nt][mt]);
            // The V^T fragments of the second product do not depend on the
            // probabilities: reading them now overlaps the reads with the
            // softmax.
            const int k4 = lane >> 2 & 3;  // key row within the lane's group of 4
            uint2 vlo[2][MT], vhi[2][MT];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const unsigned char* v0 = vt + (32 * kk + 4 * kg + k4) * VROW + (lane & 3) * 8;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    vlo[kk][mt] = ld_tr(v0 + mt * 32);
                    vhi[kk][mt] = ld_tr(v0 + 16 * VROW + mt * 32);
                }
            }
            // Only a tile that crosses some row's last visible key (a
            // wave-uniform test) needs the causal mask.
            const bool masked = j0 + kKeys - 1 > wlim_min;
            float sc[kNT][16], mx[kNT];
            bool need_any = false;
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sc[nt][mt * 4 + r] = st[nt][mt][r];
                if (masked) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (j0 + mt * 16 + kg * 4 + r > lim[nt]) sc[nt][mt * 4 + r] = kNegInf;
                }
                float x = kNegInf;
#pragma unroll
                for (int i = 0; i < 16; ++i) x = fmaxf(x, sc[nt][i]);
                x = max_across_row_lanes(x);
                mx[nt] = x * sl2;  // sl2 > 0: the max of the scaled scores
                need_any |= mx[nt] > m[nt] + 8.0f;
            }
            // Lazy rescaling: the reference max moves only when a score exceeds
            // it by more than 2^8, so the accumulators are rescaled rarely and
            // the exponentials stay below 256.  The test is made wave-uniform
            // so it stays a real branch.
            if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    const float mn = mx[nt] > m[nt] + 8.0f ? mx[nt] : m[nt];
                    const float alpha = fast_exp2(m[nt] - mn);
                    lsum[nt] *= alpha;
#pragma unroll
                    for (int i = 0; i < MT; ++i) acc[nt][i] *= alpha;
                    m[nt] = mn;
                }
            }
            uint32_t pk[kNT][8];
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const float nmref = (m[nt] == kNegInf) ? 0.0f : -m[nt];
                float psum = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p0 = fast_exp2(fmaf(sc[nt][2 * i], sl2, nmref));
                    const float p1 = fast_exp2(fmaf(sc[nt][2 * i + 1], sl2, nmref));
                    psum += p0 + p1;
                    pk[nt][i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){p0, p1}, bf16x2v));
                }
                lsum[nt] += psum;
            }
            // O^T += V^T P^T; each V^T fragment feeds both row tiles.
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                // keys 32*kk .. 32*kk+31: slots 0-3 from st[.][2kk], 4-7 from st[.][2kk+1]
                bf16x8 pb[kNT];
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt)
                    pb[nt] = as_bf16x8(make_uint4(pk[nt][4 * kk], pk[nt][4 * kk + 1], pk[nt][4 * kk + 2], pk[nt][4 * kk + 3]));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const bf16x8 va = as_bf16x8(make_uint4(vlo[kk][mt].x, vlo[kk][mt].y, vhi[kk][mt].x, vhi[kk][mt].y));
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt) acc[nt][mt] = mfma(va, pb[nt], acc[nt][mt]);
                }
            }
        }
    };

    // Pipeline: LDS holds the tile being computed and the next one; DEPTH
    // register buffers hold the tiles after that, loading from memory.  The
    // tile loaded at step it is stored to LDS at step it+DEPTH.  The step count
    // is rounded up to a multiple of DEPTH so the unrolled body runs whole:
    // steps past the last tile compute nothing and store unused buffers.
    if (ntiles > 0) {  // ntiles == 0 only for a sequence with no visible keys
        uint4 tile0k[LOADS], tile0v[LOADS];
        load_tile(0, tile0k, tile0v);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load_tile(d + 1, kreg[d], vreg[d]);
        // An identity DPP move makes the q registers the result of a vector
        // instruction: the tile loop then never waits on memory for them (its
        // memory waits are for the tile prefetch only).
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const uint32_t keep = 0u - (uint32_t)row_ok[nt];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint4 v = qraw[nt][ks];
                v.x = __builtin_amdgcn_update_dpp(0u, v.x & keep, 0xE4, 0xf, 0xf, false);
                v.y = __builtin_amdgcn_update_dpp(0u, v.y & keep, 0xE4, 0xf, 0xf, false);
                v.z = __builtin_amdgcn_update_dpp(0u, v.z & keep, 0xE4, 0xf, 0xf, false);
                v.w = __builtin_amdgcn_update_dpp(0u, v.w & keep, 0xE4, 0xf, 0xf, false);
                qf[nt][ks] = as_bf16x8(v);
            }
        }
        store_tile(0, 0, tile0k, tile0v);
        __syncthreads();
        const int nsteps = (ntiles + DEPTH - 1) / DEPTH * DEPTH;
        for (int it0 = 0; it0 < nsteps; it0 += DEPTH) {
#pragma unroll
            for (int r = 0; r < DEPTH; ++r) {  // unrolled: static register buffers
                const int it = it0 + r;
                const int j0 = it * kKeys;
                compute_tile(j0, it & 1);
                store_tile((it + 1) & 1, j0 + kKeys, kreg[r], vreg[r]);
                load_tile(it + 1 + DEPTH, kreg[r], vreg[r]);
                __syncthreads();
            }
        }
    }

#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        float l = lsum[nt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (!row_ok[nt]) continue;
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        uint16_t* out = static_cast<uint16_t*>(a.out) + ((int64_t)(qs + trow[nt]) * Hq + g * G + hh[nt]) * D + kg * 4;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint2 o = make_uint2(pack_bf16x2(acc[nt][mt][0] * inv, acc[nt][mt][1] * inv),
                                       pack_bf16x2(acc[nt][mt][2] * inv, acc[nt][mt][3] * inv));
            *reinterpret_cast<uint2*>(out + mt * 16) = o;
        }
    }
}

}  // namespace

bool chunks_supported(int32_t dtype, int32_t head_dim, int32_t group) {
    return dtype == PA_BF16 && (head_dim == 64 || head_dim == 128) && group >= 1 &&
           group <= kMaxGroup;
}

int32_t launch_chunks(const ChunkArgs& a, hipStream_t stream) {
    const int group = a.num_q_heads / a.num_kv_heads;
    if (!chunks_supported(a.dtype, a.head_dim, group)) return PA_ERR_UNSUPPORTED;
    if (a.num_seqs == 0 || a.max_query_len == 0) return PA_OK;
    const int64_t tiles = ((int64_t)a.max_query_len * group + kRowsPerGroup - 1) / kRowsPerGroup;
    if (tiles > INT32_MAX || a.num_seqs > 65535) return PA_ERR_SHAPE;
    dim3 grid((unsigned)tiles, a.num_kv_heads, a.num_seqs);
    if (a.head_dim == 128)
        hipLaunchKernelGGL((chunk_kernel<128, kNT, kDepth>), grid, dim3(kWaves * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((chunk_kernel<64, kNT, kDepth>), grid, dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
