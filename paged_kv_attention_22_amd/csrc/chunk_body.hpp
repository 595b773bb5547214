// Device code of the matrix-core chunk attention: the workgroup body
// (chunk_block, which takes its block index and LDS from the caller) and its
// helpers.
//
// A chunk of n new query tokens of a sequence with context length L holds
// rows (token t, head hh) of the kv head's GQA group, n*G rows in all; row
// (t, hh) sees keys 0 .. L-n+t.  One workgroup owns 64 or 128 rows of one
// (sequence, kv head), one or two 16-row tiles per wave (two tiles let one K
// or V fragment read from LDS feed two MFMAs).  Keys arrive in
// tiles of 64 (four 16-token blocks, gathered through the block table into
// LDS, K and V both row-major); a tile is shared by the four row waves.  With
// key halves, a second set of four waves takes every other tile for the same
// rows and the two softmax states are merged at the end.
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
// Two LDS buffers per key half: the next tile is written while the current
// one is read, one barrier per tile; the tile after that is already loading
// from memory.
//
// The same kernel attends a prefix shared by a group of decode sequences: the
// group's members are the "chunk" rows (one token each), every row sees all
// of the prefix (no causal limit), the keys come through the group's first
// member's table, the keys are split into parts over workgroups, and each
// part leaves its softmax state (m, l, unnormalised acc) as a partial for the
// log-sum-exp merge instead of writing the output.
#pragma once

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace chunk_impl {


typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// Per 16-bit element type (uint16_t: bf16 bits, _Float16: fp16): the 8-wide
// operand vector, the 16x16x32 product, and two probabilities packed with
// the conversion instruction (nearest even).
template <typename T>
struct Mma;
template <>
struct Mma<uint16_t> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ floatx4 mfma(v8 a, v8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ floatx4 mfma(v8 a, v8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKeys = 64;     // keys per tile
constexpr int kRowWaves = 4;  // waves splitting a workgroup's rows
// Shape of the launch: 16-row tiles per wave (register blocking), tiles of
// keys in flight from memory (register buffers) while one is computed, and
// key halves (a second set of waves takes every other tile of the same rows;
// the two softmax states are merged at the end).
constexpr int kDepth = 1;
// Two launch shapes.  A launch with fewer workgroups than the chip has compute
// units is bound by its longest chain of tiles: there each workgroup owns 64
// rows (one 16-row tile per wave) and runs two key halves (twice the waves and
// LDS, half the chain).  A larger launch is bound by throughput and shares
// the chip with the decode rows of a mixed batch: there each workgroup owns 128
// rows (two row tiles per wave, so each K/V fragment read from LDS feeds two
// MFMAs) and one key range, which leaves a compute unit's LDS and wave slots
// for the other kernel.
constexpr int kSplitBelow = kChunkSplitBelow;
constexpr int kRowsSmall = 16 * 1 * kRowWaves;
static_assert(kRowsSmall == kChunkRowsSmall, "the planner's view of the small shape");
constexpr int kRowsLarge = 16 * 2 * kRowWaves;



__device__ __forceinline__ uint2 ld_tr(const unsigned char* p) {
    const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
    return __builtin_bit_cast(uint2, v);
}

// Cross-lane steps for the four lanes l, l^16, l^32, l^48 that hold one row's
// scores.  The gfx950 swaps exchange the upper 32 lanes of their first operand
// with the lower 32 of the second (and odd 16-lane rows of the first with even
// rows of the second); with both operands holding x, the two results hold x
// and its partner lanes, without a trip through LDS.  The results are copied
// out element by element: bit-casting an element of the returned vector in
// place reads element 0 for both.
__device__ __forceinline__ float2 swap_halves(float x) {  // (x, lanes l^32)
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    return make_float2(__uint_as_float(r0), __uint_as_float(r1));
}
__device__ __forceinline__ float2 swap_rows(float x) {  // (x, lanes l^16)
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    return make_float2(__uint_as_float(r0), __uint_as_float(r1));
}
__device__ __forceinline__ float max_across_row_lanes(float x) {
    const float2 a = swap_halves(x);
    const float2 b = swap_rows(fmaxf(a.x, a.y));
    return fmaxf(b.x, b.y);
}
__device__ __forceinline__ float sum_across_row_lanes(float x) {
    const float2 a = swap_halves(x);
    const float2 b = swap_rows(a.x + a.y);
    return b.x + b.y;
}

// Loads from a wave-uniform base plus a 32-bit lane offset.  The base goes
// through readfirstlane, so the compiler keeps it in scalar registers and uses
// the scalar-base form of the global load (no 64-bit vector address arithmetic
// per load); the pointer stays in the global address space.
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
__device__ __forceinline__ uint4 ld16_at(const unsigned char* base, uint32_t off) {
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    typedef __attribute__((address_space(1))) const unsigned char global_u8;
    const global_u8* b = reinterpret_cast<const global_u8*>(((uint64_t)hi << 32) | lo);
    const u32x4 x = *reinterpret_cast<const global_u32x4*>(b + off);
    return make_uint4(x.x, x.y, x.z, x.w);
}

// LDS of one workgroup with key halves: two K and two V tiles per half
// (rows padded, filled from registers).
template <int D, int KSPLIT>
constexpr int lds_bytes() {
    return KSPLIT * 2 * kKeys * ((D * 2 + 32) + (D * 2 + 32));
}

// Without key halves the tiles come straight from memory into LDS
// (global_load_lds_dwordx4: each wave instruction fills 1 KiB of LDS, lane i
// the 16 bytes at i*16, so rows cannot be padded): kStages K and kStages V
// tiles of unpadded rows, each its own LDS array so that the compiler, which
// tracks these loads per LDS object, does not make reads of one stage wait
// for loads into another.  A row's 16-byte chunks are stored in swizzled
// order (chunk j of tile row r at slot j ^ swz(r)) to keep the fragment reads
// free of bank conflicts.
constexpr int kStages = 3;
template <int D>
constexpr int stage_bytes() {
    return kKeys * D * 2;
}
// K fragment reads take one chunk of 16 consecutive rows: the rows must fall
// on 16 different 16-byte bank groups (the 64 banks of 4 bytes).
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    constexpr int cpr = D / 8;  // chunks per row
    return (r / (16 / cpr)) & (cpr - 1);
}
// The transposing V reads take 32 bytes (2 chunks) of 4 consecutive rows per
// 16 lanes: the chunk pairs of those rows must not share bank groups.
template <int D>
__device__ __forceinline__ int swz_v(int r) {
    constexpr int cpr = D / 8;
    return 2 * ((r / (16 / cpr)) & (cpr / 2 - 1));
}
// Wait until at most N vector-memory operations of this wave are outstanding
// (the counter drains in issue order for loads).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;
// One 16-byte-per-lane load from (wave-uniform base + lane offset) into LDS
// at `dst` (wave-uniform) + lane*16.
__device__ __forceinline__ void ld16_to_lds(const unsigned char* base, uint32_t off, unsigned char* dst) {
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const unsigned char* b = reinterpret_cast<const unsigned char*>(((uint64_t)hi << 32) | lo);
    __builtin_amdgcn_global_load_lds((global_void*)(b + off), (lds_void*)dst, 16, 0, 0);
}

// One workgroup's work: row tile / key part bx, kv head by, sequence bz.
// With key halves (KSPLIT = 2) `lds` holds lds_bytes<D, KSPLIT>() bytes;
// without, kst and vst are the kStages K and V stage arrays of
// stage_bytes<D>() bytes each (all 16-byte aligned).  Called by every thread
// of the workgroup.
template <typename T, int D, int NT, int DEPTH, int KSPLIT>
__device__ __forceinline__ void chunk_block(const ChunkArgs& a, int bx, int by, int bz, unsigned char* lds,
                                            unsigned char* const (&kst)[kStages],
                                            unsigned char* const (&vst)[kStages]) {
    constexpr bool kDma = KSPLIT == 1;
    using V8 = typename Mma<T>::v8;
    using V2 = typename Mma<T>::v2;
    auto as_v8 = [](uint4 v) { return __builtin_bit_cast(V8, v); };
    constexpr int kNT = NT;
    constexpr int kRowsPerWave = 16 * NT;
    constexpr int kRowsPerGroup = kRowsPerWave * kRowWaves;
    constexpr int KS = D / 32;           // 32-wide slices of head_dim (first product)
    constexpr int MT = D / 16;           // 16-dim tiles of the output (second product)
    constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
    constexpr int HT = kRowWaves * 64;   // threads of one key half
    constexpr int LOADS = kKeys * CPR / HT;  // chunks per thread per tile
    // LDS row strides: K rows are read 16 lanes x 16 bytes down a column and V
    // rows by the transposing loads as 4 rows x 32 bytes per 16 lanes; a
    // 32-byte pad spreads both over the banks (a 16-byte pad measured half the
    // read rate of the 32-byte one for the K pattern).
    constexpr int KROW = D * 2 + 32;
    constexpr int VROW = D * 2 + 32;
    constexpr int KTILE = kKeys * KROW;
    constexpr int VTILE = kKeys * VROW;
    constexpr int KEYS_PER_WAVE_LOAD = 64 / CPR;  // keys one wave covers per load slot
    // a wave's keys of one load slot lie inside one pool block (8 tokens or more)
    static_assert(LOADS >= 1 && 8 % KEYS_PER_WAVE_LOAD == 0, "tile loader");
    // Two buffers per key half; the halves' states are merged through lds_k.
    static_assert(KSPLIT == 1 || (kRowWaves * 64 * NT * (MT * 4 + 2) * 4 <= KSPLIT * 2 * KTILE), "merge space");
    static_assert(KSPLIT * 2 * (KTILE + VTILE) == lds_bytes<D, KSPLIT>(), "LDS layout");
    unsigned char* const lds_k = lds;  // (null without key halves)
    unsigned char* const lds_v = kDma ? nullptr : lds + KSPLIT * 2 * KTILE;

    const int s = bz, g = by;
    const int nkp = max(a.key_parts, 1);
    const int kp = bx % nkp;  // key part (0 unless keys are split)
    const int G = a.num_q_heads / a.num_kv_heads;
    const int qs = a.query_start_loc[s];
    const int n = a.query_start_loc[s + 1] - qs;
    const int rows = n * G;
    if (rows < a.min_pairs) return;  // the vector path handles this sequence
    const int row0 = bx / nkp * kRowsPerGroup;
    if (row0 >= rows) return;
    const int bsh = a.block_shift;  // pool blocks of 1 << bsh tokens
    const int cap = (int)min((int64_t)a.max_context_len, (int64_t)a.max_blocks << bsh);
    const bool causal = a.causal != 0;
    // without a causal limit (a shared prefix) the keys are taken in whole
    // 16-token chunks: the decode kernels take the rest from that chunk on
    const int L = min(max(a.context_lens[s], 0), cap) & (causal ? ~0 : ~15);
    const int prior = causal ? L - n : L;  // keys before the chunk (all L without a causal limit)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform branches below
    const int half = wave / kRowWaves;  // which key half this wave works on
    const int rw = wave % kRowWaves;    // which rows
    const int htid = tid % HT;          // thread index within the half
    const int li = lane & 15, kg = lane >> 4;
    const int wrow0 = row0 + rw * kRowsPerWave;
    // This lane's rows: wrow0 + 16*nt + li, nt = 0..kNT-1.
    bool row_ok[kNT];
    int trow[kNT], hh[kNT], lim[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int R = wrow0 + nt * 16 + li;
        row_ok[nt] = R < rows;
        trow[nt] = R / G;
        hh[nt] = R - trow[nt] * G;
        lim[nt] = causal ? prior + trow[nt] : L - 1;  // last visible key of the row
    }

    // Keys this workgroup / this wave needs: 0 .. kend-1 in all, of which this
    // workgroup's key part takes kb .. ke-1 (whole tiles: parts are multiples
    // of the tile).
    const int last_row = min(row0 + kRowsPerGroup, rows) - 1;
    const int kend = causal ? min(prior + last_row / G + 1, L) : L;
    const int kb = nkp > 1 ? kp * a.key_part_tokens : 0;
    const int ke = nkp > 1 ? min(kb + a.key_part_tokens, kend) : kend;
    const int tbase = kb / kKeys;
    const int ntiles = ke > kb ? (ke - kb + kKeys - 1) / kKeys : 0;
    if (a.partials != nullptr && ntiles == 0) return;  // no keys in this part: the merge skips it
    const int wkend = wrow0 < rows
                          ? min(causal ? min(prior + (min(wrow0 + kRowsPerWave, rows) - 1) / G + 1, L) : L, ke)
                          : 0;
    // smallest last-visible key among the wave's rows
    const int wlim_min = causal ? prior + wrow0 / G : L - 1;

    // The block table is read-only for the whole kernel: reading it through
    // the constant address space makes the (wave-uniform) id loads scalar, so
    // they do not queue behind the K/V loads.
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    const int trow_of_table = a.table_row_qsl ? qs : s;  // a group's keys: its first member's table
    const const_i32* bt = (const const_i32*)(a.block_tables + (int64_t)trow_of_table * a.max_blocks);

    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const T* q = static_cast<const T*>(a.q);
    // q rows: every lane loads (rows past the chunk read its last row and are
    // zeroed after), so the loads are issued together and waited for once.
    uint4 qraw[kNT][KS];
    V8 qf[kNT][KS];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int R = min(wrow0 + nt * 16 + li, rows - 1);
        const int t = R / G, h = R - t * G;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qraw[nt][ks] = ld16(q + ((int64_t)(qs + t) * Hq + g * G + h) * D + ks * 32 + kg * 8);
    }

    const int64_t tok_stride = (int64_t)Hkv * D;

    // Loader: thread htid of a half moves chunks ci = htid + 256*u of a tile
    // (key ci/CPR, 16-byte piece ci%CPR) from the pool into registers.  For one
    // u the 64 lanes of a wave cover 64/CPR consecutive keys inside one block,
    // so the block id is wave-uniform: one scalar load per (wave, u).  Every
    // lane loads, and every step loads a tile (past the last tile it reloads
    // the last one; the clamped ids keep each address inside the pool): loads
    // that are never skipped are counted exactly by the memory counter, so the
    // wait before storing one register buffer leaves the later buffers in
    // flight.  Keys at or past kend (no row of this workgroup sees them) are
    // masked out of the scores; their V rows, whatever the slots hold (NaN
    // included), are stored as zeros so that a zero probability times them
    // stays zero.
    uint4 kreg[DEPTH][LOADS], vreg[DEPTH][LOADS];
    // A tile starts on a block boundary (tiles of kKeys keys, blocks of at
    // most 32), so each chunk's row inside its block, and with it the chunk's
    // byte offset inside the block, is the same for every tile: only the
    // (wave-uniform) block base changes, and the loads take it as a scalar
    // base plus this per-lane offset.
    static_assert(kKeys % 32 == 0, "tiles start on block boundaries");
    const int64_t blk_bytes = ((int64_t)tok_stride * 2) << bsh;
    uint32_t lane_off[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
        const int ci = htid + u * HT;
        const int key = ci / CPR, c = ci % CPR;
        lane_off[u] = (uint32_t)(((key & ((1 << bsh) - 1)) * tok_stride + g * D + c * 8) * 2);
    }
    const unsigned char* kbase = static_cast<const unsigned char*>(a.k_pool);
    const unsigned char* vbase = static_cast<const unsigned char*>(a.v_pool);
    auto load_tile = [&](int tile, uint4 (&kr)[LOADS], uint4 (&vr)[LOADS]) {
        const int j0 = (tbase + min(tile, ntiles - 1)) * kKeys;
        int blk[LOADS];
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {  // scalar loads first, one wait for all
            const int key0 = (rw * 64 + u * HT) / CPR;  // wave-uniform
            blk[u] = bt[min((j0 + key0) >> bsh, a.max_blocks - 1)];
        }
        // Left to itself the compiler clamps each id as soon as it is loaded,
        // a full scalar-memory round trip per load; keeping the clamps apart
        // puts all the loads in flight behind one wait.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < LOADS; ++u) blk[u] = min(max(blk[u], 0), a.num_blocks - 1);
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int64_t boff = (int64_t)blk[u] * blk_bytes;
            kr[u] = ld16_at(kbase + boff, lane_off[u]);
            vr[u] = ld16_at(vbase + boff, lane_off[u]);
        }
    };
    // This half's LDS buffers.
    unsigned char* const hk = kDma ? nullptr : lds_k + half * 2 * KTILE;
    unsigned char* const hv = kDma ? nullptr : lds_v + half * 2 * VTILE;
    auto store_tile = [&](int buf, int j0, const uint4 (&kr)[LOADS], const uint4 (&vr)[LOADS]) {
        const bool tail = j0 + kKeys > kend;  // wave-uniform: only the last tile
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int ci = htid + u * HT;
            const int key = ci / CPR, c = ci % CPR;
            uint4 v = vr[u];
            if (tail) {
                const uint32_t keep = 0u - (uint32_t)(j0 + key < kend);  // all ones or zero
                v = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
            }
            st16(hk + buf * KTILE + key * KROW + c * 16, kr[u]);
            st16(hv + buf * VTILE + key * VROW + c * 16, v);
        }
    };
    // Direct-to-LDS loader (no key halves).  For each u, thread htid loads
    // tile row r = (htid + u*HT) / CPR into its slot htid % CPR, taking the
    // row's chunk slot ^ swz(r) (K and V swizzled differently); the 64 lanes
    // of a wave fill 64/CPR whole rows (1 KiB of LDS), which lie in one pool
    // block.  A key at or past kend (no row of this workgroup sees it) loads
    // key kend-1 instead: finite data, whose scores are masked and whose V
    // rows meet zero probabilities.
    const int bmask = (1 << bsh) - 1;
    uint32_t k_off[LOADS], v_off[LOADS];  // lane offsets inside the block, for rows below kend
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
        const int r = (htid + u * HT) / CPR, slot = htid % CPR;
        const int base = (r & bmask) * tok_stride + g * D;
        k_off[u] = (uint32_t)((base + (slot ^ swz_k<D>(r)) * 8) * 2);
        v_off[u] = (uint32_t)((base + (slot ^ swz_v<D>(r)) * 8) * 2);
    }
    auto issue_tile = [&](int tile, unsigned char* kd, unsigned char* vd) {
        const int j0 = (tbase + min(tile, ntiles - 1)) * kKeys;
        int blk[LOADS];
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {  // scalar loads first, one wait for all
            const int key0 = (rw * 64 + u * HT) / CPR;  // the wave's first row (wave-uniform)
            blk[u] = bt[min(min(j0 + key0, kend - 1) >> bsh, a.max_blocks - 1)];
        }
        __builtin_amdgcn_sched_barrier(0);  // as in load_tile: one wait for all the id loads
#pragma unroll
        for (int u = 0; u < LOADS; ++u) blk[u] = min(max(blk[u], 0), a.num_blocks - 1);
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int64_t boff = (int64_t)blk[u] * blk_bytes;
            // the lane's key moves back only in the last tile (branch-free:
            // d is zero elsewhere, as tiles start on block boundaries)
            const int r = (htid + u * HT) / CPR;
            const int kc = min(j0 + r, kend - 1);
            const uint32_t d = (uint32_t)(((kc & bmask) - (r & bmask)) * tok_stride * 2);
            const uint32_t ko = k_off[u] + d, vo = v_off[u] + d;
            const int row = (rw * 64 + u * HT) / CPR;  // the wave's first row (wave-uniform)
            ld16_to_lds(kbase + boff, ko, kd + row * (D * 2));
            ld16_to_lds(vbase + boff, vo, vd + row * (D * 2));
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

    // LDS read offsets of this lane's fragments: K fragment (mt, ks) at
    // kt + mt*16 rows + kro[ks]; V^T fragment (kk, mt) at vt + kk*32 rows +
    // vro[mt] (and 16 rows further for its second half).
    constexpr int KRB = kDma ? D * 2 : KROW;  // row strides in LDS
    constexpr int VRB = kDma ? D * 2 : VROW;
    int kro[KS], vro[MT];
    {
        const int k4 = lane >> 2 & 3;  // key row within the lane's group of 4
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kro[ks] = li * KRB + (kDma ? ((ks * 4 + kg) ^ swz_k<D>(li)) * 16 : (ks * 32 + kg * 8) * 2);
        const int vr = 4 * kg + k4;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int b = (lane & 3) * 8 + mt * 32;  // byte of the row this lane reads
            vro[mt] = vr * VRB + (kDma ? ((b >> 4) ^ swz_v<D>(vr)) * 16 + (b & 15) : b);
        }
    }
    // The math of one tile (keys j0 .. j0+63), in four parts: the scores
    // (first product), the V^T fragments read from LDS, the online softmax,
    // and the second product.
    using Scores = floatx4[kNT][4];
    using VFrags = uint4[2][MT];  // (keys 32kk..+15, keys 32kk+16..+31) halves, as the A operand
    using Probs = uint32_t[kNT][8];
    // S^T from the K tile at kt.  Every K fragment is read first and the
    // products follow, so the LDS reads overlap one another instead of each
    // waiting in front of its product; each fragment feeds the kNT row tiles.
    auto s_part = [&](const unsigned char* kt, Scores& st) __attribute__((always_inline)) {
        uint4 kf[4][KS];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[mt][ks] = ld16(kt + mt * 16 * KRB + kro[ks]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) st[nt][mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) st[nt][mt] = Mma<T>::mfma(as_v8(kf[mt][ks]), qf[nt][ks], st[nt][mt]);
    };
    // The V^T fragments of the V tile at vt (they do not depend on the
    // probabilities, so they are read before the softmax that overlaps them).
    auto v_read = [&](const unsigned char* vt, VFrags& vf) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint2 lo = ld_tr(vt + 32 * kk * VRB + vro[mt]);
                const uint2 hi = ld_tr(vt + (32 * kk + 16) * VRB + vro[mt]);
                vf[kk][mt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
        }
    };
    // Online softmax of the scores: the running max and sum, the lazy
    // rescaling of the accumulators, and the probabilities packed for the
    // second product.
    auto sm_part = [&](int j0, const Scores& st, Probs& pk) __attribute__((always_inline)) {
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
                const int rel = lim[nt] - j0 - kg * 4;  // last visible key, tile-relative
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (mt * 16 + r > rel) sc[nt][mt * 4 + r] = kNegInf;
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
                // A row that has seen no key yet (possible in the second key
                // half, whose first tile can lie wholly past a row's last
                // visible key) has nothing to rescale: -inf - -inf is NaN.
                const float alpha = m[nt] == kNegInf ? 0.0f : fast_exp2(m[nt] - mn);
                lsum[nt] *= alpha;
#pragma unroll
                for (int i = 0; i < MT; ++i) acc[nt][i] *= alpha;
                m[nt] = mn;
            }
        }
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const float nmref = (m[nt] == kNegInf) ? 0.0f : -m[nt];
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p0 = fast_exp2(fmaf(sc[nt][2 * i], sl2, nmref));
                const float p1 = fast_exp2(fmaf(sc[nt][2 * i + 1], sl2, nmref));
                psum += p0 + p1;
                pk[nt][i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){p0, p1}, V2));
            }
            lsum[nt] += psum;
        }
    };
    // O^T += V^T P^T; each V^T fragment feeds the kNT row tiles.
    auto pv_part = [&](const Probs& pk, const VFrags& vf) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // keys 32*kk .. 32*kk+31: slots 0-3 from st[.][2kk], 4-7 from st[.][2kk+1]
            V8 pb[kNT];
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
                pb[nt] = as_v8(make_uint4(pk[nt][4 * kk], pk[nt][4 * kk + 1], pk[nt][4 * kk + 2], pk[nt][4 * kk + 3]));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const V8 va = as_v8(vf[kk][mt]);
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) acc[nt][mt] = Mma<T>::mfma(va, pb[nt], acc[nt][mt]);
            }
        }
    };
    // One whole tile on the K and V tiles at kt, vt.
    auto compute_tile = [&](int j0, const unsigned char* kt, const unsigned char* vt) __attribute__((always_inline)) {
        if (j0 < wkend) {
            Scores st;
            s_part(kt, st);
            VFrags vf;
            v_read(vt, vf);
            Probs pk;
            sm_part(j0, st, pk);
            pv_part(pk, vf);
        }
    };

    // Pipeline, per key half h (tiles h, h+KSPLIT, h+2*KSPLIT, ...): LDS holds
    // the tile being computed and the next one; DEPTH register buffers hold the
    // tiles after that, loading from memory.  The tile loaded at step i is
    // stored to LDS at step i+DEPTH.  Both halves run the same number of steps
    // (rounded up to a multiple of DEPTH so the unrolled body runs whole); a
    // step past the half's last tile computes nothing and stores an unused
    // buffer.  One barrier per step serves both halves.
    // An identity DPP move makes the q registers the result of a vector
    // instruction: the tile loop then never waits on memory for them (its
    // memory waits are for the tile prefetch only).
    auto finish_q = [&]() {
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
                qf[nt][ks] = as_v8(v);
            }
        }
    };

    if constexpr (kDma) {
        // Pipeline without key halves: kStages LDS stages; at step i tile i
        // is computed from stage i % kStages while tiles i+1 and i+2 are on
        // their way into the other two.  Each step waits for its own loads of
        // tile i (leaving tile i+1's in flight), then one barrier makes every
        // wave's share of tile i visible and tells that every wave is done
        // with tile i-1, whose stage then receives tile i+2.  The steps are
        // unrolled by kStages so every stage is a fixed LDS array; steps past
        // the last tile compute nothing and reload the last tile.
        if (ntiles > 0) {  // ntiles == 0 only for a sequence with no visible keys
            issue_tile(0, kst[0], vst[0]);
            issue_tile(1, kst[1], vst[1]);
            finish_q();
            const int nsteps = (ntiles + kStages - 1) / kStages * kStages;
            for (int i0 = 0; i0 < nsteps; i0 += kStages) {
#pragma unroll
                for (int r = 0; r < kStages; ++r) {
                    const int i = i0 + r;
                    wait_vmem<2 * LOADS>();
                    __builtin_amdgcn_s_barrier();
                    // keeps the compiler from moving LDS reads above the barrier
                    asm volatile("" ::: "memory");
                    issue_tile(i + 2, kst[(r + 2) % kStages], vst[(r + 2) % kStages]);
                    compute_tile((tbase + i) * kKeys, kst[r], vst[r]);
                }
            }
            wait_vmem<0>();  // the reloads past the last tile
        }
    } else if (ntiles > 0) {  // ntiles == 0 only for a sequence with no visible keys
        uint4 tile0k[LOADS], tile0v[LOADS];
        load_tile(half, tile0k, tile0v);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load_tile(half + KSPLIT * (d + 1), kreg[d], vreg[d]);
        finish_q();
        store_tile(0, (tbase + half) * kKeys, tile0k, tile0v);
        __syncthreads();
        const int hsteps = (ntiles + KSPLIT - 1) / KSPLIT;
        const int nsteps = (hsteps + DEPTH - 1) / DEPTH * DEPTH;
        // End of step i: tile i+1 into the other LDS buffer, the tile after
        // the register buffers' ones requested, and the barrier.
        auto advance = [&](int i, int r) __attribute__((always_inline)) {
            const int tile = half + KSPLIT * i;
            store_tile((i + 1) & 1, (tbase + tile + KSPLIT) * kKeys, kreg[r], vreg[r]);
            load_tile(tile + KSPLIT * (1 + DEPTH), kreg[r], vreg[r]);
            __syncthreads();
        };
        for (int i0 = 0; i0 < nsteps; i0 += DEPTH) {
#pragma unroll
            for (int r = 0; r < DEPTH; ++r) {  // unrolled: static register buffers
                const int i = i0 + r;
                compute_tile((tbase + half + KSPLIT * i) * kKeys, hk + (i & 1) * KTILE, hv + (i & 1) * VTILE);
                advance(i, r);
            }
        }
    }

    if constexpr (KSPLIT == 2) {
        // Merge the two halves' softmax states (same rows, disjoint keys):
        // the second half leaves (m, l, acc) in LDS, lane-fastest, and the
        // first rescales both to the larger reference max.  The tile loop
        // ended with a barrier, so the tile buffers are free.
        float* xs = reinterpret_cast<float*>(lds_k) + rw * 64 + lane;
        constexpr int kStride = kRowWaves * 64;
        if (half == 1) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                float* x = xs + nt * (MT * 4 + 2) * kStride;
                x[0] = m[nt];
                x[kStride] = lsum[nt];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[(2 + mt * 4 + r) * kStride] = acc[nt][mt][r];
            }
        }
        __syncthreads();
        if (half == 1) return;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const float* x = xs + nt * (MT * 4 + 2) * kStride;
            const float m1 = x[0];
            const float M = fmaxf(m[nt], m1);
            const float a0 = m[nt] == kNegInf ? 0.0f : fast_exp2(m[nt] - M);
            const float a1 = m1 == kNegInf ? 0.0f : fast_exp2(m1 - M);
            lsum[nt] = lsum[nt] * a0 + x[kStride] * a1;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[nt][mt][r] = acc[nt][mt][r] * a0 + x[(2 + mt * 4 + r) * kStride] * a1;
            m[nt] = M;  // the reference of the merged state (a partial carries it)
        }
    }

    if (a.partials != nullptr) {
        // Partial state of the key part: unnormalised acc, the reference max
        // m (log2 units) and the sum l, in the layout the merge reads.
        const int64_t nslots = (int64_t)a.num_items * Hq * a.part_slots;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const float l = sum_across_row_lanes(lsum[nt]);
            const int item = qs + trow[nt];
            if (!row_ok[nt] || item < 0 || item >= a.num_items) continue;
            const int64_t slot = ((int64_t)item * Hq + g * G + hh[nt]) * a.part_slots + kp;
            float* pa = a.partials + slot * D + kg * 4;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                st16(pa + mt * 16, make_uint4(__float_as_uint(acc[nt][mt][0]), __float_as_uint(acc[nt][mt][1]),
                                              __float_as_uint(acc[nt][mt][2]), __float_as_uint(acc[nt][mt][3])));
            if (kg == 0) {
                a.partials[nslots * D + slot] = m[nt];
                a.partials[nslots * D + nslots + slot] = l;
            }
        }
        return;
    }
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const float l = sum_across_row_lanes(lsum[nt]);
        if (!row_ok[nt]) continue;
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        T* out = static_cast<T*>(a.out) + ((int64_t)(qs + trow[nt]) * Hq + g * G + hh[nt]) * D + kg * 4;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint2 o = make_uint2(pack16<T>(acc[nt][mt][0] * inv, acc[nt][mt][1] * inv),
                                       pack16<T>(acc[nt][mt][2] * inv, acc[nt][mt][3] * inv));
            *reinterpret_cast<uint2*>(out + mt * 16) = o;
        }
    }
}


}  // namespace chunk_impl
}  // namespace pa
