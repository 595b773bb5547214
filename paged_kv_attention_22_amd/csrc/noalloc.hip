// pa_decode_noalloc: pa_decode for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  The workspace pa_decode takes from its caller (the
// longest-first order of a large batch, the split-context partials) comes
// instead from a fixed array in device memory that the library holds, one per
// device, for the life of the process.
#include <mutex>

#include "pa_internal.hpp"

// The scratch array.  In host code its name is only a stand-in for the
// symbol: the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_addr[kMaxDevices];  // device address of `scratch` on each device (null: lookup failed)

// The device address of this device's copy of `scratch`, looked up the first
// time with that device current.
void* scratch_on(int dev) {
    std::call_once(scratch_once[dev], [dev] {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return;
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) scratch_addr[dev] = p;
        if (cur != dev) (void)hipSetDevice(cur);
    });
    return scratch_addr[dev];
}

}  // namespace

extern "C" {

int32_t pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool, pa_pool_desc pool,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads, float scale, void* out,
                          int32_t partition_tokens, void* stream) {
    if (int32_t st = pa::check_decode(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens,
                                      num_seqs, max_context_len, num_q_heads, out, partition_tokens))
        return st;
    // The workspace pa_decode would need for these arguments.
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, pool.num_kv_heads, pool.head_dim,
                                                  max_context_len, partition_tokens);
    if (need > kScratchBytes) return PA_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        hipStream_t s = static_cast<hipStream_t>(stream);
        int dev = 0;
        if (s != nullptr) {
            if (hipStreamGetDevice(s, &dev) != hipSuccess) return PA_ERR_LAUNCH;
        } else if (hipGetDevice(&dev) != hipSuccess) {
            return PA_ERR_LAUNCH;
        }
        if (dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
        ws = scratch_on(dev);
        if (ws == nullptr) return PA_ERR_LAUNCH;
    }
    return pa::decode_impl(q, nullptr, nullptr, 0, 0, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                           context_lens, num_seqs, max_context_len, num_q_heads, scale, out, partition_tokens,
                           ws, ws != nullptr ? kScratchBytes : 0, stream);
}

}  // extern "C"
