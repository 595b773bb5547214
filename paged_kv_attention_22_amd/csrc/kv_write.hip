// Slot-mapped KV-cache write: token t's K and V rows go to row slot[t] of the
// pools viewed as [num_blocks * 16, num_kv_heads * head_dim] (slot = block *
// 16 + offset, so the flat slot is the pool row).  Pure data movement: each
// thread copies one 16-byte piece of a K row and the matching piece of the V
// row; a wave covers 1 KiB of consecutive row bytes, so reads and writes are
// whole 128-byte lines whatever the slots are.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void kv_write_kernel(const KvWriteArgs a) {
    const int cpr = a.row_bytes >> 4;  // 16-byte pieces per row
    const int64_t total = (int64_t)a.num_tokens * cpr;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / cpr;
        const int piece = (int)(i - t * cpr);
        const int64_t slot = a.slots[t];
        if (slot < 0 || slot >= a.pool_rows) continue;
        const char* ks = static_cast<const char*>(a.k) + t * a.k_stride + piece * 16;
        const char* vs = static_cast<const char*>(a.v) + t * a.v_stride + piece * 16;
        const uint4 kk = ld16(ks);
        const uint4 vv = ld16(vs);
        st16(static_cast<char*>(a.k_pool) + slot * a.row_bytes + piece * 16, kk);
        st16(static_cast<char*>(a.v_pool) + slot * a.row_bytes + piece * 16, vv);
    }
}

}  // namespace

int32_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
    if (a.num_tokens == 0) return PA_OK;
    const int64_t total = (int64_t)a.num_tokens * (a.row_bytes >> 4);
    const int64_t want = (total + 255) / 256;
    const int blocks = (int)(want < 16384 ? want : 16384);
    hipLaunchKernelGGL(kv_write_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
