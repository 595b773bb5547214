// Slot-mapped KV-cache write: token t's K and V rows go to row slot[t] of the
// pools viewed as [num_blocks * 16, num_kv_heads * head_dim] (slot = block *
// 16 + offset, so the flat slot is the pool row).  Pure data movement: each
// thread copies 16-byte pieces of a K row and the matching pieces of the V
// row; a wave covers 1 KiB of consecutive row bytes, so reads and writes are
// whole 128-byte lines whatever the slots are.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

// One workgroup per token: the slot is a scalar load, and the row loads do
// not depend on it, so both are in flight together; only the stores wait.
__global__ __launch_bounds__(256) void kv_write_kernel(const KvWriteArgs a) {
    const int64_t t = blockIdx.x;
    const int cpr = a.row_bytes >> 4;  // 16-byte pieces per row
    const int64_t slot = a.slots[t];
    const char* ks = static_cast<const char*>(a.k) + t * a.k_stride;
    const char* vs = static_cast<const char*>(a.v) + t * a.v_stride;
    char* kd = static_cast<char*>(a.k_pool) + slot * a.row_bytes;
    char* vd = static_cast<char*>(a.v_pool) + slot * a.row_bytes;
    for (int piece = threadIdx.x; piece < cpr; piece += blockDim.x) {
        const uint4 kk = ld16(ks + piece * 16);
        const uint4 vv = ld16(vs + piece * 16);
        if (slot < 0 || slot >= a.pool_rows) continue;
        st16(kd + piece * 16, kk);
        st16(vd + piece * 16, vv);
    }
}

}  // namespace

int32_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
    if (a.num_tokens == 0) return PA_OK;
    const int cpr = a.row_bytes >> 4;
    const int threads = cpr >= 256 ? 256 : ((cpr + 63) / 64) * 64;
    hipLaunchKernelGGL(kv_write_kernel, dim3(a.num_tokens), dim3(threads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
