// Host-only stand-ins for the kernel launchers of libpa.so, for a CPU build
// of the library's host code (pa_api.cpp, block_manager.cpp) under the
// address and undefined-behaviour sanitizers.  Every launcher accepts its
// arguments and launches nothing; the host code around them (argument
// validation, workspace layout, stream and event handling, the block
// manager) is the real one.  Test infrastructure: never part of libpa.so.
#include "../../paged_kv_attention_22_amd/csrc/pa_internal.hpp"

namespace pa {

int32_t launch_rows(const RowsArgs&, hipStream_t) { return PA_OK; }
int32_t launch_merge(const RowsArgs&, hipStream_t) { return PA_OK; }
int32_t launch_plan(const int32_t*, int32_t, int32_t, int32_t, int32_t*, hipStream_t) { return PA_OK; }
int32_t launch_kv_write(const KvWriteArgs&, hipStream_t) { return PA_OK; }
int32_t launch_qkv_write(const QkvArgs&, hipStream_t) { return PA_OK; }
int32_t launch_chunks(const ChunkArgs&, hipStream_t) { return PA_OK; }

}  // namespace pa

// pa_decode_noalloc lives in a HIP source (its scratch array is device
// memory); the binding resolves every entry point when it loads a library, so
// the stand-in exports it too, as a call that is never made here.
extern "C" int32_t pa_decode_noalloc(const void*, const void*, const void*, pa_pool_desc, const int32_t*, int32_t,
                                     const int32_t*, int32_t, int32_t, int32_t, float, void*, int32_t, void*) {
    return PA_ERR_UNSUPPORTED;
}
