// retention_chunkwise_fwd_noalloc: the chunkwise forward with its scratch memory in a file-scope
// device array instead of a caller workspace, for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc). Nothing here allocates:
// the array is part of the loaded code object, one copy per GPU, held until the process ends.
#include <cstdio>
#include <mutex>

#include "../../include/retention.h"
#include "common.hpp"
#include "entry.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)RETENTION_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The scratch of every no-allocation call on one GPU. In host code `scratch` is only a stand-in
// for the symbol, never a device address: its address on each device comes from
// hipGetSymbolAddress and is kept in g_scratch[device].
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// The workspace of a no-allocation call: after validation, and only when the call needs some.
// Sizes beyond the array are refused before any HIP call; otherwise the array's address on the
// current device, looked up once per device with that device current.
int provide_scratch(size_t need, void** ws, size_t* bytes) {
    char msg[256];
    if (need > kScratchBytes) {
        snprintf(msg, sizeof(msg),
                 "retention_chunkwise_fwd_noalloc: this call needs %zu bytes of scratch, above the library's fixed %zu-byte "
                 "array (use retention_chunkwise_fwd with a workspace)", need, kScratchBytes);
        ret::set_last_error(msg);
        return RET_ERR_WORKSPACE;
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (!g_scratch[dev]) {
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e == hipSuccess && !p) e = hipErrorInvalidSymbol;
            if (e == hipSuccess) g_scratch[dev] = p;
        }
        *ws = g_scratch[dev];
    }
    if (e != hipSuccess) {
        snprintf(msg, sizeof(msg), "retention_chunkwise_fwd_noalloc: address of the scratch array on device %d: %s", dev,
                 hipGetErrorString(e));
        ret::set_last_error(msg);
        return RET_ERR_DEVICE;
    }
    *bytes = kScratchBytes;
    return RET_OK;
}

}  // namespace

extern "C" ret_status retention_chunkwise_fwd_noalloc(const ret_shape* shape, int32_t chunk, const void* q, const void* k,
                                                      const void* v, const double* gamma, const ret_rotation* rotation,
                                                      const float* state_in, const ret_groupnorm* groupnorm, void* out,
                                                      float* state_out, void* hip_stream) {
    return (ret_status)ret::chunkwise_fwd_entry(shape, chunk, q, k, v, gamma, rotation, state_in, groupnorm, out, state_out, nullptr, 0,
                                                provide_scratch, hip_stream);
}
