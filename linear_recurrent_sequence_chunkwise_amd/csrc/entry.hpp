// Internal: the chunkwise forward shared by retention_chunkwise_fwd (caller workspace) and
// retention_chunkwise_fwd_noalloc (the library's fixed scratch array).
#pragma once
#include <stddef.h>

#include "../../include/retention.h"

namespace ret {
// Validates every argument on the host, then asks provide (when not null, and only when the call
// needs workspace) for need bytes of it; provide returns RET_OK with the buffer, or a status whose
// message it has set. Then launches as retention_chunkwise_fwd does. Returns a ret_status.
int chunkwise_fwd_entry(const ret_shape* shape, int32_t chunk, const void* q, const void* k, const void* v, const double* gamma,
                        const ret_rotation* rotation, const float* state_in, const ret_groupnorm* groupnorm, void* out,
                        float* state_out, void* workspace, size_t workspace_bytes,
                        int (*provide)(size_t need, void** ws, size_t* bytes), void* hip_stream);
}  // namespace ret
