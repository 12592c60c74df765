// ssd_forward.hpp -- the one-call forward split into its host-side pieces, so
// that the C ABI entry points that run it (with a caller's workspace, or with
// the library's own scratch memory) share one validation and one pipeline.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "ssd.h"
#include "ssd_launch.hpp"

namespace ssd {

// Every argument check of ssd_forward except the workspace (host only, before
// any HIP call); fills `d` on success.
ssd_status forward_validate(const ssd_shape* shape, const void* x, const float* dt, const float* A, const void* Bm,
                            const void* Cm, const float* D, ssd_dtype in, const float* initial_states, const void* y,
                            ssd_dtype y_dtype, const float* final_states, ssd_mma mma, Dims* d);

// Workspace bytes the forward uses for a validated shape on one precision path:
// dA_cumsum and dt_bhl (fp32 [B,H,nc,Q]) and one [B,nc,H,N,P] state area
// (bf16 with SSD_MMA_BF16, fp32 with SSD_MMA_F32), each 256-byte aligned.
size_t forward_workspace_bytes(const Dims& d, bool f32_mma);

// Enqueue the forward (cumsum -> state path -> chunk scan) on `stream` for a
// validated shape; `workspace` holds at least forward_workspace_bytes(d, mma)
// bytes, 16-byte aligned.
ssd_status forward_run(const Dims& d, const void* x, const float* dt, const float* A, const void* Bm, const void* Cm,
                       const float* D, ssd_dtype in, const float* initial_states, void* y, ssd_dtype y_dtype,
                       float* final_states, void* workspace, ssd_mma mma, hipStream_t stream);

}  // namespace ssd
