// forward_noalloc.hip -- ssd_forward for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid allocation): the forward's workspace is the library's own static
// device array `scratch` instead of a caller buffer.
//
// `scratch` is a file-scope __device__ array, so every GPU the library runs
// on holds its own copy (SSD_NOALLOC_SCRATCH_BYTES bytes) from the moment the
// code object is loaded until the process ends.  Host code never uses the
// array's name as an address (on the host it only names the symbol): the
// device address of each GPU's copy is looked up once per device, with that
// device current, by hipGetSymbolAddress, and only that address is passed to
// the kernels.  Nothing here calls hipMalloc, hipFree or any allocating
// routine.  Every call on one GPU shares that GPU's copy, so calls that
// overlap on one GPU (two streams, or two host threads) race on it; calls in
// order on one stream are safe.  The forward writes every scratch byte it
// reads before reading it, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ssd.h"
#include "ssd_forward.hpp"

namespace {

constexpr size_t kScratchBytes = SSD_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_init_mu;
std::atomic<void*> g_scratch_addr[kMaxDevices];  // device address of `scratch` per device

// The current device's copy of `scratch`, looked up on the first call on that
// device.
ssd_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_init_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SSD_OK;
}

}  // namespace

extern "C" ssd_status ssd_forward_noalloc(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                                          const void* Bm, const void* Cm, const float* D, ssd_dtype in,
                                          const float* initial_states, void* y, ssd_dtype y_dtype,
                                          float* final_states, ssd_mma mma, void* stream) {
  ssd::Dims d;
  const ssd_status st =
      ssd::forward_validate(shape, x, dt, A, Bm, Cm, D, in, initial_states, y, y_dtype, final_states, mma, &d);
  if (st != SSD_OK) return st;
  if (ssd::forward_workspace_bytes(d, mma == SSD_MMA_F32) > kScratchBytes) return SSD_ERR_SCRATCH;
  void* ws = nullptr;
  const ssd_status sp = scratch_for_current_device(&ws);
  if (sp != SSD_OK) return sp;
  return ssd::forward_run(d, x, dt, A, Bm, Cm, D, in, initial_states, y, y_dtype, final_states, ws, mma,
                          (hipStream_t)stream);
}
