// loglin_fwd_noalloc: the forward pass for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, hosts that
// forbid allocation during a step).  The forward's workspace (segment
// states, level slots and their log-decays) lives in a fixed array of
// device memory that the library's code object carries; each GPU the
// library runs on holds its own copy until the process ends.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "loglin.h"

namespace {
constexpr size_t kScratchBytes = size_t(LOGLIN_NOALLOC_SCRATCH_MIB) << 20;
constexpr int kMaxDevices = 64;
}  // namespace

// The workspace of loglin_fwd_noalloc.  In host code this name is only a
// stand-in: kernels get the device address looked up below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept for later calls.
int current_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LOGLIN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LOGLIN_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return LOGLIN_OK;
}

}  // namespace

extern "C" {

size_t loglin_noalloc_scratch_bytes(void) { return kScratchBytes; }

int loglin_fwd_noalloc(const void* X, const void* B, const void* C, const float* log_a,
                       const void* lambda, int chunk, void* out, const loglin_dims* dims,
                       void* stream) {
  // Host checks first: the arguments, then the workspace against the fixed
  // array (the address below only stands in for it: aligned, never used).
  const size_t need = loglin_workspace_bytes(dims, chunk);
  const void* stand_in = reinterpret_cast<const void*>(uintptr_t(256));
  int rc = loglin_validate(X, B, C, log_a, lambda, chunk, out, dims, stand_in,
                           need > kScratchBytes ? need : kScratchBytes, nullptr);
  if (rc) return rc;
  if (need > kScratchBytes) return LOGLIN_ERR_SCRATCH;
  void* ws = nullptr;
  rc = current_scratch(&ws);
  if (rc) return rc;
  return loglin_fwd(X, B, C, log_a, lambda, chunk, out, dims, ws, kScratchBytes, stream);
}

}  // extern "C"
