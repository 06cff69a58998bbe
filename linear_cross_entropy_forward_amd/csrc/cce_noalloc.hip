// The forward without a caller-provided state buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): its state (counters, per-block partials,
// per-row loss, column sums) lives in one static device array per GPU.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/cce.h"
#include "cce_internal.hpp"

namespace cce {

constexpr size_t kScratchBytes = CCE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

// Every GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current.  The array's name in host code is a host-side stand-in,
// not a device address: only these pointers reach the kernels.
constexpr int kMaxDevices = 64;
static void* g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

static cce_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CCE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CCE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CCE_OK;
}

}  // namespace cce

extern "C" cce_status cce_forward_noalloc(const void* e, const void* c, const void* bias, const int64_t* targets,
                                          int64_t N, int64_t D, int64_t V, int dtype, int64_t ignore_index,
                                          int reduction, float softcap, float label_smoothing, float z_loss,
                                          float* loss, float* lse, int32_t* n_valid, cce_stream_t stream) {
  // sizes first: an oversized problem is refused before any HIP call
  const size_t need = cce_state_size(N, D, V, dtype);
  if (need == 0) return CCE_ERR_INVALID_ARG;
  if (need > cce::kScratchBytes) return CCE_ERR_WORKSPACE;
  void* state = nullptr;
  const cce_status st = cce::scratch_on_current_device(&state);
  if (st != CCE_OK) return st;
  // the same validation and kernels as cce_forward, with the device array as
  // the state; the forward writes every state word it later reads (nothing
  // in it needs to start at zero)
  return cce_forward(e, c, bias, targets, N, D, V, dtype, ignore_index, reduction, softcap, label_smoothing, z_loss,
                     loss, lse, n_valid, state, cce::kScratchBytes, stream);
}
