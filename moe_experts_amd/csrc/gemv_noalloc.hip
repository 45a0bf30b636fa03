// Allocation-free q4_0_gemv for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc). The
// K-split partial sums live in a static device array instead of a workspace
// argument; the kernels are the ones q4_0_gemv launches.
#include "q4moe.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr size_t kScratchBytes = (size_t)Q4_GEMV_NOALLOC_MAX_WS;
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends. Host code
// never uses this name as an address: the device address of each GPU's copy
// comes from hipGetSymbolAddress (scratch_on_current_device).
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return Q4_EHIP;
  if (dev >= kMaxDevices) return Q4_ETOOBIG;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return Q4_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return Q4_OK;
}

}  // namespace

extern "C" {

int q4_0_gemv_noalloc(const float* x, const q4_0_block* B, float* y, int M, int N, int K,
                      void* stream) {
  // q4_0_gemv_workspace_bytes is host arithmetic only; an unsupported shape
  // gives 0 here and its own error from q4_0_gemv below.
  const size_t need = q4_0_gemv_workspace_bytes(M, N, K);
  if (need > kScratchBytes) return Q4_ETOOBIG;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_on_current_device(&ws);
    if (rc != Q4_OK) return rc;
  }
  return q4_0_gemv(x, B, y, M, N, K, ws, need, stream);
}

}  // extern "C"
