// Allocation-free acceptance: spdec_acceptance with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops).
//
// The array is zero when the code object loads on a device and every call
// leaves its leading sync region zero again, which is all the acceptance
// kernels need from a fresh workspace. Each device holds its own copy until
// the process ends; its device address is looked up once per device, with
// that device current, and kept. In host code `scratch` names a host-side
// stand-in, so only the looked-up address is ever passed to a kernel.
#include <atomic>
#include <mutex>

#include "launch.h"
#include "spdec.h"

namespace {

constexpr size_t kScratchBytes = (size_t)SPDEC_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's `scratch` (looked up on the first call per device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" spdec_status spdec_acceptance_noalloc(const float* logits_a, const float* logits_b, int rows, int vocab,
                                                 int64_t row_stride, float temperature, float* alpha, hipStream_t stream) {
  const spdec_status st = spdec::acceptance_args(logits_a, logits_b, rows, vocab, row_stride, temperature, alpha);
  if (st != SPDEC_OK) return st;
  if (spdec::acceptance_workspace_bytes(rows, vocab) > kScratchBytes) return SPDEC_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return SPDEC_ERR_HIP;
  const hipError_t e = spdec::launch_acceptance(logits_a, logits_b, rows, vocab, row_stride, temperature, alpha, ws,
                                                stream, nullptr);
  return e == hipSuccess ? SPDEC_OK : SPDEC_ERR_HIP;
}
