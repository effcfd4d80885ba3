// Backward entry point that allocates nothing: its workspace is a fixed device array.
//
// attn_bwd needs scratch memory (the row statistics -Delta and LSE * log2(e), the planner's two
// item lists, a dense mask's bits) that the caller normally provides. Callers that cannot allocate
// (code under HIP graph capture, tight serving loops) call attn_bwd_noalloc instead, which runs the
// same kernels on `scratch`, a file-scope device array of kScratchBytes. Each device the library
// runs on holds its own copy of the array until the process ends. The array's address on a device
// is looked up once, with that device current, by hipGetSymbolAddress; host code uses only that
// address (the array's name on the host is a stand-in, not a device address).
//
// Every call on one device shares that device's array and leaves the previous call's contents in
// it: nothing the kernels read starts at zero (each call writes the statistics and lists it reads),
// but calls that overlap in time on one device (different streams or threads) race on the array.
#include <hip/hip_runtime.h>

#include <atomic>

#include "api_internal.h"
#include "attn.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch`, per device; null until looked up

// Workspace provider of attn_bwd_noalloc: the current device's copy of `scratch`, looked up on the
// first call on that device. Rejects a problem whose workspace would not fit before any HIP call.
attn_status scratch_of_current_device(size_t need, void** workspace, size_t* bytes) {
  if (need > kScratchBytes) return ATTN_ERR_TOO_LARGE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return ATTN_ERR_HIP;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *workspace = ptr;
  *bytes = kScratchBytes;
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_bwd_noalloc_scratch_bytes(void) { return kScratchBytes; }

attn_status attn_bwd_noalloc(const attn_problem* problem, const void* Q, const void* K, const void* V,
                             const void* O, const void* dO, const float* LSE, const attn_mask* mask, float scale,
                             void* dQ, void* dK, void* dV, void* stream) {
  return attn::bwd_call(problem, Q, K, V, O, dO, LSE, mask, scale, dQ, dK, dV, nullptr, 0, 0, stream,
                        scratch_of_current_device);
}

}  // extern "C"
