// verify_block_noalloc: verify_block with its workspace in a file-scope
// device array instead of caller memory, for callers that cannot allocate
// (code under HIP graph capture, serving loops that never call hipMalloc).
//
// The array `scratch` is this library's own, one copy per GPU, held until
// the process ends.  Host code never passes its name to a kernel (on the
// host the name stands for a host-side shadow, not device memory): the
// device address is looked up once per device with hipGetSymbolAddress, at
// the first call with that device current, and only that address is used.
// Each call first clears the arrival counters at the start of the array
// with a small kernel (no memset node in a captured graph), then runs
// verify_block on the array.  Calls on one GPU share the array: calls that
// overlap in time on one GPU race (serialise them on one stream).

#include "acceptmoe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "amoe_launch.h"

namespace {

constexpr size_t kScratchBytes = ACCEPTMOE_NOALLOC_WORKSPACE_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device (looked up once).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return amoe::set_error(ACCEPTMOE_EHIP, "verify_block_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return amoe::set_error(ACCEPTMOE_EINVAL, "verify_block_noalloc: device index out of range");
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return amoe::set_error(ACCEPTMOE_EHIP,
                               "verify_block_noalloc: hipGetSymbolAddress(scratch) failed");
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ACCEPTMOE_OK;
}

__global__ __launch_bounds__(256) void clear_words(uint32_t* p, int n) {
  for (int i = static_cast<int>(threadIdx.x); i < n; i += 256) p[i] = 0u;
}

}  // namespace

extern "C" int verify_block_noalloc(const acceptmoe_shape* shape, const acceptmoe_inputs* in,
                                    const acceptmoe_outputs* out, hipStream_t stream) {
  size_t need = 0;
  int rc = amoe::check_verify_args(shape, in, out, &need);
  if (rc) return rc;
  if (need > kScratchBytes)
    return amoe::set_error(ACCEPTMOE_EINVAL,
                           "verify_block_noalloc: the shape needs more workspace than the "
                           "library's ACCEPTMOE_NOALLOC_WORKSPACE_BYTES; use verify_block");
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  const int words = static_cast<int>(amoe::workspace_counter_bytes() / 4);
  clear_words<<<1, 256, 0, stream>>>(static_cast<uint32_t*>(ws), words);
  if (hipGetLastError() != hipSuccess)
    return amoe::set_error(ACCEPTMOE_EHIP, "verify_block_noalloc: clearing the counters failed");
  return verify_block(shape, in, out, ws, kScratchBytes, stream);
}
