// fa_forward_ex without a caller workspace: the split-KV partials go to a
// fixed scratch array that the library holds on each device, so the call
// allocates nothing (for callers that cannot allocate: code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array.  Its name in host code is a
// host-side stand-in, not a device address: the address of each device's
// copy is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; only that address is handed to kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fa.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` per device id (nullptr: not looked up yet).
std::atomic<void*> g_scratch[kMaxDevices];

// This device's copy of the scratch array, looked up on the first call on
// the device.  Concurrent first calls may both look it up; they store the
// same address.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_DEVICE;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FA_OK;
}

}  // namespace

extern "C" int fa_forward_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
                                     int dtype, int num_splits, void* stream) {
  // the workspace fa_forward_ex would need (this also checks the sizes,
  // the storage type and the split count)
  const int64_t need = fa_forward_ex_workspace_bytes(B, H, N, D, dtype, causal, num_splits);
  if (need < 0) return (int)need;
  if (need > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(&ws);
    if (st != FA_OK) return st;
  }
  // Every partial the merge reads is written by the range kernel of the
  // same call, so nothing in the scratch has to start at zero.
  return fa_forward_ex(q, k, v, o, lse, B, H, N, D, scale, causal, dtype, num_splits, ws,
                       need > 0 ? kScratchBytes : 0, stream);
}
