// C ABI of the forward library: argument checks, kernel choice, launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "fa.h"
#include "fa_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, -1 = other device.
std::atomic<int> g_device_ok[kMaxDevices];

bool head_dim_supported(int64_t D) { return D == 64 || D == 96 || D == 128; }

bool ranges_overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// Is the current device a gfx950?  Cached per device id.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_DEVICE;
  if (dev >= kMaxDevices) return FA_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_DEVICE;
    state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? FA_OK : FA_ERR_DEVICE;
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
               int64_t N, int64_t D, float scale, int causal, int dtype, void* stream) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 0 || D < 1) return FA_ERR_DIM;
  if (!head_dim_supported(D)) return FA_ERR_UNSUPPORTED_D;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (N == 0) return FA_OK;
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;

  // Sizes: per-head indexing is 32-bit, the grid is one workgroup per block
  // of query rows of every head.
  const int64_t block_m = dtype == FA_F32 ? fa::kF32BlockM : fa::kMfmaBlockM;
  if (N * D >= ((int64_t)1 << 31)) return FA_ERR_TOO_LARGE;
  if (B > ((int64_t)1 << 31) / H) return FA_ERR_TOO_LARGE;
  const int64_t BH = B * H;
  const int64_t qtiles = (N + block_m - 1) / block_m;
  if (BH > (((int64_t)1 << 31) - 1) / qtiles) return FA_ERR_TOO_LARGE;
  const int64_t elem = dtype == FA_F32 ? 4 : 2;
  if (BH > INT64_MAX / (N * D * elem)) return FA_ERR_TOO_LARGE;
  const size_t bytes = (size_t)(BH * N * D * elem);
  if (ranges_overlap(o, bytes, q, bytes) || ranges_overlap(o, bytes, k, bytes) ||
      ranges_overlap(o, bytes, v, bytes))
    return FA_ERR_ALIAS;

  const int dev = check_device();
  if (dev != FA_OK) return dev;

  fa::Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.BH = BH;
  p.N = (int)N;
  p.D = (int)D;
  p.scale = scale;
  p.causal = causal != 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err;
  switch (dtype) {
    case FA_F16: err = fa::launch_mfma_f16(p, s); break;
    case FA_BF16: err = fa::launch_mfma_bf16(p, s); break;
    default: err = fa::launch_f32(p, s); break;
  }
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a tensor pointer is NULL";
    case FA_ERR_DIM: return "invalid sizes (need B >= 1, H >= 1, N >= 0, D >= 1)";
    case FA_ERR_UNSUPPORTED_D: return "unsupported head dimension (supported: 64, 96, 128)";
    case FA_ERR_DTYPE: return "unknown dtype (FA_F32, FA_F16 or FA_BF16)";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_ALIAS: return "output overlaps an input";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_TOO_LARGE: return "problem too large (N*D must be < 2^31)";
    case FA_ERR_DEVICE: return "current HIP device is not a gfx950 (MI355X)";
    default: return "unknown status";
  }
}

const char* fa_version(void) { return "fa-mi355x 0.1.0 gfx950"; }

}  // extern "C"
