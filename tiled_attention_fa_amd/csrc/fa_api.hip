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

// Checks shared by both forward entry points, in the documented order
// (dtype, sizes, head dim, scale, N == 0, pointers, alignment, size limits,
// aliasing).  *BH receives B * H.  Returns FA_OK, a negative status, or 1
// for an accepted N == 0 call (nothing to do).
int validate(const void* q, const void* k, const void* v, const void* o, int64_t B, int64_t H,
             int64_t N, int64_t D, float scale, int dtype, int64_t block_m, int64_t* BH) {
  if (B < 1 || H < 1 || N < 0 || D < 1) return FA_ERR_DIM;
  if (!head_dim_supported(D)) return FA_ERR_UNSUPPORTED_D;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (N == 0) return 1;
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;

  // Sizes: per-head indexing is 32-bit; the grid is one workgroup per block
  // of query rows of every head, and its work-item count must fit in 32
  // bits (at most 512 work-items per 64 rows: 8 * N + 512 per head bounds
  // every kernel's total).
  if (N * D >= ((int64_t)1 << 31)) return FA_ERR_TOO_LARGE;
  if (B > ((int64_t)1 << 31) / H) return FA_ERR_TOO_LARGE;
  *BH = B * H;
  const int64_t qtiles = (N + block_m - 1) / block_m;
  if (*BH > (((int64_t)1 << 31) - 1) / qtiles) return FA_ERR_TOO_LARGE;
  if (*BH > (int64_t)UINT32_MAX / (8 * N + 512)) return FA_ERR_TOO_LARGE;
  const int64_t elem = dtype == FA_F32 ? 4 : 2;
  if (*BH > INT64_MAX / (N * D * elem)) return FA_ERR_TOO_LARGE;
  const size_t bytes = (size_t)(*BH * N * D * elem);
  if (ranges_overlap(o, bytes, q, bytes) || ranges_overlap(o, bytes, k, bytes) ||
      ranges_overlap(o, bytes, v, bytes))
    return FA_ERR_ALIAS;
  return FA_OK;
}

constexpr int64_t kWsAlign = 256;
// Longest rows of the three-pass path (a workgroup's 128 rows of P then
// span less than 2^31 bytes; the workspace for one such head is already
// 12 TiB).
constexpr int64_t kNaiveMaxN = (int64_t)1 << 20;

int64_t align_up(int64_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Workspace of the three-pass path: S (fp32, BH x N x NP), then P (16-bit,
// BH x N x NP), then for bf16 the low parts of P (same size); each part
// starts on a 256-byte boundary.  Returns the offsets, or false when the
// total does not fit in int64.
bool naive_layout(int64_t BH, int64_t N, int dtype, int64_t* p_off, int64_t* plo_off, int64_t* total) {
  const int64_t NP = (N + 63) / 64 * 64;
  if (N > 0 && BH > INT64_MAX / 16 / N / NP) return false;  // 4 + 2 + 2 bytes per entry, with room
  const int64_t s_bytes = BH * N * NP * 4;
  const int64_t p_bytes = BH * N * NP * 2;
  *p_off = align_up(s_bytes);
  *plo_off = align_up(*p_off + p_bytes);
  *total = dtype == FA_BF16 ? align_up(*plo_off + p_bytes) : *plo_off;
  return true;
}

fa::Problem dense_problem(const void* q, const void* k, const void* v, void* o, int64_t H, int64_t BH,
                          int64_t N, int64_t D, float scale, int causal) {
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
  p.H = (int)H;
  p.group = 1;
  p.lq = p.lk = p.lv = p.lo = fa::dense_layout(H, N, D);
  return p;
}

hipError_t launch_kernel(const fa::Problem& p, int dtype, hipStream_t s) {
  switch (dtype) {
    case FA_F16: return fa::launch_mfma_f16(p, s);
    case FA_BF16: return fa::launch_mfma_bf16(p, s);
    default: return fa::launch_f32(p, s);
  }
}

int launch_forward(const fa::Problem& p, int dtype, hipStream_t s) {
  return launch_kernel(p, dtype, s) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Elements from a tensor's base to one past its last element, for the
// (b, h, n) extents and strides given (d contiguous, D wide); -1 when that
// does not fit in int64.
int64_t extent_elems(const int64_t* st, int64_t B, int64_t Hx, int64_t N, int64_t D) {
  const __int128 e = (__int128)(B - 1) * st[0] + (__int128)(Hx - 1) * st[1] + (__int128)(N - 1) * st[2] + D;
  return e > (__int128)(INT64_MAX / 8) ? -1 : (int64_t)e;
}

// No two (b, h, n) rows of a written tensor share an element: with the
// dimensions of more than one entry ordered by stride, each stride reaches
// past everything the smaller ones span.
bool rows_disjoint(const int64_t* st, int64_t B, int64_t Hx, int64_t N, int64_t D) {
  int64_t s[3] = {st[0], st[1], st[2]}, c[3] = {B, Hx, N};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (s[j] < s[i]) {
        const int64_t ts = s[i], tc = c[i];
        s[i] = s[j];
        c[i] = c[j];
        s[j] = ts;
        c[j] = tc;
      }
  __int128 span = D;  // elements spanned by the dimensions placed so far
  for (int i = 0; i < 3; ++i) {
    if (c[i] <= 1) continue;
    if ((__int128)s[i] < span) return false;
    span += (__int128)s[i] * (c[i] - 1);
  }
  return true;
}

constexpr int kMaxSplits = 64;
std::atomic<int> g_cus[kMaxDevices];  // CU count per device, 0 = not queried yet

// CUs of the current device (cached), or a negative status.
int current_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_DEVICE;
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return FA_ERR_DEVICE;
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Workgroup shape of the fp32 kernel: key groups (returned) and waves of 16
// rows per group (*row_waves), from the fp32 calibration sweep on MI355X
// (22 grids, tile_sweep.py; f = B*H times the blocks of 64 rows over the
// CUs):
//  * f < 1, and causal f <= 1: the grid leaves SIMDs idle (or, causal, the
//    rows that see every key set the time), and the shape with the least
//    work on one SIMD runs (workgroups per CU x waves per SIMD x key tiles
//    per group); on a tie, more waves per SIMD: 32 rows in four groups (8
//    waves), 16 rows in four, 32 rows in two, 64 rows in two.  Up to 2.5x
//    faster than 64-row workgroups on the smallest grids, 12-35% on causal
//    grids of one pass.
//  * causal 1 < f <= 2: D = 64, 32 rows in two groups (20% faster); D = 96
//    and 128, 64 rows in two groups.
//  * fuller grids: 64 rows, in two groups once the rows have 8 or more
//    32-key tiles (5-12% faster there), except non-causal D = 128 from
//    f = 2 on, where one group runs 8% faster (two 4-wave workgroups per
//    CU in one pass, against 8-wave workgroups that registers hold to one
//    per CU).
int f32_key_groups(int64_t BH, int64_t N, int64_t D, bool causal, int cus, int* row_waves) {
  *row_waves = 4;
  const int64_t w4 = BH * ((N + 63) / 64);
  if (N <= 32) return 1;
  if (w4 < cus || (causal && w4 <= cus)) {
    const int64_t nt = (N + 31) / 32;
    static const int shapes[4][2] = {{2, 4}, {1, 4}, {2, 2}, {4, 2}};
    int64_t best = INT64_MAX;
    int kg = 1;
    for (const auto& sh : shapes) {
      const int rw = sh[0], g = sh[1];
      const int64_t wgs = BH * ((N + 16 * rw - 1) / (16 * rw));
      const int64_t per_simd = (wgs + cus - 1) / cus * (rw * g / 4) * ((nt + g - 1) / g);
      if (per_simd < best) {
        best = per_simd;
        kg = g;
        *row_waves = rw;
      }
    }
    return kg;
  }
  if (causal && w4 <= 2 * (int64_t)cus) {
    if (D == 64) *row_waves = 2;
    return 2;
  }
  if (!causal && D == 128 && w4 >= 2 * (int64_t)cus) return 1;
  return N >= 256 ? 2 : 1;
}

// Key-range splits that fill the device: enough workgroups for every
// resident slot, while each range keeps at least 16 key tiles (measured on
// MI355X: below that the partials' round trip through memory and the merge
// cost more than the extra workgroups gain).
int suggest_splits(int64_t BH, int64_t N, int64_t D, int dtype, bool causal, int cus) {
  const bool f32 = dtype == FA_F32;
  const int64_t block_m = f32 ? fa::kF32BlockM : 32 * fa::mfma_waves((int)D, causal);
  const int64_t per_cu = f32 ? 1 : fa::mfma_wgs_per_cu((int)D, causal);
  const int64_t bn = f32 ? 32 : 64;
  const int64_t total = BH * ((N + block_m - 1) / block_m);
  const int64_t slots = (int64_t)cus * per_cu;
  if (N == 0 || total >= slots) return 1;
  int64_t s = slots / total;
  const int64_t by_tiles = ((N + bn - 1) / bn) / 16;
  if (s > by_tiles) s = by_tiles;
  if (s > 16) s = 16;
  if (s < 1) return 1;
  if (f32) {
    // fp32: the key-group shapes of one range compete; the ranges (64-row
    // workgroups, one group) win unless the one-range shape leaves less
    // key-tile work on one SIMD (3-13% faster on a tie, measured; 35% slower
    // where the 16-row shape halves it)
    int rw = 4;
    const int kg = f32_key_groups(BH, N, D, causal, cus, &rw);
    const int64_t nt = (N + 31) / 32;
    const int64_t wgs = BH * ((N + 16 * rw - 1) / (16 * rw));
    const int64_t one = (wgs + cus - 1) / cus * (rw * kg / 4) * ((nt + kg - 1) / kg);
    const int64_t split = (total * s + cus - 1) / cus * ((nt + s - 1) / s);
    if (one < split) return 1;
  }
  return (int)s;
}

// Key groups per workgroup (1, 2 or 4) for the matrix-core kernel, and the
// waves of the multi-group workgroup (*ks_waves, 4 or 8), measured on MI355X.
// Two groups halve each workgroup's chain of key tiles; the workgroup shape
// decides how many passes of workgroups over the CUs the grid needs.  Rows within one key
// tile have nothing to split.
//  * Non-causal, with w = B*H times the blocks of 256 rows: w <= CUs / 4
//    takes 4-wave workgroups of 64 rows (all CUs busy in one pass; 24-47%
//    faster); w <= CUs / 2 at D = 64 and 128 takes 8-wave workgroups of 128
//    rows (one pass, two waves per SIMD; 4-30% faster); fuller grids, and
//    D = 96 beyond a quarter, run faster with one group.
//  * Causal, with the one-group grid's fill of the device's workgroup
//    slots: up to one half, 4-wave workgroups; up to three quarters, where
//    the rows that see every key set the time, 4 waves at D = 64 and 8 at
//    D = 96 and 128 (2-29% faster), except bf16 at D = 96 and 128, which
//    runs one group in that band too (its two-group kernels always form the
//    two-term P; one group runs 6-17% faster); up to one pass with rows of
//    4096 keys or more, 8-wave workgroups in two groups (four at D = 96;
//    bf16 at D = 128 excepted); fuller grids run one group.
//  * At D = 96 and 128, where those rules take the 4-wave two-group shape,
//    four groups of two 32-row blocks with 32-key tiles run instead (8
//    waves, two per SIMD, each chain a quarter of the keys; 1.5-7% faster
//    in the sweep; at D = 64 they are slower).
int suggest_key_groups(int64_t BH, int64_t N, int64_t D, int dtype, bool causal, int cus, int* ks_waves) {
  *ks_waves = fa::mfma_ks_waves;
  if (dtype == FA_F32) {
    int row_waves = 4;
    return f32_key_groups(BH, N, D, causal, cus, &row_waves);
  }
  if (N <= 64) return 1;
  // the 4-wave two-group shape, or four groups where they measured faster
  auto small = [&]() {
    if (D == 64) return 2;
    *ks_waves = 8;
    return 4;
  };
  if (!causal) {
    const int64_t w = BH * ((N + 255) / 256);
    if (4 * w <= cus) return small();
    if (D != 96 && 2 * w <= cus) {
      *ks_waves = 8;
      return 2;
    }
    return 1;
  }
  const int64_t block_m = 32 * fa::mfma_waves((int)D, causal);
  const int64_t total = BH * ((N + block_m - 1) / block_m);
  const int64_t slots = (int64_t)cus * fa::mfma_wgs_per_cu((int)D, causal);
  if (2 * total <= slots) return small();
  // (at D = 64 a grid of exactly three quarters runs one group: 4-8% faster)
  if (4 * total < 3 * slots || (D != 64 && 4 * total == 3 * slots)) {
    if (dtype == FA_BF16 && D != 64) return 1;
    if (D != 64) *ks_waves = 8;
    return 2;
  }
  // up to one pass with rows of 4096 keys or more: the blocks that see
  // every key set the time, and 8-wave workgroups in two groups (four at
  // D = 96) halve (quarter) their chains: 3-12% faster at N = 4096 and 8192
  // (bf16 at D = 128 keeps one group: its two-group kernel splits P on
  // every tile)
  if (total <= slots && N >= 4096 && !(dtype == FA_BF16 && D == 128)) {
    *ks_waves = 8;
    return D == 96 ? 4 : 2;
  }
  return 1;
}

// The one-group shape of causal grids where it differs from the table
// (measured on MI355X with the causal calibration sweep; f = the table
// shape's workgroups over the CUs' workgroup slots):
//   D = 64:  32-key tiles beyond a pass and a quarter (f > 1.25), 4-10%
//            faster; fp16 at about two passes (1.5 < f <= 2.5) 8 waves with
//            64-key tiles instead, 4-6% faster;
//   D = 96:  32-key tiles from three passes (f >= 3), which halves the ring
//            and fits two workgroups per CU, 15-20% faster;
//   D = 128: 2 waves with 32-key tiles up to one pass (f <= 1; for fp16 only
//            above 3/4, where the key groups do not run), 4-21% faster; 4
//            waves with 32-key tiles beyond: bf16 always (the 8-wave bf16
//            kernel has too few registers for split P), fp16 for 1 < f < 2
//            with rows below 8192 keys and for f >= 3 (2-9%), the table's 8
//            waves otherwise.
// Sets *waves1 and *block_n1 (0 = the table's).
void one_group_shape(int64_t BH, int64_t N, int64_t D, int dtype, bool causal, int cus, int* waves1,
                     int* block_n1) {
  *waves1 = 0;
  *block_n1 = 0;
  if (dtype == FA_F32 || !causal || N <= 64) return;
  const int64_t block_m = 32 * fa::mfma_waves((int)D, causal);
  const int64_t total = BH * ((N + block_m - 1) / block_m);
  const int64_t slots = (int64_t)cus * fa::mfma_wgs_per_cu((int)D, causal);
  if (D == 64) {
    if (dtype == FA_F16 && 2 * total > 3 * slots && 2 * total <= 5 * slots) {
      *waves1 = 8;  // about two passes: 8 waves, 64-key tiles (4-6%)
      return;
    }
    if (4 * total > 5 * slots) *block_n1 = 32;
  } else if (D == 96) {
    if (total >= 3 * slots) *block_n1 = 32;
  } else if (D == 128) {
    if (total <= slots) {
      *waves1 = 2;
    } else if (dtype == FA_BF16 || (total < 2 * slots && N < 8192) || total >= 3 * slots) {
      *waves1 = 4;
    } else {
      return;
    }
    *block_n1 = 32;
  }
}

// Key groups and workgroup shape of a forward problem with one key range.
void choose_shape(fa::Problem& p, int dtype, int cus) {
  const bool causal = p.causal;
  if (dtype == FA_F32) {
    p.key_groups = f32_key_groups(p.BH, p.N, p.D, causal, cus, &p.f32_row_waves);
    return;
  }
  p.key_groups = suggest_key_groups(p.BH, p.N, p.D, dtype, causal, cus, &p.ks_waves);
  if (p.key_groups == 1) one_group_shape(p.BH, p.N, p.D, dtype, causal, cus, &p.waves1, &p.block_n1);
}

// Workspace of split-KV: the fp32 partials [splits, BH, N, D], then their
// log-sum-exp [splits, BH, N], each on a 256-byte boundary.  -1 when the
// size does not fit in int64.
int64_t split_layout(int64_t BH, int64_t N, int64_t D, int splits, int64_t* lse_off) {
  *lse_off = 0;
  if (splits <= 1 || N == 0) return 0;
  if (BH > INT64_MAX / 8 / splits / N / (D + 1)) return -1;
  const int64_t o_bytes = (int64_t)splits * BH * N * D * 4;
  *lse_off = align_up(o_bytes);
  return align_up(*lse_off + (int64_t)splits * BH * N * 4);
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
               int64_t N, int64_t D, float scale, int causal, int dtype, void* stream) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  int64_t BH = 0;
  const int64_t block_m = dtype == FA_F32 ? fa::kF32BlockM : fa::kMfmaBlockM;
  const int st = validate(q, k, v, o, B, H, N, D, scale, dtype, block_m, &BH);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;

  const int dev = check_device();
  if (dev != FA_OK) return dev;
  const int cus = current_cus();
  if (cus < 0) return cus;

  fa::Problem p = dense_problem(q, k, v, o, H, BH, N, D, scale, causal);
  choose_shape(p, dtype, cus);
  return launch_forward(p, dtype, (hipStream_t)stream);
}

int64_t fa_naive_workspace_bytes(int64_t B, int64_t H, int64_t N, int dtype) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 0) return FA_ERR_DIM;
  if (B > INT64_MAX / H) return FA_ERR_TOO_LARGE;
  int64_t p_off, plo_off, total;
  if (!naive_layout(B * H, N, dtype, &p_off, &plo_off, &total)) return FA_ERR_TOO_LARGE;
  return total;
}

int fa_naive_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                     int64_t N, int64_t D, float scale, int causal, int dtype, void* workspace,
                     int64_t workspace_bytes, void* stream) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  int64_t BH = 0;
  const int st = validate(q, k, v, o, B, H, N, D, scale, dtype, fa::kMfmaBlockM, &BH);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  if (N > kNaiveMaxN) return FA_ERR_TOO_LARGE;
  int64_t p_off, plo_off, total;
  if (!naive_layout(BH, N, dtype, &p_off, &plo_off, &total)) return FA_ERR_TOO_LARGE;
  if (!workspace || ((uintptr_t)workspace & (kWsAlign - 1)) || workspace_bytes < total)
    return FA_ERR_WORKSPACE;
  const size_t bytes = (size_t)(BH * N * D * 2);
  if (ranges_overlap(workspace, (size_t)total, q, bytes) || ranges_overlap(workspace, (size_t)total, k, bytes) ||
      ranges_overlap(workspace, (size_t)total, v, bytes) || ranges_overlap(workspace, (size_t)total, o, bytes))
    return FA_ERR_WORKSPACE;

  const int dev = check_device();
  if (dev != FA_OK) return dev;

  fa::NaiveProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.s = workspace;
  p.p = (char*)workspace + p_off;
  p.plo = dtype == FA_BF16 ? (char*)workspace + plo_off : nullptr;
  p.BH = BH;
  p.N = (int)N;
  p.NP = (int)((N + 63) / 64 * 64);
  p.D = (int)D;
  p.scale = scale;
  p.causal = causal != 0;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t err = dtype == FA_F16 ? fa::launch_naive_f16(p, s) : fa::launch_naive_bf16(p, s);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_splitkv_suggest(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int causal) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 0 || D < 1) return FA_ERR_DIM;
  if (!head_dim_supported(D)) return FA_ERR_UNSUPPORTED_D;
  if (B > ((int64_t)1 << 31) / H) return FA_ERR_TOO_LARGE;
  const int cus = current_cus();
  if (cus < 0) return cus;
  return suggest_splits(B * H, N, D, dtype, causal != 0, cus);
}

int fa_key_groups_suggest(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int causal) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 0 || D < 1) return FA_ERR_DIM;
  if (!head_dim_supported(D)) return FA_ERR_UNSUPPORTED_D;
  if (B > ((int64_t)1 << 31) / H) return FA_ERR_TOO_LARGE;
  const int cus = current_cus();
  if (cus < 0) return cus;
  int waves = 0;
  return suggest_key_groups(B * H, N, D, dtype, causal != 0, cus, &waves);
}

int fa_workgroup_shape(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int causal, int* waves,
                       int* key_groups, int* block_n) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 0 || D < 1) return FA_ERR_DIM;
  if (!head_dim_supported(D)) return FA_ERR_UNSUPPORTED_D;
  if (B > ((int64_t)1 << 31) / H) return FA_ERR_TOO_LARGE;
  const int cus = current_cus();
  if (cus < 0) return cus;
  fa::Problem p{};
  p.BH = B * H;
  p.N = (int)std::min<int64_t>(N, INT32_MAX);
  p.D = (int)D;
  p.causal = causal != 0;
  choose_shape(p, dtype, cus);
  int w = p.ks_waves, g = p.key_groups, bn = p.key_groups == 4 ? 32 : 64;
  if (dtype == FA_F32) {
    w = p.f32_row_waves * p.key_groups;
    bn = 32;
  } else if (p.key_groups == 1) {
    g = 1;
    w = p.waves1 ? p.waves1 : fa::mfma_waves(p.D, p.causal);
    bn = p.block_n1 ? p.block_n1 : fa::mfma_block_n(p.D, dtype == FA_BF16);
  }
  if (waves) *waves = w;
  if (key_groups) *key_groups = g;
  if (block_n) *block_n = bn;
  return FA_OK;
}

int64_t fa_forward_ex_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int causal,
                                      int num_splits) {
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_SPLITS;
  int splits = num_splits;
  if (splits == 0) {
    splits = fa_splitkv_suggest(B, H, N, D, dtype, causal);
    if (splits < 0) return splits;
  }
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 0 || D < 1) return FA_ERR_DIM;
  if (!head_dim_supported(D)) return FA_ERR_UNSUPPORTED_D;
  if (B > ((int64_t)1 << 31) / H) return FA_ERR_TOO_LARGE;
  int64_t lse_off;
  const int64_t bytes = split_layout(B * H, N, D, splits, &lse_off);
  return bytes < 0 ? FA_ERR_TOO_LARGE : bytes;
}

int fa_forward_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                  int64_t N, int64_t D, float scale, int causal, int dtype, int num_splits, void* workspace,
                  int64_t workspace_bytes, void* stream) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  int64_t BH = 0;
  const int64_t block_m = dtype == FA_F32 ? fa::kF32BlockM : fa::kMfmaBlockM;
  const int st = validate(q, k, v, o, B, H, N, D, scale, dtype, block_m, &BH);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_SPLITS;
  const int64_t elem = dtype == FA_F32 ? 4 : 2;
  const size_t bytes = (size_t)(BH * N * D * elem);
  if (lse != nullptr) {
    if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
    const size_t lbytes = (size_t)(BH * N * 4);
    if (ranges_overlap(lse, lbytes, q, bytes) || ranges_overlap(lse, lbytes, k, bytes) ||
        ranges_overlap(lse, lbytes, v, bytes) || ranges_overlap(lse, lbytes, o, bytes))
      return FA_ERR_ALIAS;
  }
  int splits = num_splits;
  if (splits == 0) {
    const int cus = current_cus();
    if (cus < 0) return cus;
    splits = suggest_splits(BH, N, D, dtype, causal != 0, cus);
  }
  // grid: every (head, query block, range) is one workgroup
  const int64_t qtiles = (N + block_m - 1) / block_m;
  if (BH * splits > (((int64_t)1 << 31) - 1) / qtiles) return FA_ERR_TOO_LARGE;
  if (BH * splits > (int64_t)UINT32_MAX / (8 * N + 512)) return FA_ERR_TOO_LARGE;
  int64_t lse_off = 0;
  if (splits > 1) {
    const int64_t need = split_layout(BH, N, D, splits, &lse_off);
    if (need < 0) return FA_ERR_TOO_LARGE;
    if (!workspace || ((uintptr_t)workspace & (kWsAlign - 1)) || workspace_bytes < need)
      return FA_ERR_WORKSPACE;
    if (ranges_overlap(workspace, (size_t)need, q, bytes) || ranges_overlap(workspace, (size_t)need, k, bytes) ||
        ranges_overlap(workspace, (size_t)need, v, bytes) || ranges_overlap(workspace, (size_t)need, o, bytes) ||
        (lse != nullptr && ranges_overlap(workspace, (size_t)need, lse, (size_t)(BH * N * 4))))
      return FA_ERR_WORKSPACE;
  }

  const int dev = check_device();
  if (dev != FA_OK) return dev;

  fa::Problem p = dense_problem(q, k, v, o, H, BH, N, D, scale, causal);
  p.splits = splits;
  p.lse = splits == 1 ? lse : nullptr;
  if (splits == 1) {
    const int cus = current_cus();
    if (cus < 0) return cus;
    choose_shape(p, dtype, cus);
  }
  if (splits > 1) {
    p.part_o = (float*)workspace;
    p.part_lse = (float*)((char*)workspace + lse_off);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = launch_kernel(p, dtype, s);
  if (err == hipSuccess && splits > 1) {
    fa::MergeProblem m;
    m.part_o = p.part_o;
    m.part_lse = p.part_lse;
    m.o = o;
    m.lse = lse;
    m.rows = BH * N;
    m.D = (int)D;
    m.splits = splits;
    m.dtype = dtype;
    err = fa::launch_split_merge(m, s);
  }
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_forward_strided(const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
                       const void* v, const int64_t* v_strides, void* o, const int64_t* o_strides, int64_t B,
                       int64_t H, int64_t H_kv, int64_t N, int64_t D, float scale, int causal, int dtype,
                       void* stream) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || H_kv < 1 || N < 0 || D < 1 || H % H_kv != 0) return FA_ERR_DIM;
  if (!head_dim_supported(D)) return FA_ERR_UNSUPPORTED_D;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (N == 0) return FA_OK;
  if (!q || !k || !v || !o || !q_strides || !k_strides || !v_strides || !o_strides) return FA_ERR_NULL;
  const int64_t elem = dtype == FA_F32 ? 4 : 2;
  const int64_t* st[4] = {q_strides, k_strides, v_strides, o_strides};
  const int64_t heads[4] = {H, H_kv, H_kv, H};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i)
      if (st[t][i] < 0) return FA_ERR_STRIDE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i)
      if ((st[t][i] * elem) % 16 != 0) return FA_ERR_ALIGN;
  for (int t = 0; t < 4; ++t)
    if (st[t][2] < D) return FA_ERR_STRIDE;  // the rows of one head do not overlap
  if (!rows_disjoint(o_strides, B, H, N, D)) return FA_ERR_STRIDE;

  // Sizes: per-head row offsets and the key/value buffer ranges are 32-bit
  // (max(N, 64) row strides of bytes below 2^32), the grid as fa_forward.
  if (N * D >= ((int64_t)1 << 31)) return FA_ERR_TOO_LARGE;
  for (int t = 0; t < 4; ++t)
    if ((N > 64 ? N : 64) * st[t][2] * elem >= ((int64_t)1 << 32)) return FA_ERR_TOO_LARGE;
  if (B > ((int64_t)1 << 31) / H) return FA_ERR_TOO_LARGE;
  const int64_t BH = B * H;
  const int64_t block_m = dtype == FA_F32 ? fa::kF32BlockM : fa::kMfmaBlockM;
  const int64_t qtiles = (N + block_m - 1) / block_m;
  if (BH > (((int64_t)1 << 31) - 1) / qtiles) return FA_ERR_TOO_LARGE;
  if (BH > (int64_t)UINT32_MAX / (8 * N + 512)) return FA_ERR_TOO_LARGE;
  int64_t ext[4];
  for (int t = 0; t < 4; ++t) {
    ext[t] = extent_elems(st[t], B, heads[t], N, D);
    if (ext[t] < 0) return FA_ERR_TOO_LARGE;
  }
  const void* ptr[3] = {q, k, v};
  for (int t = 0; t < 3; ++t)
    if (ranges_overlap(o, (size_t)(ext[3] * elem), ptr[t], (size_t)(ext[t] * elem))) return FA_ERR_ALIAS;

  const int dev = check_device();
  if (dev != FA_OK) return dev;
  const int cus = current_cus();
  if (cus < 0) return cus;

  fa::Problem p = dense_problem(q, k, v, o, H, BH, N, D, scale, causal);
  p.group = (int)(H / H_kv);
  choose_shape(p, dtype, cus);
  fa::Layout* lay[4] = {&p.lq, &p.lk, &p.lv, &p.lo};
  for (int t = 0; t < 4; ++t) *lay[t] = fa::Layout{st[t][0], st[t][1], (int)st[t][2]};
  return launch_forward(p, dtype, (hipStream_t)stream);
}

#ifdef FA_TILE_SWEEP
int fa_tune_shapes(int64_t D, int* waves, int* occupancy, int* key_groups, int* block_n, int capacity) {
  if (!head_dim_supported(D)) return FA_ERR_UNSUPPORTED_D;
  const int n = D == 64 ? fa::kTuneShapes64Count : fa::kTuneShapesWideCount;
  for (int i = 0; i < n && i < capacity; ++i) {
    const int* s = D == 64 ? fa::kTuneShapes64[i] : fa::kTuneShapesWide[i];
    if (waves) waves[i] = s[0];
    if (occupancy) occupancy[i] = s[1];
    if (key_groups) key_groups[i] = s[2];
    if (block_n) block_n[i] = s[3];
  }
  return n;
}

int fa_tune_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H, int64_t N,
                    int64_t D, float scale, int causal, int dtype, int waves, int occupancy, int key_groups,
                    int block_n, void* stream) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  int sw[16], so[16], sk[16], sb[16];
  const int n = fa_tune_shapes(D, sw, so, sk, sb, 16);
  bool known = false;
  for (int i = 0; i < n; ++i)
    known = known || (sw[i] == waves && so[i] == occupancy && sk[i] == key_groups && sb[i] == block_n);
  int64_t BH = 0;
  // rows per workgroup bound the grid (any positive block is safe to check
  // before the shape itself is; an unknown shape is rejected below)
  const int64_t block_m = known ? 32 * (int64_t)waves / key_groups : 32;
  const int st = validate(q, k, v, o, B, H, N, D, scale, dtype, block_m, &BH);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  if (!known) return FA_ERR_UNSUPPORTED_D;
  const int dev = check_device();
  if (dev != FA_OK) return dev;
  fa::Problem p = dense_problem(q, k, v, o, H, BH, N, D, scale, causal);
  p.key_groups = key_groups;
  const hipError_t err =
      dtype == FA_F16 ? fa::launch_mfma_shape_f16(p, waves, occupancy, key_groups, block_n, (hipStream_t)stream)
                      : fa::launch_mfma_shape_bf16(p, waves, occupancy, key_groups, block_n, (hipStream_t)stream);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_tune_f32_shapes(int64_t D, int* row_waves, int* key_groups, int capacity) {
  if (!head_dim_supported(D)) return FA_ERR_UNSUPPORTED_D;
  for (int i = 0; i < fa::kTuneF32ShapesCount && i < capacity; ++i) {
    if (row_waves) row_waves[i] = fa::kTuneF32Shapes[i][0];
    if (key_groups) key_groups[i] = fa::kTuneF32Shapes[i][1];
  }
  return fa::kTuneF32ShapesCount;
}

int fa_tune_forward_f32(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H, int64_t N,
                        int64_t D, float scale, int causal, int row_waves, int key_groups, void* stream) {
  int sr[8], sg[8];
  const int n = fa_tune_f32_shapes(D, sr, sg, 8);
  bool known = false;
  for (int i = 0; i < n; ++i) known = known || (sr[i] == row_waves && sg[i] == key_groups);
  int64_t BH = 0;
  const int64_t block_m = known ? 16 * (int64_t)row_waves : 16;
  const int st = validate(q, k, v, o, B, H, N, D, scale, FA_F32, block_m, &BH);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  if (!known) return FA_ERR_UNSUPPORTED_D;
  // up to 16 work-items per row here, against the 8 that validate bounds
  if (BH * ((N + block_m - 1) / block_m) * 64 * row_waves * key_groups > (int64_t)UINT32_MAX)
    return FA_ERR_TOO_LARGE;
  const int dev = check_device();
  if (dev != FA_OK) return dev;
  fa::Problem p = dense_problem(q, k, v, o, H, BH, N, D, scale, causal);
  const hipError_t err = fa::launch_f32_shape(p, row_waves, key_groups, (hipStream_t)stream);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

/* The split-KV merge alone, on caller-made partials (for its closed-form
 * checks): part_o [splits, rows, D] fp32 and part_lse [splits, rows] fp32 in,
 * o [rows, D] in the storage type and, if not NULL, lse [rows] out. */
int fa_tune_split_merge(const float* part_o, const float* part_lse, void* o, float* lse, int64_t rows, int64_t D,
                        int splits, int dtype, void* stream) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (rows < 0 || !head_dim_supported(D)) return FA_ERR_DIM;
  if (splits < 1 || splits > kMaxSplits) return FA_ERR_SPLITS;
  if (rows == 0) return FA_OK;
  if (!part_o || !part_lse || !o) return FA_ERR_NULL;
  if (((uintptr_t)part_o | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  const int dev = check_device();
  if (dev != FA_OK) return dev;
  fa::MergeProblem m;
  m.part_o = part_o;
  m.part_lse = part_lse;
  m.o = o;
  m.lse = lse;
  m.rows = rows;
  m.D = (int)D;
  m.splits = splits;
  m.dtype = dtype;
  return fa::launch_split_merge(m, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
#endif

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a tensor pointer is NULL";
    case FA_ERR_DIM: return "invalid sizes (need B >= 1, H >= 1, N >= 0, D >= 1)";
    case FA_ERR_UNSUPPORTED_D: return "unsupported head dimension (supported: 64, 96, 128)";
    case FA_ERR_DTYPE: return "dtype not accepted here (fa_forward: FA_F32, FA_F16, FA_BF16; naive: FA_F16, FA_BF16)";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_ALIAS: return "output overlaps an input";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_TOO_LARGE: return "problem too large (N*D must be < 2^31 and the grid must fit)";
    case FA_ERR_DEVICE: return "current HIP device is not a gfx950 (MI355X)";
    case FA_ERR_WORKSPACE: return "workspace NULL, not 256-byte aligned, too small or overlapping a tensor";
    case FA_ERR_SPLITS: return "num_splits out of range (0 for the suggestion, else 1..64)";
    case FA_ERR_STRIDE: return "invalid strides (negative, rows shorter than D, or overlapping output rows)";
    case FA_ERR_SCRATCH: return "split-KV partials exceed the fixed scratch of fa_forward_ex_noalloc (64 MiB)";
    default: return "unknown status";
  }
}

int fa_device_info(int* cus, int* max_clock_khz) {
  int dev = -1, n = 0, clk = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_DEVICE;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, dev) != hipSuccess)
    return FA_ERR_DEVICE;
  if (cus != nullptr) *cus = n;
  if (max_clock_khz != nullptr) *max_clock_khz = clk;
  return FA_OK;
}

const char* fa_version(void) { return "fa-mi355x 0.1.0 gfx950"; }

}  // extern "C"
