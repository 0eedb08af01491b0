// Internal interface between the C ABI (fa_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Where element (b, h, n, d) of a tensor sits: b*sb + h*sh + n*sn + d
// elements from its base (d contiguous).
struct Layout {
  int64_t sb;
  int64_t sh;
  int sn;
};

// Dense [B, H, N, D].
inline Layout dense_layout(int64_t H, int64_t N, int64_t D) { return Layout{H * N * D, N * D, (int)D}; }

// One validated forward problem.  Query heads bh = b*H + h, h < H; query
// head h reads key/value head h / group (group = H / H_kv).
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t BH;
  int N;
  int D;
  float scale;
  bool causal;
  int H = 1;
  int group = 1;
  Layout lq{}, lk{}, lv{}, lo{};
  // Key-range split (split-KV): with splits > 1 each query block's key
  // tiles are cut into `splits` ranges, one workgroup each, and the kernel
  // writes normalised fp32 partials part_o [splits, BH, N, D] and their
  // log-sum-exp part_lse [splits, BH, N] for the merge kernel instead of o.
  int splits = 1;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  // Optional [BH, N] log-sum-exp of each row's scaled scores (splits == 1;
  // with splits > 1 the merge kernel writes it).
  float* lse = nullptr;
  // Key groups per workgroup (1, 2 or 4; more than one only with
  // splits == 1): the wave groups share the query rows of a workgroup and
  // take alternate key tiles, merged in LDS at the end.  16-bit kernel:
  // ks_waves is that workgroup's wave count (4, or 8 for D = 96 and 128).
  // fp32 kernel: f32_row_waves waves of 16 rows per group (4, 2 or 1).
  int key_groups = 1;
  int ks_waves = 4;
  int f32_row_waves = 4;
  // One key group and one key range: the host may replace the table's
  // workgroup shape (mfma_waves, mfma_block_n) for causal grids with
  // waves1 waves (2 or 4 at D = 128, 8 at D = 64; 0 elsewhere) and block_n1
  // keys per LDS tile (32); 0 keeps the table's choice.
  int waves1 = 0;
  int block_n1 = 0;
};

// Merge of split-KV partials: O = sum_s exp(lse_s - lse) O_s with
// lse = ln sum_s exp(lse_s), O in the storage type (dtype as in fa.h).
struct MergeProblem {
  const float* part_o;
  const float* part_lse;
  void* o;
  float* lse;  // optional
  int64_t rows;  // BH * N
  int D;
  int splits;
  int dtype;
};

// Workgroup shape of the matrix-core kernel per head dimension and mask:
// waves per workgroup (32 query rows each) and workgroups resident per CU,
// the fastest of the calibration sweep (tiled_attention_fa_amd/tile_sweep.py,
// every shape of the tuning build timed on MI355X for each D, storage type
// and mask).  Eight waves (256 rows, two waves per SIMD in lockstep) where
// rows are long and uniform; four waves for causal D = 64, where the finer
// grain balances the triangle better (two workgroups per CU), and for D = 96
// (one wave per SIMD: 128-element LDS rows leave room for one workgroup per
// CU).
constexpr int mfma_waves(int D, bool causal) { return D == 96 || (D == 64 && causal) ? 4 : 8; }
// Keys per LDS tile of the one-group kernel, from the same sweep over 32, 64
// and 128: 64, except bf16 at D = 128 (split P), where the 64-key build of
// the kernel needs a few more registers than it has.  128-key tiles come
// within 1% at best.  (For causal grids the host names 32-key tiles in
// more cases: Problem::block_n1.)
constexpr int mfma_block_n(int D, bool split_p) { return D == 128 && split_p ? 32 : 64; }
constexpr int mfma_wgs_per_cu(int D, bool causal) { return D == 64 && causal ? 2 : 1; }
// With two key groups: 4 waves (2 row blocks of 32 x 2 groups, 64 rows per
// workgroup), two workgroups per CU where the LDS allows it (D = 64); or, on
// grids that would need more than one pass of those over the CUs, 8 waves (128 rows).
constexpr int mfma_ks_waves = 4;
constexpr int mfma_ks_occupancy(int D) { return D == 64 ? 2 : 1; }

// One validated three-pass problem: the forward problem plus the caller's
// workspace, cut into the fp32 score matrix S [BH, N, N] and the
// probabilities P [BH, N, NP] (NP = N rounded up to 64; for bf16 a second
// array of the low parts).
struct NaiveProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  void* s;
  void* p;
  void* plo;
  int64_t BH;
  int N;
  int NP;
  int D;
  float scale;
  bool causal;
};

// Query rows per workgroup of each kernel family that the host bounds grid
// sizes with (larger blocks only mean fewer workgroups).  The matrix-core
// kernel's smallest block with one key group is 128 rows; its two-key-group
// shape (64 rows) is chosen only for grids smaller than the device's
// workgroup slots, far below these bounds.  Likewise the fp32 kernel's 16-
// and 32-row shapes serve only grids smaller than the device's SIMDs.
constexpr int kMfmaBlockM = 128;
constexpr int kF32BlockM = 64;

// Kernel launchers.  Each returns the launch status and touches nothing
// else.  D must be 64, 96 or 128 and N >= 1 (checked by the caller).
hipError_t launch_mfma_f16(const Problem& p, hipStream_t stream);
hipError_t launch_mfma_bf16(const Problem& p, hipStream_t stream);
hipError_t launch_f32(const Problem& p, hipStream_t stream);
hipError_t launch_split_merge(const MergeProblem& p, hipStream_t stream);
#ifdef FA_TILE_SWEEP
// The calibration sweep's shapes (tuning library only): (waves per
// workgroup, waves_per_eu hint, key groups, keys per LDS tile).
constexpr int kTuneShapes64[][4] = {{2, 1, 1, 64},  {4, 1, 1, 64},  {4, 2, 1, 64},  {8, 1, 1, 64},
                                    {4, 1, 2, 64},  {4, 2, 2, 64},  {8, 1, 2, 64},  {2, 1, 1, 32},
                                    {4, 1, 1, 32},  {4, 2, 1, 32},  {8, 1, 1, 32},  {2, 1, 1, 128},
                                    {4, 1, 1, 128}, {8, 1, 1, 128}, {8, 1, 4, 32}};
constexpr int kTuneShapesWide[][4] = {{2, 1, 1, 64}, {4, 1, 1, 64}, {8, 1, 1, 64}, {4, 1, 2, 64},
                                      {8, 1, 2, 64}, {2, 1, 1, 32}, {4, 1, 1, 32}, {8, 1, 1, 32},
                                      {8, 1, 4, 32}};
constexpr int kTuneShapes64Count = 15, kTuneShapesWideCount = 9;
hipError_t launch_mfma_shape_f16(const Problem& p, int waves, int occupancy, int key_groups, int block_n,
                                  hipStream_t stream);
hipError_t launch_mfma_shape_bf16(const Problem& p, int waves, int occupancy, int key_groups, int block_n,
                                   hipStream_t stream);
// The fp32 kernel's shapes: (waves of 16 query rows per key group, key
// groups taking alternate tiles), the same for every head dim.
constexpr int kTuneF32Shapes[][2] = {{4, 1}, {4, 2}, {2, 2}, {2, 4}, {1, 4}};
constexpr int kTuneF32ShapesCount = 5;
hipError_t launch_f32_shape(const Problem& p, int row_waves, int key_groups, hipStream_t stream);
#endif
hipError_t launch_naive_f16(const NaiveProblem& p, hipStream_t stream);
hipError_t launch_naive_bf16(const NaiveProblem& p, hipStream_t stream);

// Workgroup placement shared by the kernels.  MI355X has 8 accelerator
// complex dies (XCDs), each with its own L2; the dispatcher deals
// workgroups round-robin over them (workgroup id % 8).  Both functions are
// plain integer arithmetic, callable on the host as well, where a test
// checks them over whole grids.
constexpr int kXcds = 8;

// Workgroup id -> logical tile id.  Workgroups are dispatched round-robin
// over the 8 XCDs (id % 8), each with its own L2; this gives every XCD a
// contiguous range of logical tiles, so the query tiles of one head, which
// all read that head's K and V, run on the same XCD and share its L2.
__host__ __device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int per = total / kXcds, extra = total % kXcds;
  const int x = wg % kXcds, slot = wg / kXcds;
  return x * per + (x < extra ? x : extra) + slot;
}

// Causal launches: the query blocks of one XCD's share (a contiguous range
// of head-major tile ids, as xcd_remap hands them out) in order of row
// length, longest first across every head of the range, instead of head by
// head.  The dispatcher starts workgroups in order as slots free up, so this
// is longest-processing-time-first list scheduling: the short blocks fill
// the slots at the end of the launch instead of the last heads' long ones
// running alone.  Each XCD keeps the same heads, and so its L2 the same K/V.
// Returns the head-major tile id h * nq + r, where rank r = 0 is a head's
// longest rows.
__host__ __device__ __forceinline__ int causal_lpt(int wg, int total, int nq) {
  const int per = total / kXcds, extra = total % kXcds;
  const int x = wg % kXcds, s = wg / kXcds;
  const int lo = x * per + (x < extra ? x : extra);
  const int last = lo + per - (x < extra ? 0 : 1);
  const int hA = lo / nq, rA = lo - hA * nq;  // first head, its first rank in the range
  const int hB = last / nq, rB = last - hB * nq;
  if (hA == hB) return lo + s;
  const int full = hB - hA - 1;  // heads with all their ranks in the range
  // tiles of the range with rank below r
  auto before = [&](int r) { return full * r + (r > rA ? r - rA : 0) + (r < rB + 1 ? r : rB + 1); };
  int r0 = 0, r1 = nq - 1;  // the largest r with before(r) <= s
  while (r0 < r1) {
    const int m = (r0 + r1 + 1) >> 1;
    if (before(m) <= s) r0 = m;
    else r1 = m - 1;
  }
  int j = s - before(r0);  // position among the tiles of rank r0: head hA, full heads, head hB
  if (r0 >= rA) {
    if (j == 0) return hA * nq + r0;
    --j;
  }
  return (j < full ? hA + 1 + j : hB) * nq + r0;
}

}  // namespace fa
