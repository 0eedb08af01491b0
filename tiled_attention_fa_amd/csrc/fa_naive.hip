// Naive three-pass attention: the baseline that FlashAttention is measured
// against.  "Android Transformer Optimization: Attention and Mobile GPU
// Bottlenecks", section "The Self-Attention Bottleneck Is Memory Traffic,
// Not Compute", describes it: S = Q K^T is written out whole, read back for
// the row softmax that writes P, and P is read back for O = P V; "Flash
// Attention on Android: tiled SGEMM with RenderScript", section "The
// bottleneck most engineers misdiagnose", makes the same point with the
// n x n matrix's round trips.  Here the three passes are three kernels, the
// products on the matrix cores, with S (fp32) and P (the storage type; for
// bf16 a rounded value and its rounded remainder) in a workspace the caller
// provides, both with a row pitch of NP = N rounded up to 64:
//
//   scores:  S[i][j] = scale * q_i . k_j
//   softmax: P[i][j] = exp(S[i][j] - m_i) / l_i
//   pv:      O[i] = sum_j P[i][j] v_j
//
// Each pass is built to stream its bytes at the memory's rate (the traffic
// of S and P is what the comparison is about, so it should not be inflated
// by avoidable inefficiency):
//  * scores: a workgroup of 4 waves owns 128 query rows; 64-key tiles of K
//    go to LDS (direct loads, two slots) and are shared by the 4 waves;
//    each 32 x 32 block C = Q K^T (lane = key) is stored as 32 consecutive
//    keys of two rows per instruction.
//  * softmax: one wave per row, the row held in registers (16-byte loads),
//    so S is read once; the maximum and the sum are wave reductions.  Rows
//    longer than the registers hold are read twice (online max and sum,
//    then the normalised write).  Within each group of 16 keys P is stored
//    in the order the P V pass's operand wants, keys 0-3, 8-11, 4-7, 12-15,
//    so that a lane's 8 keys are 16 contiguous bytes.
//  * pv: a workgroup of 4 waves owns 128 query rows; per 64-key tile the
//    P rows (128 x 128 bytes) and the V rows go to LDS by direct loads (two
//    slots); O^T += V^T P^T on the matrix cores with the transposed V
//    reads of the fused kernel.
//
// Causal: the scores pass stops at each wave's diagonal block, the softmax
// pass writes zeros from key i+1 to the end of row i's 64-key block, and
// the P V pass stops at each wave's diagonal tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"
#include "fa_mfma.h"

namespace fa {
namespace naive {

using mfma::f32x16;
using mfma::Ops;
using mfma::u32x2;
using mfma::u32x4;

constexpr int kRows = 128;  // query rows per workgroup of the scores and P V passes
constexpr int kBN = 64;     // keys per tile
constexpr int kNT = 256;    // threads per workgroup (4 waves)
constexpr int kSoftmaxChunks = 32;  // most 16-byte chunks per lane held in registers
constexpr int kSoftmaxRegRow = 256 * kSoftmaxChunks;  // longest row read once (8192)
constexpr int64_t kSoftmaxMaxWgs = 1 << 20;  // softmax grid cap (its waves stride over the rows)
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* s;       // [BH, N, NP] scores
  uint16_t* p;    // [BH, N, NP] probabilities (the rounded value when split)
  uint16_t* plo;  // [BH, N, NP] rounded remainders of split probabilities
  int N;
  int NP;
  int num_qtiles;
  int total_tiles;
  float scale;
};

// Direct global -> LDS load of 16 bytes per lane through a buffer resource
// (offsets at or past `bytes` read as zero).
__device__ __forceinline__ void dma16(const void* base, int bytes, uint32_t off, uint16_t* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
#endif
}

// Pass 1: S = scale * Q K^T.  The MFMA takes Q as the A operand (lane = query
// row, 8 consecutive columns) and K as the B operand (lane = key), so the
// 32 x 32 result has lane = key and element e = query row 8*(e/4) + 4*hi +
// e%4 of the block.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kNT) void scores_kernel(Args a) {
  constexpr int BN = kBN, NT = kNT;
  constexpr int DP = D <= 64 ? 64 : 128, CPR = DP / 8, DC = D / 16, TILE = BN * DP;
  constexpr int LOADS = BN * CPR / NT;
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[TILE], k1s[TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, a.total_tiles);
  const int bh = logical / a.num_qtiles;
  const int qt = logical - bh * a.num_qtiles;
  const int N = a.N, NP = a.NP;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Q = a.q + head;
  [[maybe_unused]] const uint16_t* K = a.k + head;
  float* S = a.s + (size_t)bh * N * NP;
  const int q0 = qt * kRows + wave * 32;
  const int qrow = q0 + l32;

  u32x4 qf[DC];
#pragma unroll
  for (int ch = 0; ch < DC; ++ch) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qrow < N) x = *(const u32x4*)(Q + (size_t)qrow * D + 16 * ch + 8 * hi);
    qf[ch] = x;
  }

  const int kv_end = CAUSAL ? min(N, qt * kRows + kRows) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int nt_w = q0 >= N ? 0 : CAUSAL ? min(ntiles, q0 / BN + 1) : ntiles;

  uint32_t koff[LOADS];
  bool kpred[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = i * NT + tid;
    const int row = p / CPR, pc = p % CPR;
    koff[i] = (row * D + 8 * (pc ^ mfma::k_swz<DP>(row))) * 2;
    kpred[i] = DP == D || (pc ^ mfma::k_swz<DP>(row)) < D / 8;
  }
  auto tile_load = [&](int t, uint16_t* dst) {
    const int k0 = t * BN;
    const int bytes = (int)((uint32_t)(N - k0) * (uint32_t)(2 * D));  // < 2^32; rows past N read 0
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      if (kpred[i]) dma16(K + (size_t)k0 * D, bytes, koff[i], dst + (size_t)(i * NT + wave * 64) * 8);
  };
  auto body = [&](int t, const uint16_t* kt) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kblk = t * BN + 32 * kb;
      if (CAUSAL && kblk > q0 + 31) continue;  // wave-uniform: past the diagonal
      f32x16 c = {};
      const int row = 32 * kb + l32;
#pragma unroll
      for (int ch = 0; ch < DC; ++ch) {
        const int pc = (2 * ch + hi) ^ mfma::k_swz<DP>(row);
        const u32x4 kf = *(const u32x4*)(kt + row * DP + 8 * pc);
        c = Ops<T>::mma(qf[ch], kf, c);
      }
      const int key = kblk + l32;
      if (key < N) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = q0 + 8 * (e >> 2) + 4 * hi + (e & 3);
          if (r < N) S[(size_t)r * NP + key] = c[e] * a.scale;
        }
      }
    }
  };

  tile_load(0, k0s);
  for (int t = 0; t < ntiles; t += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (t + 1 < ntiles) tile_load(t + 1, k1s);
    if (t < nt_w) body(t, k0s);
    if (t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (t + 2 < ntiles) tile_load(t + 2, k0s);
      if (t + 1 < nt_w) body(t + 1, k1s);
    }
  }
}

// Pass 2.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Element offset, within its row, of the 4 probabilities of keys j..j+3
// (j % 4 == 0): groups of 4 keys 1 and 2 of every 16 trade places.
__device__ __forceinline__ int p_pos(int j) {
  const int g = (j >> 2) & 3;
  return (j & ~15) | ((((g & 1) << 1) | (g >> 1)) << 2);
}

template <typename T, bool SPLIT>
__device__ __forceinline__ void store_p4(const Args& a, int64_t row, int j, float p0, float p1, float p2, float p3) {
  const size_t at = (size_t)row * a.NP + p_pos(j);
  const uint32_t w0 = Ops<T>::pack(p0, p1), w1 = Ops<T>::pack(p2, p3);
  *(u32x2*)(a.p + at) = u32x2{w0, w1};
  if constexpr (SPLIT) {
    const uint32_t r0 = Ops<T>::pack(p0 - Ops<T>::lo_to_f32(w0), p1 - Ops<T>::hi_to_f32(w0));
    const uint32_t r1 = Ops<T>::pack(p2 - Ops<T>::lo_to_f32(w1), p3 - Ops<T>::hi_to_f32(w1));
    *(u32x2*)(a.plo + at) = u32x2{r0, r1};
  }
}

// Rows of up to 256 * R keys: lane `lane` holds keys 4*(64*c + lane) .. +3
// for chunk c; keys past the visible end are -inf.  Every lane loads every
// chunk, from an address clamped to the row's last visible chunk (so past
// the end the loads repeat one cached line instead of branching).
template <typename T, bool SPLIT, bool CAUSAL, int R>
__global__ __launch_bounds__(256) void softmax_kernel(Args a, int64_t rows) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int N = a.N, NP = a.NP;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4) {
    const int i = (int)(row % N);
    const int n_vis = CAUSAL ? i + 1 : N;
    const int n_out = CAUSAL ? min(NP, (i / 64 + 1) * 64) : NP;
    const int j_last = (n_vis - 1) & ~3;
    const float* Srow = a.s + (size_t)row * NP;
    f32x4 x[R];
#pragma unroll
    for (int c = 0; c < R; ++c) x[c] = *(const f32x4*)(Srow + min(4 * (64 * c + lane), j_last));
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int j = 4 * (64 * c + lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[c][e] = j + e < n_vis ? x[c][e] : -INFINITY;
      m = fmaxf(m, fmaxf(fmaxf(x[c][0], x[c][1]), fmaxf(x[c][2], x[c][3])));
    }
    const float M = wave_max(m);  // finite: key 0 is always visible
    const float mc = M * kLog2e;
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < R; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[c][e], kLog2e, -mc));  // exp2(-inf) = 0
        l += x[c][e];
      }
    }
    const float inv = 1.f / wave_sum(l);
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int j = 4 * (64 * c + lane);
      if (j < n_out)
        store_p4<T, SPLIT>(a, row, j, x[c][0] * inv, x[c][1] * inv, x[c][2] * inv, x[c][3] * inv);
    }
  }
}

// Rows longer than the registers hold: an online maximum and sum over the
// row, then a second read that writes the normalised row.
template <typename T, bool SPLIT, bool CAUSAL>
__global__ __launch_bounds__(256) void softmax_long_kernel(Args a, int64_t rows) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int N = a.N, NP = a.NP;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4) {
    const int i = (int)(row % N);
    const int n_vis = CAUSAL ? i + 1 : N;
    const int n_out = CAUSAL ? min(NP, (i / 64 + 1) * 64) : NP;
    const float* Srow = a.s + (size_t)row * NP;
    float m = -INFINITY, l = 0.f;
    for (int j = 4 * lane; j < n_vis; j += 256) {
      f32x4 v = *(const f32x4*)(Srow + j);
      if (j + 1 >= n_vis) v[1] = -INFINITY;
      if (j + 2 >= n_vis) v[2] = -INFINITY;
      if (j + 3 >= n_vis) v[3] = -INFINITY;
      const float mn = fmaxf(m, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));  // finite: v[0] is visible
      const float mc = mn * kLog2e;
      l = l * __builtin_amdgcn_exp2f(__builtin_fmaf(m, kLog2e, -mc));
#pragma unroll
      for (int e = 0; e < 4; ++e) l += __builtin_amdgcn_exp2f(__builtin_fmaf(v[e], kLog2e, -mc));
      m = mn;
    }
    const float M = wave_max(m);
    const float mc = M * kLog2e;
    const float L = wave_sum(m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(__builtin_fmaf(m, kLog2e, -mc)));
    const float inv = 1.f / L;
    for (int j = 4 * lane; j < n_out; j += 256) {
      f32x4 v = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (j < n_vis) v = *(const f32x4*)(Srow + j);
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p[e] = j + e < n_vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(v[e], kLog2e, -mc)) * inv : 0.f;
      store_p4<T, SPLIT>(a, row, j, p[0], p[1], p[2], p[3]);
    }
  }
}

// Pass 3.  O^T += V^T P^T: V^T from the transposed LDS reads of the fused
// kernel (lane = column of V, keys 16*kc + {4*hi..4*hi+3, 8+4*hi..+3}), P^T
// as the B operand (lane = query row): 16 contiguous bytes of the row's P
// tile in LDS, which the softmax pass stored in that same key order.  P
// tile rows are 128 bytes with the 16-byte chunks swizzled like the fused
// kernel's K rows of 64 elements.
template <typename T, int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kNT) void pv_kernel(Args a) {
  constexpr int BN = kBN, NT = kNT;
  constexpr int DP = D <= 64 ? 64 : 128, CPR = DP / 8, DB = D / 32, VTILE = BN * DP;
  constexpr int VLOADS = BN * CPR / NT;
  constexpr int PTILE = kRows * BN, PLOADS = kRows * (BN / 8) / NT;
  constexpr int LTILE = SPLIT ? PTILE : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[VTILE], v1s[VTILE];
  __shared__ __attribute__((aligned(1024))) uint16_t p0s[PTILE], p1s[PTILE];
  __shared__ __attribute__((aligned(1024))) uint16_t l0s[LTILE], l1s[LTILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, a.total_tiles);
  const int bh = logical / a.num_qtiles;
  const int qt = logical - bh * a.num_qtiles;
  const int N = a.N, NP = a.NP;
  const size_t head = (size_t)bh * N * D;
  [[maybe_unused]] const uint16_t* V = a.v + head;
  uint16_t* O = a.o + head;
  const int row0 = qt * kRows;
  [[maybe_unused]] const uint16_t* P = a.p + ((size_t)bh * N + row0) * NP;
  [[maybe_unused]] const uint16_t* PL = SPLIT ? a.plo + ((size_t)bh * N + row0) * NP : nullptr;
  const int q0 = row0 + wave * 32;
  const int qrow = q0 + l32;
  // bytes of this workgroup's P rows (at most 128 rows of NP <= 2^20 keys)
  const uint32_t p_bytes = (uint32_t)min(N - row0, kRows) * (uint32_t)NP * 2u;

  const int kv_end = CAUSAL ? min(N, row0 + kRows) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int nt_w = q0 >= N ? 0 : CAUSAL ? min(ntiles, q0 / BN + 1) : ntiles;

  uint32_t voff[VLOADS], poff[PLOADS];
  bool vpred[VLOADS];
#pragma unroll
  for (int i = 0; i < VLOADS; ++i) {
    const int p = i * NT + tid;
    const int row = p / CPR, pc = p % CPR;
    voff[i] = (row * D + 8 * (pc ^ mfma::v_swz<DP>(row))) * 2;
    vpred[i] = DP == D || (pc ^ mfma::v_swz<DP>(row)) < D / 8;
  }
#pragma unroll
  for (int i = 0; i < PLOADS; ++i) {
    const int p = i * NT + tid;
    const int row = p / 8, pc = p % 8;
    poff[i] = (uint32_t)row * (uint32_t)NP * 2u + 16u * (uint32_t)(pc ^ mfma::k_swz<64>(row));
  }
  auto tile_load = [&](int t, uint16_t* vdst, uint16_t* pdst, uint16_t* ldst) {
    const int k0 = t * BN;
    const int vbytes = (int)((uint32_t)(N - k0) * (uint32_t)(2 * D));
#pragma unroll
    for (int i = 0; i < VLOADS; ++i)
      if (vpred[i]) dma16(V + (size_t)k0 * D, vbytes, voff[i], vdst + (size_t)(i * NT + wave * 64) * 8);
    const int pb = (int)(p_bytes - 2u * (uint32_t)k0);  // rows past N read 0
#pragma unroll
    for (int i = 0; i < PLOADS; ++i) {
      dma16(P + k0, pb, poff[i], pdst + (size_t)(i * NT + wave * 64) * 8);
      if constexpr (SPLIT) dma16(PL + k0, pb, poff[i], ldst + (size_t)(i * NT + wave * 64) * 8);
    }
  };

  const int grp = lane >> 4, gl = lane & 15;
  const int tr_row = 4 * hi + (gl >> 2);
  const int tr_chunk_lo = (2 * (grp & 1) + ((gl & 3) >> 1)) ^ mfma::v_swz<DP>(tr_row);
  const int tr_byte = 8 * (gl & 1);
  const int prow = wave * 32 + l32;  // this lane's row of the P tile

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  auto body = [&](const uint16_t* vt, const uint16_t* pt, const uint16_t* lt) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int pc = (2 * kc + hi) ^ mfma::k_swz<64>(prow);
      const u32x4 pf = *(const u32x4*)(pt + prow * BN + 8 * pc);
      u32x4 pfl = {0u, 0u, 0u, 0u};
      if constexpr (SPLIT) pfl = *(const u32x4*)(lt + prow * BN + 8 * pc);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 2 * 8 * ((4 * db) ^ tr_chunk_lo) + tr_byte;
        const u32x2 v0 = mfma::tr_read((const uint16_t*)((const char*)vt + (16 * kc + tr_row) * DP * 2 + col));
        const u32x2 v1 = mfma::tr_read((const uint16_t*)((const char*)vt + (16 * kc + 8 + tr_row) * DP * 2 + col));
        const u32x4 vf = {v0[0], v0[1], v1[0], v1[1]};
        oacc[db] = Ops<T>::mma(vf, pf, oacc[db]);
        if constexpr (SPLIT) oacc[db] = Ops<T>::mma(vf, pfl, oacc[db]);
      }
    }
  };

  // Two LDS slots: at step t, tile t has landed (the barrier), the loads of
  // tile t+1 go to the other slot, then tile t is used.
  tile_load(0, v0s, p0s, l0s);
  for (int t = 0; t < ntiles; t += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (t + 1 < ntiles) tile_load(t + 1, v1s, p1s, l1s);
    if (t < nt_w) body(v0s, p0s, l0s);
    if (t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (t + 2 < ntiles) tile_load(t + 2, v0s, p0s, l0s);
      if (t + 1 < nt_w) body(v1s, p1s, l1s);
    }
  }

  if (qrow < N) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hi;
        const u32x2 out = {Ops<T>::pack(oacc[db][4 * g], oacc[db][4 * g + 1]),
                           Ops<T>::pack(oacc[db][4 * g + 2], oacc[db][4 * g + 3])};
        *(u32x2*)(O + (size_t)qrow * D + d0) = out;
      }
  }
}

template <typename T, bool SPLIT, int D, bool CAUSAL>
hipError_t run(const Args& a, int64_t BH, hipStream_t stream) {
  Args x = a;
  void* args[] = {&x};
  const int wgs = a.total_tiles;
  hipError_t e = hipLaunchKernel((const void*)scores_kernel<T, D, CAUSAL>, dim3(wgs), dim3(kNT), args, 0, stream);
  if (e != hipSuccess) return e;
  int64_t rows = BH * a.N;
  void* args2[] = {&x, &rows};
  const int64_t sm_wgs = (rows + 3) / 4 < kSoftmaxMaxWgs ? (rows + 3) / 4 : kSoftmaxMaxWgs;
  // rows held in registers when they fit (chunks of 256 keys per wave)
  const void* sm = a.N <= 512    ? (const void*)softmax_kernel<T, SPLIT, CAUSAL, 2>
                   : a.N <= 2048 ? (const void*)softmax_kernel<T, SPLIT, CAUSAL, 8>
                   : a.N <= 4096 ? (const void*)softmax_kernel<T, SPLIT, CAUSAL, 16>
                   : a.N <= kSoftmaxRegRow ? (const void*)softmax_kernel<T, SPLIT, CAUSAL, kSoftmaxChunks>
                                           : (const void*)softmax_long_kernel<T, SPLIT, CAUSAL>;
  e = hipLaunchKernel(sm, dim3((unsigned)sm_wgs), dim3(256), args2, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)pv_kernel<T, D, CAUSAL, SPLIT>, dim3(wgs), dim3(kNT), args, 0, stream);
}

template <typename T, bool SPLIT>
hipError_t launch(const NaiveProblem& p, hipStream_t stream) {
  Args a;
  a.q = (const uint16_t*)p.q;
  a.k = (const uint16_t*)p.k;
  a.v = (const uint16_t*)p.v;
  a.o = (uint16_t*)p.o;
  a.s = (float*)p.s;
  a.p = (uint16_t*)p.p;
  a.plo = (uint16_t*)p.plo;
  a.N = p.N;
  a.NP = p.NP;
  a.num_qtiles = (p.N + kRows - 1) / kRows;
  a.total_tiles = (int)(p.BH * a.num_qtiles);
  a.scale = p.scale;
  switch (p.D) {
    case 64: return p.causal ? run<T, SPLIT, 64, true>(a, p.BH, stream) : run<T, SPLIT, 64, false>(a, p.BH, stream);
    case 96: return p.causal ? run<T, SPLIT, 96, true>(a, p.BH, stream) : run<T, SPLIT, 96, false>(a, p.BH, stream);
    case 128:
      return p.causal ? run<T, SPLIT, 128, true>(a, p.BH, stream) : run<T, SPLIT, 128, false>(a, p.BH, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace naive

hipError_t launch_naive_f16(const NaiveProblem& p, hipStream_t stream) {
  return naive::launch<_Float16, false>(p, stream);
}
hipError_t launch_naive_bf16(const NaiveProblem& p, hipStream_t stream) {
  return naive::launch<__bf16, true>(p, stream);
}

}  // namespace fa
