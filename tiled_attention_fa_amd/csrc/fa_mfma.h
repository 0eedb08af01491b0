// FlashAttention forward for 16-bit storage (fp16, bf16) on gfx950 matrix
// cores.
//
// The method is the tile loop of "Android Transformer Optimization: Attention
// and Mobile GPU Bottlenecks" (sections "The Essence of FlashAttention:
// Reordering the Computation" and "A Complete Tile Loop"): one workgroup owns
// a block of query rows and walks over all key/value tiles in an inner loop;
// per tile it forms the score tile on chip, raises the running row maximum m,
// rescales the running denominator l and the output accumulator by
// exp(m_old - m_new), adds the tile's exp(S - m_new) to l and exp(S - m_new) V
// to the accumulator, and at the end divides the accumulator by l once.
//
// gfx950 mapping (not from the pages, which target mobile GPUs):
//  * A workgroup is 4 wave64s and owns kBlockM = 128 query rows of one
//    (batch, head); each wave owns 32 of them.  Its Q rows are loaded once
//    into VGPRs, as the B operand of v_mfma_f32_32x32x16_{f16,bf16}.
//  * Per iteration a 64-key tile of K is staged in LDS row-major and the
//    matching V tile is staged transposed (V^T, keys contiguous), both with
//    16-byte row padding so that the ds_read_b128 operand reads of 8
//    consecutive lanes hit 8 distinct 4-bank groups.
//  * Scores are computed transposed, S^T = K Q^T, so each lane holds 16
//    keys x 1 query per 32-key block: row max and row sum are in-lane,
//    plus one exchange between the two 32-lane halves.
//  * The exp'd scores are converted to 16 bits in registers and fed back as
//    the B operand of O^T += V^T P^T.  The accumulator layout puts, for lane
//    half h, keys {4h..4h+3, 8+4h..8+4h+3} of each 16-key chunk in
//    consecutive elements; V^T is stored with the second and third 4-key
//    groups of every 16 keys swapped so that each lane's A operand is one
//    contiguous 16-byte read with the same key order.
//  * Softmax runs in base 2: p = exp2(s * c - m * c) with c = |scale| *
//    log2(e) folded into one FMA; a negative scale flips the sign of Q.
//  * bf16 keeps P as an unevaluated sum of two bf16 numbers (hi + lo) and
//    issues two PV products, so P carries ~16 significant bits, as fp16 does
//    with one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace mfma {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockM = kMfmaBlockM;  // query rows per workgroup
constexpr int kWaveM = 32;            // query rows per wave
constexpr int kWaves = kBlockM / kWaveM;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockN = 64;           // keys per iteration
constexpr int kPad = 8;               // 16-byte LDS row padding (in 16-bit elements)
constexpr int kXcds = 8;              // MI355X: 8 accelerator complex dies
static_assert(kWaves == 4, "4 waves per workgroup");

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int N;
  int num_qtiles;   // ceil(N / kBlockM)
  int total_tiles;  // BH * num_qtiles
  float c;          // |scale| * log2(e)
  uint32_t qxor;    // 0x80008000 flips the sign of both halves when scale < 0
};

template <typename T>
struct Ops;

template <>
struct Ops<_Float16> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // Two fp32 values -> packed 16-bit pair, round to nearest even.
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo_to_f32(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2, w)[0];
  }
  static __device__ __forceinline__ float hi_to_f32(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2, w)[1];
  }
};

template <>
struct Ops<__bf16> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo_to_f32(uint32_t w) {
    return __builtin_bit_cast(float, w << 16);
  }
  static __device__ __forceinline__ float hi_to_f32(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
  }
};

// Workgroup id -> logical tile id.  Workgroups are dispatched round-robin
// over the 8 XCDs (id % 8), each with its own L2; this gives every XCD a
// contiguous range of logical tiles, so the query tiles of one head, which
// all read that head's K and V, run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int per = total / kXcds, extra = total % kXcds;
  const int x = wg % kXcds, slot = wg / kXcds;
  return x * per + (x < extra ? x : extra) + slot;
}

// Both 32-lane halves combined with a symmetric op: after the swap each lane
// holds its own value and its partner's (lane ^ 32), in some order.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Position of key group g (4 keys) inside its 16-key chunk of V^T: groups 1
// and 2 trade places (see the header comment).
__device__ __forceinline__ int vt_group(int g) { return (g == 1 || g == 2) ? 3 - g : g; }

template <typename T, int D, bool CAUSAL, bool SPLIT_P>
__global__ __launch_bounds__(kThreads, 2) void fa_forward_kernel(Args a) {
  constexpr int BN = kBlockN;
  constexpr int KS = D + kPad;   // K row stride in LDS (elements)
  constexpr int VS = BN + kPad;  // V^T row stride in LDS (elements)
  constexpr int DC = D / 16;     // 16-wide contraction chunks of QK^T
  constexpr int DB = D / 32;     // 32-row blocks of O^T
  static_assert(D % 32 == 0 && D <= 128, "head dim");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, a.total_tiles);
  const int bh = logical / a.num_qtiles;
  int qt = logical - bh * a.num_qtiles;
  if (CAUSAL) qt = a.num_qtiles - 1 - qt;  // longest rows first
  const int N = a.N;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Q = a.q + head;
  const uint16_t* __restrict__ K = a.k + head;
  const uint16_t* __restrict__ V = a.v + head;
  uint16_t* __restrict__ O = a.o + head;
  const float c = a.c;

  const int q0 = qt * kBlockM + wave * kWaveM;  // first query row of this wave
  const int qrow = q0 + l32;                    // this lane's query row

  // Q fragment: row qrow, columns 16*ch + 8*hi .. +7 (B operand layout).
  u32x4 qf[DC];
#pragma unroll
  for (int ch = 0; ch < DC; ++ch) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qrow < N) x = *(const u32x4*)(Q + (size_t)qrow * D + 16 * ch + 8 * hi);
    qf[ch] = x ^ a.qxor;
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // running max of raw scores q.k (sign-adjusted)
  float l_run = 0.f;        // this lane's share of the running denominator

  const int kv_end = CAUSAL ? min(N, qt * kBlockM + kBlockM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;

  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();  // previous tile's LDS reads are done

    // K tile -> LDS, row-major, 16-byte chunks; rows >= N are zero.
    constexpr int KCH = BN * D / 8;
#pragma unroll
    for (int idx = tid; idx < KCH; idx += kThreads) {
      const int r = idx / (D / 8), c8 = idx - r * (D / 8);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (k0 + r < N) x = *(const u32x4*)(K + (size_t)(k0 + r) * D + 8 * c8);
      *(u32x4*)(Ks + r * KS + 8 * c8) = x;
    }
    // V tile -> LDS transposed: each thread moves a 4-key x 4-column block.
    constexpr int VBL = (BN / 4) * (D / 4);
#pragma unroll
    for (int idx = tid; idx < VBL; idx += kThreads) {
      const int dg = idx % (D / 4), kg = idx / (D / 4);
      u32x2 rw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * kg + r;
        u32x2 x = {0u, 0u};
        if (key < N) x = *(const u32x2*)(V + (size_t)key * D + 4 * dg);
        rw[r] = x;
      }
      const int pos = 16 * (kg >> 2) + 4 * vt_group(kg & 3);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int w = cc >> 1, sh = (cc & 1) * 16;
        const uint32_t e0 = (rw[0][w] >> sh) & 0xffffu, e1 = (rw[1][w] >> sh) & 0xffffu;
        const uint32_t e2 = (rw[2][w] >> sh) & 0xffffu, e3 = (rw[3][w] >> sh) & 0xffffu;
        u32x2 out = {e0 | (e1 << 16), e2 | (e3 << 16)};
        *(u32x2*)(Vt + (4 * dg + cc) * VS + pos) = out;
      }
    }
    __syncthreads();

    // S^T = K Q^T for two 32-key blocks.  s[kb][e] is the score of key
    // k0 + 32*kb + 8*(e/4) + 4*hi + (e%4) against query qrow.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ch = 0; ch < DC; ++ch) {
        const u32x4 kf = *(const u32x4*)(Ks + (32 * kb + l32) * KS + 16 * ch + 8 * hi);
        s[kb] = Ops<T>::mma(kf, qf[ch], s[kb]);
      }
    }

    const bool edge = (k0 + BN > N) || (CAUSAL && (k0 + BN - 1 > q0));
    if (edge) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * hi + (e & 3);
          if (key >= N || (CAUSAL && key > qrow)) s[kb][e] = -INFINITY;
        }
    }

    // Online softmax update (base 2).
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    mx = half_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run * c - mc);
    m_run = m_new;

    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], c, -mc));
        if (edge && s[kb][e] == -INFINITY) p = 0.f;  // also right when c == 0
        s[kb][e] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

    // O^T += V^T P^T, one 16-key chunk at a time.
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kb = kc >> 1, base = 8 * (kc & 1);
      u32x4 pf, pl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = s[kb][base + 2 * j], p1 = s[kb][base + 2 * j + 1];
        pf[j] = Ops<T>::pack(p0, p1);
        if (SPLIT_P)
          pl[j] = Ops<T>::pack(p0 - Ops<T>::lo_to_f32(pf[j]), p1 - Ops<T>::hi_to_f32(pf[j]));
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4 vf = *(const u32x4*)(Vt + (32 * db + l32) * VS + 16 * kc + 8 * hi);
        oacc[db] = Ops<T>::mma(vf, pf, oacc[db]);
        if (SPLIT_P) oacc[db] = Ops<T>::mma(vf, pl, oacc[db]);
      }
    }
  }

  // Epilogue: divide by the row's denominator once, round, store.
  const float l = half_sum(l_run);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (qrow < N) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // elements 4g..4g+3 are columns d0..d0+3 of row qrow
        const int d0 = 32 * db + 8 * g + 4 * hi;
        u32x2 out = {Ops<T>::pack(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                     Ops<T>::pack(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *(u32x2*)(O + (size_t)qrow * D + d0) = out;
      }
  }
}

template <typename T, bool SPLIT_P>
hipError_t launch(const Problem& p, hipStream_t stream) {
  Args a;
  a.q = (const uint16_t*)p.q;
  a.k = (const uint16_t*)p.k;
  a.v = (const uint16_t*)p.v;
  a.o = (uint16_t*)p.o;
  a.N = p.N;
  a.num_qtiles = (p.N + kBlockM - 1) / kBlockM;
  a.total_tiles = (int)(p.BH * a.num_qtiles);
  a.c = __builtin_fabsf(p.scale) * 1.4426950408889634f;
  a.qxor = p.scale < 0.f ? 0x80008000u : 0u;
  void (*kern)(Args) = nullptr;
#define FA_PICK(DD)                                                                   \
  if (p.D == DD)                                                                      \
    kern = p.causal ? fa_forward_kernel<T, DD, true, SPLIT_P> : fa_forward_kernel<T, DD, false, SPLIT_P>;
  FA_PICK(64)
  FA_PICK(96)
  FA_PICK(128)
#undef FA_PICK
  if (!kern) return hipErrorInvalidValue;
  void* args[] = {&a};
  return hipLaunchKernel((const void*)kern, dim3(a.total_tiles), dim3(kThreads), args, 0, stream);
}

}  // namespace mfma
}  // namespace fa
