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
// gfx950 mapping (the pages target mobile GPUs; none of this is from them):
//  * A workgroup is NW wave64s and owns BM = NW * WM query rows of one
//    (batch, head); each wave owns WM (32 or 64) of them, in WM/32 column
//    blocks.  A wave's Q rows are loaded once into VGPRs as the B operand of
//    v_mfma_f32_32x32x16_{f16,bf16}.
//  * K and V tiles of 64 keys are loaded with 16-byte coalesced loads into
//    registers one iteration ahead (the loads of tile t+1 are in flight while
//    tile t is computed) and stored row-major into a double-buffered LDS
//    area, so one barrier per tile suffices.
//  * Scores are computed transposed, S^T = K Q^T: each lane holds 16 keys of
//    one query per 32-key block, so row max and row sum are in-lane plus one
//    exchange between the two 32-lane halves (v_permlane32_swap).
//  * P^T goes from the score accumulators straight into the B operand of
//    O^T += V^T P^T (converted to 16 bits in registers).  The V^T A operand
//    is read from the row-major V tile with ds_read_b64_tr_b16, whose
//    16-lane transpose hands each lane 4 keys of one head-dim column; the
//    source addresses are chosen so that lane half h gets keys
//    {4h..4h+3, 8+4h..8+4h+3} of each 16-key chunk, the key order in which
//    the score accumulator layout holds P.
//  * LDS rows are padded (K by 16 bytes, V by 32 bytes) so that the 16-byte
//    operand reads of K and the 8-byte transpose reads of V hit distinct
//    banks within each group of lanes the LDS serves together.
//  * Softmax runs in base 2: p = exp2(s * c - m * c) with c = |scale| *
//    log2(e) in one FMA; a negative scale flips the sign of Q.  The running
//    maximum is only raised when a tile's maximum exceeds it by more than
//    kLazy (in log2 units): otherwise the old maximum stays and the tile's p
//    values may reach 2^kLazy, which fp32 accumulators and 16-bit P hold
//    without loss; the rescale of O is then skipped for the whole wave.
//    The result is the same softmax, exp(s - m) / sum exp(s - m), for any
//    choice of m.
//  * fp16: P is rounded once to fp16, and l sums exactly those rounded
//    values (v_dot2_f32_f16 against 1.0), so the weights applied to V sum to
//    one.  bf16: P is kept as an unevaluated sum of two bf16 numbers
//    (hi + lo) and two PV products are issued, so P carries ~16 significant
//    bits, as with fp16; l sums the fp32 p.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kBlockN = 64;  // keys per iteration
constexpr int kXcds = 8;     // MI355X: 8 accelerator complex dies, one L2 each
constexpr float kLazy = 8.f;  // log2 of the largest p the lazy maximum allows

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int N;
  int num_qtiles;   // ceil(N / BM)
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
  // acc + w.lo + w.hi, exact products with 1.0 and fp32 accumulation.
  static __device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
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

// Combine both 32-lane halves with a symmetric op: after the swap each lane
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

__device__ __forceinline__ u32x2 tr_read(const uint16_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_u16*)p);
  return __builtin_bit_cast(u32x2, r);
}

template <int D, int WM, int NW, int KSPLIT>
struct Shape {
  static constexpr int BN = kBlockN;
  static constexpr int NQW = NW / KSPLIT;  // waves per key group
  static constexpr int BM = WM * NQW;    // query rows per workgroup
  static constexpr int QB = WM / 32;     // 32-query column blocks per wave
  static constexpr int NT = 64 * NW;     // threads per workgroup
  static constexpr int DP = D <= 64 ? 64 : 128;  // LDS row length (elements)
  static constexpr int CPR = DP / 8;     // 16-byte chunks per LDS row
  static constexpr int DC = D / 16;      // 16-wide contraction chunks of QK^T
  static constexpr int DB = D / 32;      // 32-row blocks of O^T
  static constexpr int TILE = BN * DP;   // elements per LDS tile buffer
  static constexpr int LOADS = KSPLIT * BN * CPR / NT;  // 16-byte loads per thread per step
  static_assert(D % 32 == 0 && D <= 128, "head dim");
  static_assert(WM == 32 || WM == 64, "queries per wave");
  static_assert((KSPLIT * BN * CPR) % NT == 0, "whole wave-loads per step");
  static_assert(KSPLIT == 1 || KSPLIT == 2, "key groups");
};

// LDS tile layouts.  A tile row (one key) is DP elements = CPR chunks of 16
// bytes, rows back to back (the direct global->LDS loads write each wave's
// 64 x 16 bytes contiguously, so rows cannot be padded).  Chunks are
// permuted within a row by an XOR with a function of the row:
//  * K (read by ds_read_b128, 8 consecutive rows per LDS cycle at one
//    logical chunk): physical chunk = chunk ^ (row & 7).
//  * V (read by ds_read_b64_tr_b16, 4 consecutive rows x 2 adjacent chunks
//    per 16-lane group): physical chunk = chunk ^ (2 * (row & 3)).
// Both spread the lanes served together over all 32 banks.
__device__ __forceinline__ int k_swz(int row) { return row & 7; }
__device__ __forceinline__ int v_swz(int row) { return 2 * (row & 3); }

template <typename T, int D, bool CAUSAL, bool SPLIT_P, int WM, int NW, int KSPLIT, int OCC>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC)))
void fa_forward_kernel(Args a) {
  using S = Shape<D, WM, NW, KSPLIT>;
  constexpr int BN = S::BN, BM = S::BM, QB = S::QB, NT = S::NT, DP = S::DP, CPR = S::CPR;
  constexpr int DC = S::DC, DB = S::DB, TILE = S::TILE, LOADS = S::LOADS, NQW = S::NQW;
  // K tiles [buffer][key group], then V tiles [buffer][key group]
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * 2 * KSPLIT * TILE];
  auto kbuf = [&](int buf, int g) { return lds + (buf * KSPLIT + g) * TILE; };
  auto vbuf = [&](int buf, int g) { return lds + ((2 + buf) * KSPLIT + g) * TILE; };

  const int tid = threadIdx.x;
  // wave-uniform, so everything derived from it lives in SGPRs
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kgrp = wave_id / NQW;  // key group: tiles t with t % KSPLIT == kgrp
  const int wave = wave_id - kgrp * NQW;  // query slot within the workgroup
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

  const int q0 = qt * BM + wave * WM;  // first query row of this wave

  // Q fragments: query q0 + 32*qb + l32, columns 16*ch + 8*hi .. +7.
  u32x4 qf[DC][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = q0 + 32 * qb + l32;
#pragma unroll
    for (int ch = 0; ch < DC; ++ch) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qrow < N) x = *(const u32x4*)(Q + (size_t)qrow * D + 16 * ch + 8 * hi);
      qf[ch][qb] = x ^ a.qxor;
    }
  }

  f32x16 oacc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x16{};
  float m_run[QB], l_run[QB];  // running max of raw scores; this lane's share of l
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  const int kv_end = CAUSAL ? min(N, qt * BM + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;

  // Direct global -> LDS loads of one step: tiles KSPLIT*st .. +KSPLIT-1
  // into dst[0 .. KSPLIT-1], through a buffer resource whose range starts at
  // the step's first key and ends at key N, so rows past N read as zero
  // (the hardware range check).  Load i of this thread fills chunk
  // p = (i * NT + tid) of the step's area: tile p / (BN*CPR), row
  // (p / CPR) % BN, physical chunk p % CPR, which holds logical chunk
  // (p % CPR) ^ swz(row).  Chunks past D (D = 96) are not loaded.
  uint32_t koff[LOADS], voff[LOADS];
  bool lpred[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = i * NT + tid;
    const int tl = p / (BN * CPR);
    const int row = (p / CPR) % BN, pc = p % CPR;
    koff[i] = ((tl * BN + row) * D + 8 * (pc ^ k_swz(row))) * 2;
    voff[i] = ((tl * BN + row) * D + 8 * (pc ^ v_swz(row))) * 2;
    lpred[i] = DP == D || (pc ^ k_swz(row)) < D / 8;
  }
  // (the V swizzle moves chunks differently, so its predicate is separate)
  bool vpred[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = i * NT + tid;
    const int row = (p / CPR) % BN, pc = p % CPR;
    vpred[i] = DP == D || (pc ^ v_swz(row)) < D / 8;
  }
  auto step_load = [&](uint16_t* dst, const uint16_t* __restrict__ src, int st, auto is_v) {
    constexpr bool IS_V = decltype(is_v)::value;
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist in device code only
    const int k0 = KSPLIT * st * BN;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + (size_t)k0 * D), 0, (N - k0) * D * 2, 0x00020000);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (IS_V ? vpred[i] : lpred[i])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(dst + (size_t)(i * NT + wave_id * 64) * 8),
            16, IS_V ? voff[i] : koff[i], 0, 0, 0);
    }
#endif
  };

  // S^T = K Q^T for the two 32-key blocks of the tile in K buffer kbuf.
  // s[kb][qb][e] is the score of key k0 + 32*kb + 8*(e/4) + 4*hi + (e%4)
  // against query q0 + 32*qb + l32.  The two key blocks form independent
  // MFMA chains, issued alternately.
  auto qk = [&](const uint16_t* kt, f32x16 (&s)[2][QB]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int ch = 0; ch < DC; ++ch)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + l32;
        const int pc = (2 * ch + hi) ^ k_swz(row);
        const u32x4 kf = *(const u32x4*)(kt + row * DP + 8 * pc);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = Ops<T>::mma(kf, qf[ch][qb], s[kb][qb]);
      }
  };

  // V^T transpose-read source of this lane: within each 16-lane group g,
  // lane 4*i + j addresses key row i (+4*hi) and the 8 bytes at columns
  // 16*(g&1) + 4*j .. +3 of each 32-column block.
  const int grp = lane >> 4, gl = lane & 15;
  const int tr_row = 4 * hi + (gl >> 2);  // + 16*kc (+ 8 for the second read)
  // chunk of column 32*db + 16*(g&1) + 4*j is 4*db + 2*(g&1) + (j>>1); the
  // row's swizzle depends on row & 3 = gl >> 2 only
  const int tr_chunk_lo = (2 * (grp & 1) + ((gl & 3) >> 1)) ^ v_swz(tr_row);
  const int tr_byte = 8 * (gl & 1);

  uint32_t pk[QB][2][8];  // P packed to 16 bits: [qb][kb][pair]
  uint32_t pl[QB][2][8];  // bf16 low parts (split P)
  float alpha[QB];
  bool any_raise;

  // exp2(s*c - m*c) for one query block, packed to 16 bits; returns this
  // lane's sum of the packed P.  MASK zeroes masked keys (s == -inf) exactly,
  // also when c == 0.
  auto exp_pack = [&](auto mask_tag, f32x16 (&s)[2][QB], int qb, float mc) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float s0 = s[kb][qb][2 * j], s1 = s[kb][qb][2 * j + 1];
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, c, -mc));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, c, -mc));
        if constexpr (MASK) {
          p0 = s0 == -INFINITY ? 0.f : p0;
          p1 = s1 == -INFINITY ? 0.f : p1;
        }
        const uint32_t w = Ops<T>::pack(p0, p1);
        pk[qb][kb][j] = w;
        if constexpr (SPLIT_P) {
          pl[qb][kb][j] = Ops<T>::pack(p0 - Ops<T>::lo_to_f32(w), p1 - Ops<T>::hi_to_f32(w));
          psum += p0 + p1;
        } else {
          psum = Ops<T>::add_pair(w, psum);
        }
      }
    return psum;
  };

  // Full online-softmax update of one tile: row maximum, lazy raise of the
  // running maximum, exp / pack.  EDGE applies the ragged and causal masks.
  auto softmax_full = [&](auto edge_tag, int t, f32x16 (&s)[2][QB]) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int k0 = t * BN;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = q0 + 32 * qb + l32;
      if constexpr (EDGE) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * hi + (e & 3);
            if (key >= N || (CAUSAL && key > qrow)) s[kb][qb][e] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][qb][e]);
      mx = half_max(mx);
      // Lazy maximum: raise it only when the tile's maximum is more than
      // kLazy (log2 units) above it.
      const bool raise = (m_run[qb] == -INFINITY) || ((mx - m_run[qb]) * c > kLazy);
      const float m_new = raise ? mx : m_run[qb];
      alpha[qb] = (m_run[qb] == -INFINITY) ? 0.f
                  : raise ? __builtin_amdgcn_exp2f((m_run[qb] - m_new) * c) : 1.f;
      any_raise |= raise;
      m_run[qb] = m_new;
      const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
      const float psum = exp_pack(edge_tag, s, qb, mc);
      l_run[qb] = l_run[qb] * alpha[qb] + psum;
    }
  };

  // One tile's softmax.  Interior tiles first try the running maximum as it
  // stands (no row maximum needed): if every lane's sum of P stays within
  // 2^kLazy, no p exceeds 2^kLazy and the running maximum is kept, as the
  // lazy rule would keep it.  Otherwise (and on the first and edge tiles)
  // the full update runs.
  auto softmax = [&](int t, bool edge, bool first, f32x16 (&s)[2][QB]) {
    any_raise = false;
    if (edge) {
      softmax_full(std::true_type{}, t, s);
      return;
    }
    if (!first) {
      bool over = false;
      float psum[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        psum[qb] = exp_pack(std::false_type{}, s, qb, m_run[qb] * c);
        over |= !(psum[qb] <= __builtin_amdgcn_ldexpf(1.f, (int)kLazy));
      }
      if (!__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          alpha[qb] = 1.f;
          l_run[qb] += psum[qb];
        }
        return;
      }
    }
    softmax_full(std::false_type{}, t, s);
  };

  // O^T = O^T * alpha + V^T P^T for the tile in V buffer vt.  Chunk kc (16
  // keys) holds pairs 4*(kc&1) .. +3 of key block kc>>1.
  auto pv = [&](const uint16_t* vt) {
    if (__builtin_amdgcn_ballot_w64(any_raise)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] *= alpha[qb];
    }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kb = kc >> 1, base = 4 * (kc & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // rows 16*kc + tr_row and +8 share the swizzle (row & 3)
        const uint16_t* src = vt + (16 * kc + tr_row) * DP + 8 * ((4 * db) ^ tr_chunk_lo);
        const u32x2 v0 = tr_read((const uint16_t*)((const char*)src + tr_byte));
        const u32x2 v1 = tr_read((const uint16_t*)((const char*)(src + 8 * DP) + tr_byte));
        const u32x4 vf = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const u32x4 pf = {pk[qb][kb][base], pk[qb][kb][base + 1], pk[qb][kb][base + 2],
                            pk[qb][kb][base + 3]};
          oacc[db][qb] = Ops<T>::mma(vf, pf, oacc[db][qb]);
          if constexpr (SPLIT_P) {
            const u32x4 pfl = {pl[qb][kb][base], pl[qb][kb][base + 1], pl[qb][kb][base + 2],
                               pl[qb][kb][base + 3]};
            oacc[db][qb] = Ops<T>::mma(vf, pfl, oacc[db][qb]);
          }
        }
      }
    }
  };

  // Step loop, LDS double-buffered.  Step st holds tiles KSPLIT*st ..
  // KSPLIT*st + KSPLIT-1; key group g works on tile KSPLIT*st + g (the
  // groups split the keys of every query row between them).  The loads of
  // step st+1 go out right after the barrier of step st, into the buffers
  // step st-1 used (every wave has finished with them once it passes that
  // barrier), and are awaited at the next barrier.
  const int nsteps = (ntiles + KSPLIT - 1) / KSPLIT;
  step_load(kbuf(0, 0), K, 0, std::false_type{});
  step_load(vbuf(0, 0), V, 0, std::true_type{});
  bool first = true;
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's loads have landed
    __syncthreads();
    if (st + 1 < nsteps) {
      step_load(kbuf(buf ^ 1, 0), K, st + 1, std::false_type{});
      step_load(vbuf(buf ^ 1, 0), V, st + 1, std::true_type{});
    }
    const int t = KSPLIT * st + kgrp;
    const int k0 = t * BN;
    // Causal: a tile whose first key is past this wave's last query
    // contributes nothing.
    if (t >= ntiles || (CAUSAL && k0 > q0 + WM - 1)) continue;
    f32x16 s[2][QB];
    qk(kbuf(buf, kgrp), s);
    const bool edge = (k0 + BN > N) || (CAUSAL && (k0 + BN - 1 > q0));
    softmax(t, edge, first, s);
    first = false;
    pv(vbuf(buf, kgrp));
  }

  if constexpr (KSPLIT == 2) {
    // Merge the two key groups.  Each holds, per query, a running maximum
    // m_g, a share l_g of the denominator and an accumulator O_g, all
    // relative to exp(m_g); with m = max(m_0, m_1) the union of their keys
    // gives l = sum_g l_g exp(m_g - m) and O = sum_g O_g exp(m_g - m), the
    // same rescale rule as the online softmax.  Group 1 hands its state to
    // group 0 through LDS (the tile buffers are free after the barrier).
    constexpr int PER_LANE = DB * QB * 16 + 2 * QB;  // floats per lane
    static_assert(NQW * 64 * PER_LANE * 4 <= (int)sizeof(lds), "merge area");
    float* xch = (float*)lds + (size_t)(wave * 64 + lane) * PER_LANE;
    __syncthreads();
    if (kgrp == 1) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) xch[(qb * DB + db) * 16 + e] = oacc[db][qb][e];
        xch[DB * QB * 16 + 2 * qb] = m_run[qb];
        xch[DB * QB * 16 + 2 * qb + 1] = l_run[qb];
      }
    }
    __syncthreads();
    if (kgrp == 1) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m1 = xch[DB * QB * 16 + 2 * qb];
      const float l1 = xch[DB * QB * 16 + 2 * qb + 1];
      const float m0 = m_run[qb];
      const float m = fmaxf(m0, m1);
      const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m0 - m) * c);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - m) * c);
      l_run[qb] = l_run[qb] * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          oacc[db][qb][e] = oacc[db][qb][e] * a0 + xch[(qb * DB + db) * 16 + e] * a1;
    }
  }

  // Epilogue: divide by the row's denominator once, round, store.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = half_sum(l_run[qb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int qrow = q0 + 32 * qb + l32;
    if (qrow < N) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // elements 4g..4g+3 are columns d0..d0+3 of row qrow
          const int d0 = 32 * db + 8 * g + 4 * hi;
          const f32x16& acc = oacc[db][qb];
          u32x2 out = {Ops<T>::pack(acc[4 * g] * inv, acc[4 * g + 1] * inv),
                       Ops<T>::pack(acc[4 * g + 2] * inv, acc[4 * g + 3] * inv)};
          *(u32x2*)(O + (size_t)qrow * D + d0) = out;
        }
    }
  }
}

template <typename T, int D, bool CAUSAL, bool SPLIT_P, int WM, int NW, int KSPLIT, int OCC>
hipError_t launch_one(const Args& base, int64_t BH, hipStream_t stream) {
  using S = Shape<D, WM, NW, KSPLIT>;
  Args a = base;
  a.num_qtiles = (a.N + S::BM - 1) / S::BM;
  a.total_tiles = (int)(BH * a.num_qtiles);
  void* args[] = {&a};
  return hipLaunchKernel((const void*)fa_forward_kernel<T, D, CAUSAL, SPLIT_P, WM, NW, KSPLIT, OCC>,
                         dim3(a.total_tiles), dim3(S::NT), args, 0, stream);
}

inline Args make_args(const Problem& p) {
  Args a;
  a.q = (const uint16_t*)p.q;
  a.k = (const uint16_t*)p.k;
  a.v = (const uint16_t*)p.v;
  a.o = (uint16_t*)p.o;
  a.N = p.N;
  a.num_qtiles = 0;
  a.total_tiles = 0;
  a.c = __builtin_fabsf(p.scale) * 1.4426950408889634f;
  a.qxor = p.scale < 0.f ? 0x80008000u : 0u;
  return a;
}

// Tile shape per head dimension: 4 waves of 32 query rows (128 rows per
// workgroup).
template <typename T, bool SPLIT_P>
hipError_t launch(const Problem& p, hipStream_t stream) {
  const Args a = make_args(p);
  switch (p.D) {
    case 64:
      return p.causal ? launch_one<T, 64, true, SPLIT_P, 32, 8, 2, 4>(a, p.BH, stream)
                      : launch_one<T, 64, false, SPLIT_P, 32, 8, 2, 4>(a, p.BH, stream);
    case 96:
      return p.causal ? launch_one<T, 96, true, SPLIT_P, 32, 4, 1, 2>(a, p.BH, stream)
                      : launch_one<T, 96, false, SPLIT_P, 32, 4, 1, 2>(a, p.BH, stream);
    case 128:
      return p.causal ? launch_one<T, 128, true, SPLIT_P, 32, 4, 1, 2>(a, p.BH, stream)
                      : launch_one<T, 128, false, SPLIT_P, 32, 4, 1, 2>(a, p.BH, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mfma
}  // namespace fa
