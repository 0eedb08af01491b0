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
//  * A workgroup is NW wave64s (4 or 8) and owns 32*NW query rows of one
//    (batch, head); each wave owns 32 of them and keeps its Q rows in VGPRs
//    as the B operand of v_mfma_f32_32x32x16_{f16,bf16}.  With eight waves
//    the two waves that share a SIMD belong to one workgroup and advance in
//    lockstep (one barrier per tile); waves of different workgroups on one
//    SIMD would not: the older one wins issue and the younger ends alone.
//  * Grids that leave CUs idle (the host's choice, key_groups == 2): the
//    waves of a workgroup form two groups over the same query rows, group g
//    taking key tiles g, g+2, ...; K and V then run in separate two-slot
//    rings of tile pairs (the same eight LDS arrays), and after the loop the
//    two groups' (m, l, O) are merged in LDS by the rescaling rule above.
//  * Key/value tiles of 64 keys go straight from global memory to LDS
//    (buffer_load ... lds, 16 bytes per lane) through a buffer resource that
//    ends at key N, so rows past N read as zero.  A ring of four LDS slots
//    per operand: while tile t is used, tile t+1 is resident and tile t+2
//    is in flight.  Each slot is an array of its own and the loop is
//    unrolled over the ring, which lets the compiler see that the transpose
//    reads of one slot do not touch the loads still landing in another (it
//    would otherwise make them wait for those loads).
//  * LDS rows are not padded (the direct loads write each wave's 1 KiB
//    contiguously); 16-byte chunks are XOR-swizzled per row instead, so the
//    operand reads hit distinct banks of gfx950's 64-bank LDS.
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
//  * Software pipeline inside each wave: the MFMAs that form the scores of
//    tile t+1 issue among the exponentials of tile t, and the P V MFMAs of
//    tile t among the 16-bit conversions and the row sums.  With D = 64 the
//    K fragments of the step are read first and the exponent FMAs, the
//    tile maximum and the lazy check run while those reads are in flight;
//    with D = 96, 128 (no room for the fragments) the score MFMAs start at
//    once and the check follows.
//  * Softmax runs in base 2: p = exp2(s * c - m * c) with c = |scale| *
//    log2(e) in one FMA; a negative scale flips the sign of Q.  p is formed
//    with the running maximum as it stands and checked afterwards: only
//    when some exponent of the wave exceeds kLazy (log2 units) does the wave
//    raise m to the row maximum, rescale O and l, and form p again.  So the
//    maximum stays out of the common path, tile p values may reach 2^kLazy
//    (fp32 accumulators and 16-bit P hold that without loss), and the
//    result is the same softmax, exp(s - m) / sum exp(s - m), for any m.
//  * fp16: P is rounded once to fp16, and l sums exactly those rounded
//    values (v_fma_mix_f32, which widens a half exactly and, unlike v_dot2,
//    issues beside running MFMAs), so the weights applied to V sum to one.
//    bf16: P is kept as an unevaluated sum of two bf16 numbers (hi + lo)
//    and two PV products are issued, so P carries ~16 significant bits, as
//    with fp16, and l sums the fp32 p; except on tiles where every weight
//    is small against the row's sum so far, this tile included (below
//    kSplitTau of it), which take P rounded once to bf16 and add the
//    rounded values to l.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kBlockN = 64;  // keys per LDS tile unless the shape says otherwise
constexpr float kLazy = 8.f;  // log2 of the largest p the lazy maximum allows
// bf16: a tile whose weights all stay below this share of the row's running
// denominator is multiplied with P rounded once (see the tile body)
constexpr float kSplitTau = 0.125f;

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  Layout lq, lk, lv, lo;  // element strides of each tensor
  int H;                  // query heads per batch
  int group;              // query heads per key/value head
  int N;
  int num_qtiles;   // ceil(N / BM)
  int total_tiles;  // BH * num_qtiles * splits
  int splits;       // key-range splits per query block (1: O written directly)
  float* part_o;    // splits > 1: [splits, BH, N, D] fp32 partial O (normalised)
  float* part_lse;  // splits > 1: [splits, BH, N] partial log-sum-exp
  float* lse;       // splits == 1, optional: [BH, N] log-sum-exp of the scaled scores
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
  // acc + the low / high fp16 half of w, in fp32 (one v_fma_mix_f32 each:
  // the half is widened exactly, times 1.0, plus acc, rounded once).  Unlike
  // v_dot2 these issue beside running matrix-core instructions.
  static __device__ __forceinline__ float add_lo(uint32_t w, float acc) {
    asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w));
    return acc;
  }
  static __device__ __forceinline__ float add_hi(uint32_t w, float acc) {
    asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w));
    return acc;
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
  // acc + both bf16 halves of w, in fp32: one v_dot2c_f32_bf16 against
  // (1, 1) (the products are exact) in place of two widenings and two adds.
  static __device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
  }
};

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

// Maximum of 32 values as a tree of v_max3_f32 (depth 4, not a chain).
__device__ __forceinline__ float max32(const float (&x)[2][16]) {
  float a[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int j = 3 * i;
    a[i] = fmaxf(fmaxf(x[j / 16][j % 16], x[(j + 1) / 16][(j + 1) % 16]), x[(j + 2) / 16][(j + 2) % 16]);
  }
  a[10] = fmaxf(x[1][14], x[1][15]);
  const float b0 = fmaxf(fmaxf(a[0], a[1]), a[2]);
  const float b1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
  const float b2 = fmaxf(fmaxf(a[6], a[7]), a[8]);
  const float b3 = fmaxf(a[9], a[10]);
  return fmaxf(fmaxf(b0, b1), fmaxf(b2, b3));
}

// Maximum of 16 values (one 32-key block).
__device__ __forceinline__ float max16(const float (&x)[1][16]) {
  const float a0 = fmaxf(fmaxf(x[0][0], x[0][1]), x[0][2]), a1 = fmaxf(fmaxf(x[0][3], x[0][4]), x[0][5]);
  const float a2 = fmaxf(fmaxf(x[0][6], x[0][7]), x[0][8]), a3 = fmaxf(fmaxf(x[0][9], x[0][10]), x[0][11]);
  const float a4 = fmaxf(fmaxf(x[0][12], x[0][13]), x[0][14]);
  return fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), x[0][15]));
}
__device__ __forceinline__ float max_tile(const float (&x)[2][16]) { return max32(x); }
__device__ __forceinline__ float max_tile(const float (&x)[1][16]) { return max16(x); }

__device__ __forceinline__ u32x2 tr_read(const uint16_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_u16*)p);
  return __builtin_bit_cast(u32x2, r);
}

// BN keys per LDS tile (one barrier and one ring slot each); the softmax
// and products run on sub-tiles of CB = min(BN, 64) keys (KB blocks of 32),
// SUB of them per LDS tile.
template <int D, int NW, int BN_ = kBlockN>
struct Shape {
  static constexpr int BN = BN_;         // keys per LDS tile
  static constexpr int CB = BN < 64 ? BN : 64;  // keys per compute sub-tile
  static constexpr int KB = CB / 32;     // 32-key blocks per sub-tile
  static constexpr int SUB = BN / CB;    // sub-tiles per LDS tile
  static constexpr int NT = 64 * NW;     // threads per workgroup
  static constexpr int DP = D <= 64 ? 64 : 128;  // LDS row length (elements)
  static constexpr int CPR = DP / 8;     // 16-byte chunks per LDS row
  static constexpr int DC = D / 16;      // 16-wide contraction chunks of QK^T
  static constexpr int DB = D / 32;      // 32-row blocks of O^T
  static constexpr int TILE = BN * DP;   // elements per LDS tile buffer
  static constexpr int CHUNKS = BN * CPR;  // 16-byte chunks per tile operand
  static constexpr int LOADS = (CHUNKS + NT - 1) / NT;  // 16-byte loads per thread per tile
  static_assert(D % 32 == 0 && D <= 128, "head dim");
  static_assert(BN == 32 || BN == 64 || BN == 128, "key tile");
  static_assert(CHUNKS % 64 == 0, "whole wave-loads per tile");
};

// LDS tile layouts.  A tile row (one key) is DP elements = CPR chunks of 16
// bytes, rows back to back (the direct global->LDS loads write each wave's
// 64 x 16 bytes contiguously, so rows cannot be padded).  Chunks are
// permuted within a row by an XOR with a function of the row:
//  * K (read by ds_read_b128, 16 consecutive rows at one logical chunk per
//    LDS cycle, 64 banks of 4 bytes): with 128-byte rows (DP = 64) rows r
//    and r+1 start 32 banks apart, so physical chunk = chunk ^ ((row >> 1)
//    & 7) puts the 16 rows on 16 distinct 4-bank groups; a 256-byte row
//    (DP = 128) spans all 64 banks, so chunk ^ (row & 15) does.
//  * V (read by ds_read_b64_tr_b16, 4 consecutive rows x 4 adjacent chunks
//    per 32 lanes): physical chunk = chunk ^ (2 * (row & 3)) with 128-byte
//    rows (rows r and r+1 on different bank halves), chunk ^ (4 * (row & 3))
//    with 256-byte rows, so the 4 rows read 4 disjoint 64-byte bank groups.
template <int DP>
__device__ __forceinline__ int k_swz(int row) {
  return DP == 64 ? (row >> 1) & 7 : row & 15;
}
template <int DP>
__device__ __forceinline__ int v_swz(int row) {
  return DP == 64 ? 2 * (row & 3) : 4 * (row & 3);
}

// FULL: no causal mask and N a multiple of the key tile, so every tile of
// the loop holds keys for every row and none needs a mask (the host picks
// this instance when that holds; it skips the per-tile checks).
template <typename T, int D, bool CAUSAL, bool SPLIT_P, int NW, int OCC, int KS, int BN_, bool FULL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC)))
void fa_forward_kernel(Args a) {
  using S = Shape<D, NW, BN_>;
  // KS key groups: with KS = 2 the waves form two groups over the same query
  // rows, group g taking key tiles g, g+2, g+4, ... of the range, and their
  // results are merged at the end (for grids that leave CUs idle).
  static_assert(KS == 1 || ((KS == 2 || KS == 4) && NW % KS == 0), "key groups");
  static_assert(KS == 1 || (KS == 2 && S::BN == 64) || (KS == 4 && S::BN == 32),
                "two key groups take 64-key tiles, four take 32-key tiles");
  constexpr int NWR = NW / KS;  // waves per key group = 32-row blocks per workgroup
  constexpr int BN = S::BN, BM = 32 * NWR, NT = S::NT, DP = S::DP, CPR = S::CPR;
  constexpr int DC = S::DC, DB = S::DB, TILE = S::TILE, LOADS = S::LOADS;
  constexpr int CB = S::CB, KB = S::KB, SUB = S::SUB;
  // A ring of four LDS slots per operand (tile t in slot t % 4), each slot
  // an array of its own, and the step loop unrolled over the ring: the
  // compiler can then tell the slots apart, so a transpose read of one slot
  // does not wait for the global->LDS loads still in flight into another.
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[TILE], k1s[TILE], k2s[TILE], k3s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[TILE], v1s[TILE], v2s[TILE], v3s[TILE];
  // four key groups: two slots of four tiles per operand, eight arrays each
  constexpr int TILE4 = KS == 4 ? TILE : 1;
  __shared__ __attribute__((aligned(1024))) uint16_t k4s[TILE4], k5s[TILE4], k6s[TILE4], k7s[TILE4];
  __shared__ __attribute__((aligned(1024))) uint16_t v4s[TILE4], v5s[TILE4], v6s[TILE4], v7s[TILE4];
  auto kbuf = [&](auto slot) -> uint16_t* {
    constexpr int j = decltype(slot)::value & 7;
    if constexpr (j == 0) return k0s;
    else if constexpr (j == 1) return k1s;
    else if constexpr (j == 2) return k2s;
    else if constexpr (j == 3) return k3s;
    else if constexpr (j == 4) return k4s;
    else if constexpr (j == 5) return k5s;
    else if constexpr (j == 6) return k6s;
    else return k7s;
  };
  auto vbuf = [&](auto slot) -> uint16_t* {
    constexpr int j = decltype(slot)::value & 7;
    if constexpr (j == 0) return v0s;
    else if constexpr (j == 1) return v1s;
    else if constexpr (j == 2) return v2s;
    else if constexpr (j == 3) return v3s;
    else if constexpr (j == 4) return v4s;
    else if constexpr (j == 5) return v5s;
    else if constexpr (j == 6) return v6s;
    else return v7s;
  };

  const int tid = threadIdx.x;
  // wave-uniform, so everything derived from it lives in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int kgrp = KS == 1 ? 0 : wave / NWR;  // key group
  const int rb = wave - kgrp * NWR;            // 32-row block

  const int per_head = a.num_qtiles * a.splits;
  int bh, qt, split = 0;
  if (CAUSAL && a.splits == 1) {
    const int id = causal_lpt(blockIdx.x, a.total_tiles, a.num_qtiles);
    bh = id / a.num_qtiles;
    qt = a.num_qtiles - 1 - (id - bh * a.num_qtiles);
  } else {
    const int logical = xcd_remap(blockIdx.x, a.total_tiles);
    bh = logical / per_head;
    const int rem = logical - bh * per_head;
    qt = rem / a.splits;
    split = rem - qt * a.splits;
    if (CAUSAL) qt = a.num_qtiles - 1 - qt;  // longest rows first
  }
  const int N = a.N;
  const int b = bh / a.H, h = bh - b * a.H, hk = h / a.group;
  const uint16_t* __restrict__ Q = a.q + b * a.lq.sb + h * a.lq.sh;
  [[maybe_unused]] const uint16_t* __restrict__ K = a.k + b * a.lk.sb + hk * a.lk.sh;
  [[maybe_unused]] const uint16_t* __restrict__ V = a.v + b * a.lv.sb + hk * a.lv.sh;
  uint16_t* __restrict__ O = a.o + b * a.lo.sb + h * a.lo.sh;
  const int ldq = a.lq.sn, ldk = a.lk.sn, ldv = a.lv.sn, ldo = a.lo.sn;  // row strides
  const float c = a.c;

  const int q0 = qt * BM + rb * 32;  // first query row of this wave
  const int qrow = q0 + l32;           // this lane's query row

  // Q fragment: row qrow, columns 16*ch + 8*hi .. +7 (B operand layout).
  u32x4 qf[DC];
#pragma unroll
  for (int ch = 0; ch < DC; ++ch) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qrow < N) x = *(const u32x4*)(Q + (size_t)qrow * ldq + 16 * ch + 8 * hi);
    qf[ch] = x ^ a.qxor;
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // running (lazy) max of raw scores q.k
  float mc = 0.f;           // m_run * c once m_run is finite
  float lp[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's share of the denominator

  const int kv_end = CAUSAL ? min(N, qt * BM + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  // This workgroup's share of the key tiles: an even cut of [0, ntiles)
  // into `splits` ranges (the whole range when splits == 1).
  const int t_lo = split * ntiles / a.splits;
  const int t_hi = (split + 1) * ntiles / a.splits;
  // the same range in compute sub-tiles of CB keys
  const int u_lo = t_lo * SUB;
  const int u_hi = min(t_hi * SUB, (kv_end + CB - 1) / CB);

  // Direct global -> LDS loads of the next tile, through a buffer resource
  // whose range starts at the tile's first key and ends at key N, so rows
  // past N read as zero (the hardware range check).  Load i of this thread
  // fills chunk p = i * NT + tid of the tile: row p / CPR, physical chunk
  // p % CPR, which holds logical chunk (p % CPR) ^ swz(row).  Chunks past D
  // (D = 96) are not loaded.
  uint32_t koff[LOADS], voff[LOADS];
  bool kpred[LOADS], vpred[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = i * NT + tid;
    const int row = p / CPR, pc = p % CPR;
    koff[i] = (row * ldk + 8 * (pc ^ k_swz<DP>(row))) * 2;
    voff[i] = (row * ldv + 8 * (pc ^ v_swz<DP>(row))) * 2;
    // whole waves past the tile (fewer chunks than threads) load nothing
    const bool in_tile = S::CHUNKS % NT == 0 || p < S::CHUNKS;
    kpred[i] = in_tile && (DP == D || (pc ^ k_swz<DP>(row)) < D / 8);
    vpred[i] = in_tile && (DP == D || (pc ^ v_swz<DP>(row)) < D / 8);
  }
  // Tiles are loaded once each, in increasing order, so the loads follow a
  // running pointer and byte count (wave-uniform) instead of forming the
  // tile's address from its index.  The byte counts run from the tile's
  // first key to key N: max(N, 64) row strides stay below 2^32 (checked by
  // the host), so the unsigned arithmetic does not wrap.
  [[maybe_unused]] const char* k_next = (const char*)K + (size_t)t_lo * BN * ldk * 2;
  [[maybe_unused]] const char* v_next = (const char*)V + (size_t)t_lo * BN * ldv * 2;
  [[maybe_unused]] uint32_t k_left = (uint32_t)(N - t_lo * BN) * (uint32_t)(2 * ldk);
  [[maybe_unused]] uint32_t v_left = (uint32_t)(N - t_lo * BN) * (uint32_t)(2 * ldv);
  auto load_next_tile = [&](uint16_t* kdst, uint16_t* vdst) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist in device code only
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)k_next, 0, (int)k_left, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)v_next, 0, (int)v_left, 0x00020000);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const size_t at = (size_t)(i * NT + wave * 64) * 8;
      if (kpred[i])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(kdst + at), 16, koff[i], 0, 0, 0);
      if (vpred[i])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(vdst + at), 16, voff[i], 0, 0, 0);
    }
    k_next += (size_t)BN * ldk * 2;
    v_next += (size_t)BN * ldv * 2;
    k_left -= (uint32_t)(BN * 2 * ldk);
    v_left -= (uint32_t)(BN * 2 * ldv);
#endif
  };
  // KS == 2: K runs a pair of tiles ahead of V, so each operand follows its
  // own running pointer.
  auto load_k_tile = [&](uint16_t* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)k_next, 0, (int)k_left, 0x00020000);
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      if (kpred[i])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(dst + (size_t)(i * NT + wave * 64) * 8), 16, koff[i], 0,
            0, 0);
    k_next += (size_t)BN * ldk * 2;
    k_left -= (uint32_t)(BN * 2 * ldk);
#endif
  };
  auto load_v_tile = [&](uint16_t* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)v_next, 0, (int)v_left, 0x00020000);
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      if (vpred[i])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(dst + (size_t)(i * NT + wave * 64) * 8), 16, voff[i], 0,
            0, 0);
    v_next += (size_t)BN * ldv * 2;
    v_left -= (uint32_t)(BN * 2 * ldv);
#endif
  };

  // S^T = K Q^T for the two 32-key blocks of the tile at kt.  s[kb][e] is
  // the score of key k0 + 32*kb + 8*(e/4) + 4*hi + (e%4) against query
  // qrow.  The two key blocks form independent MFMA chains, issued
  // alternately.
  // Byte offset of this lane's K operand chunk ch within a tile (key block
  // 0; key block 1 is 32 rows further, with the same swizzle).
  uint32_t k_off[DC];
#pragma unroll
  for (int ch = 0; ch < DC; ++ch) k_off[ch] = (l32 * DP + 8 * ((2 * ch + hi) ^ k_swz<DP>(l32))) * 2;
  auto k_frag = [&](const uint16_t* kt, int ch, int kb) -> u32x4 {
    return *(const u32x4*)((const char*)kt + k_off[ch] + kb * (32 * DP * 2));
  };
  auto qk = [&](const uint16_t* kt, f32x16 (&s)[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ch = 0; ch < DC; ++ch)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = Ops<T>::mma(k_frag(kt, ch, kb), qf[ch], s[kb]);
  };

  // V^T transpose-read source of this lane: within each 16-lane group g,
  // lane 4*i + j addresses key row i (+4*hi) and the 8 bytes at columns
  // 16*(g&1) + 4*j .. +3 of each 32-column block.
  const int grp = lane >> 4, gl = lane & 15;
  const int tr_row = 4 * hi + (gl >> 2);  // + 16*kc (+ 8 for the second read)
  // chunk of column 32*db + 16*(g&1) + 4*j is 4*db + 2*(g&1) + (j>>1); the
  // row's swizzle depends on row & 3 = gl >> 2 only
  const int tr_chunk_lo = (2 * (grp & 1) + ((gl & 3) >> 1)) ^ v_swz<DP>(tr_row);
  const int tr_byte = 8 * (gl & 1);

  static_assert(!(FULL && CAUSAL), "a causal tile loop has masked tiles");
  auto live = [&](int u) {  // sub-tile u is in range and holds keys this wave sees
    // one key group: the loop stops at the last tile; two: the second
    // group's last tile may lie past the range
    if constexpr (FULL && KS == 1) return true;
    return u < u_hi && (!CAUSAL || u * CB <= q0 + 31);
  };
  auto is_edge = [&](int u) {  // sub-tile u needs the ragged / causal masks
    if constexpr (FULL) return false;
    return (u * CB + CB > N) || (CAUSAL && (u * CB + CB - 1 > q0));
  };

  // V^T fragment for P V: keys 16*kc .. +15 (in the P key order), head-dim
  // columns 32*db .. +31.  Rows 16*kc + tr_row and +8 share the swizzle
  // (row & 3); both addresses are formed from the slot base (derived one
  // from the other, the second read lost the alias information that lets
  // the compiler see it does not touch the slot being loaded).
  uint32_t v_off[DB];  // bytes: row tr_row, the lane's columns of block db
#pragma unroll
  for (int db = 0; db < DB; ++db) v_off[db] = tr_row * DP * 2 + 2 * 8 * ((4 * db) ^ tr_chunk_lo) + tr_byte;
  auto v_frag = [&](const uint16_t* vt, int kc, int db) -> u32x4 {
    const u32x2 v0 = tr_read((const uint16_t*)((const char*)vt + v_off[db] + 16 * kc * DP * 2));
    const u32x2 v1 = tr_read((const uint16_t*)((const char*)vt + v_off[db] + (16 * kc + 8) * DP * 2));
    return u32x4{v0[0], v0[1], v1[0], v1[1]};
  };
  // Marks the lane offsets as redefined: otherwise the compiler forms the
  // address of every (ring slot, chunk) pair once before the loop and keeps
  // them all in registers (48 at D = 128, which spills), instead of adding
  // the slot base as the instruction's immediate offset.
  auto refresh_offsets = [&]() {
#pragma unroll
    for (int ch = 0; ch < DC; ++ch) asm volatile("" : "+v"(k_off[ch]));
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(v_off[db]));
  };

  // The work of one tile: softmax of the tile whose scores sc were computed
  // in the previous step, the scores sn of the next tile, and P V.  The
  // exponents x = s*c - m*c are formed with the running maximum m as it
  // stands, and the tile is checked: when some x of the wave exceeds kLazy
  // (and always on the first tile, when m is still -inf) the wave takes the
  // rare path that raises m to the true row maximum, rescales O and the
  // denominator by exp(m_old - m_new), and forms x again.  Otherwise m
  // stays, p = exp2(x) may reach 2^kLazy, and no rescale is needed; the
  // result is the same softmax for any m.  The next tile's scores are
  // computed even when that tile is not used (past the end, or causally
  // masked for this wave); masked scores are -inf and c > 0, so their p is
  // exactly 0.
  //
  // Two orders, the same arithmetic.  With D = 64 (check_first) the wave
  // issues its K fragment reads, forms x, the maximum and the check while
  // they are in flight, then issues the V fragment reads and the next
  // tile's MFMAs with all exponentials beside them, then the 16-bit P, the
  // row sums and P V.
  // With D = 96, 128 the fragments would not fit in registers beside the
  // larger accumulators: the next tile's MFMAs issue among the exponent
  // FMAs and the first key block's exponentials (reading K as they go),
  // the check follows, and V is read during P V.
  constexpr bool check_first = D == 64;
  auto tile_body = [&](const uint16_t* kt_next, const uint16_t* vt, f32x16 (&sc)[KB],
                       f32x16 (&sn)[KB], bool first) {
    refresh_offsets();
    [[maybe_unused]] u32x4 kf[DC][KB], vf[2 * KB][DB];
    if constexpr (check_first) {
#pragma unroll
      for (int ch = 0; ch < DC; ++ch)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kf[ch][kb] = k_frag(kt_next, ch, kb);
    }
    float x[KB][16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) x[kb][e] = __builtin_fmaf(sc[kb][e], c, -mc);
    if constexpr (!check_first) qk(kt_next, sn);
    const float xmax = max_tile(x);
    float p[KB][16];
    if constexpr (!check_first) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[0][e] = __builtin_amdgcn_exp2f(x[0][e]);
        // issue these beside the MFMAs above, not after the check below
        asm volatile("" ::"v"(p[0][e]));
      }
    }
    if (__builtin_amdgcn_ballot_w64(first || xmax > kLazy)) {
      // keeps the compiler from turning this rare path into selects that
      // would run on every tile
      asm volatile("" ::: "memory");
      float sm[KB][16];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sm[kb][e] = sc[kb][e];
      const float mx = half_max(max_tile(sm));  // the row's maximum in this tile
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);  // 0 when m_run = -inf
      m_run = m_new;
      mc = m_new == -INFINITY ? 0.f : m_new * c;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) lp[i] *= alpha;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) x[kb][e] = __builtin_fmaf(sc[kb][e], c, -mc);
      if constexpr (!check_first) {
#pragma unroll
        for (int e = 0; e < 16; ++e) p[0][e] = __builtin_amdgcn_exp2f(x[0][e]);
      }
    }
    if constexpr (check_first) {
#pragma unroll
      for (int kc = 0; kc < 2 * KB; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) vf[kc][db] = v_frag(vt, kc, db);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sn[kb] = f32x16{};
#pragma unroll
      for (int ch = 0; ch < DC; ++ch)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sn[kb] = Ops<T>::mma(kf[ch][kb], qf[ch], sn[kb]);
#pragma unroll
      for (int e = 0; e < 16; ++e) p[0][e] = __builtin_amdgcn_exp2f(x[0][e]);
    }
#pragma unroll
    for (int kb = 1; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) p[kb][e] = __builtin_amdgcn_exp2f(x[kb][e]);
    // bf16 keeps 8 significant bits of each weight.  A wave multiplies
    // with P rounded once when no lane's largest p of this tile exceeds
    // kSplitTau of that lane's share of the row's denominator, this tile's
    // rounded weights included (lanes 0-31 and 32-63 hold the two halves of
    // each row's keys, so the row's largest weight then stays below
    // kSplitTau of the row's sum so far, and so of its final sum: the
    // rounding error any one key adds to O is at most 2^-9 kSplitTau |v - O|);
    // where a few keys carry a large share of the row, as on its first
    // tiles, it also multiplies with the rounded remainder lo = p - hi, so
    // that P carries ~16 significant bits.  xmax may be stale after a
    // rescale of m, which only overstates p.
    // (The eight-wave two-key-group kernels at D = 96 and 128 have no
    // registers to spare for the branch and always take both products,
    // interleaved; with four waves, one per SIMD, they have.)
    constexpr bool ADAPT = SPLIT_P && (KS != 2 || D == 64 || NW == 4);
    // P V over the chunks of 16 keys, with P rounded once (RNE); the row
    // sums add the rounded values, so that the weights applied to V sum to
    // one (this matters when a few keys dominate a row).
#pragma unroll
    for (int kc = 0; kc < 2 * KB; ++kc) {
      // chunk kc (16 keys) = pairs 4*(kc&1) .. +3 of key block kc>>1
      const int kb = kc >> 1, base = 8 * (kc & 1);
      u32x4 pf, pfl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = p[kb][base + 2 * j], p1 = p[kb][base + 2 * j + 1];
        const uint32_t w = Ops<T>::pack(p0, p1);
        pf[j] = w;
        if constexpr (SPLIT_P && !ADAPT) {
          const uint32_t wl = Ops<T>::pack(p0 - Ops<T>::lo_to_f32(w), p1 - Ops<T>::hi_to_f32(w));
          pfl[j] = wl;
          lp[j] += p0 + p1;  // hi + lo carry p to ~16 significant bits
        } else if constexpr (SPLIT_P) {
          lp[j] = Ops<T>::add_pair(w, lp[j]);
        } else {
          lp[j] = Ops<T>::add_hi(w, Ops<T>::add_lo(w, lp[j]));
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4 v = check_first ? vf[kc][db] : v_frag(vt, kc, db);
        oacc[db] = Ops<T>::mma(v, pf, oacc[db]);
        if constexpr (SPLIT_P && !ADAPT) oacc[db] = Ops<T>::mma(v, pfl, oacc[db]);
      }
    }
    if constexpr (ADAPT) {
      const float lane_l = (lp[0] + lp[1]) + (lp[2] + lp[3]);
      const float pmax = __builtin_amdgcn_exp2f(xmax);
      if (__builtin_amdgcn_ballot_w64(!(pmax <= kSplitTau * lane_l)) != 0) {
        // the rounded remainders, their products and their row sums
#pragma unroll
        for (int kc = 0; kc < 2 * KB; ++kc) {
          const int kb = kc >> 1, base = 8 * (kc & 1);
          u32x4 pfl;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p0 = p[kb][base + 2 * j], p1 = p[kb][base + 2 * j + 1];
            const uint32_t w = Ops<T>::pack(p0, p1);
            const uint32_t wl = Ops<T>::pack(p0 - Ops<T>::lo_to_f32(w), p1 - Ops<T>::hi_to_f32(w));
            pfl[j] = wl;
            lp[j] = Ops<T>::add_pair(wl, lp[j]);
          }
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x4 v = check_first ? vf[kc][db] : v_frag(vt, kc, db);
            oacc[db] = Ops<T>::mma(v, pfl, oacc[db]);
          }
        }
      }
    }
  };

  // Ragged / causal masks of the scores of sub-tile u.
  auto mask_scores = [&](int u, f32x16 (&sc)[KB]) {
    if (is_edge(u)) {
      const int k0 = u * CB;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * hi + (e & 3);
          if (key >= N || (CAUSAL && key > qrow)) sc[kb][e] = -INFINITY;
        }
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  f32x16 sA[KB], sB[KB];
  if constexpr (KS == 1) {
    // Software pipeline over the ring.
    if (t_lo < t_hi) {
      load_next_tile(kbuf(I0{}), vbuf(I0{}));
      if (t_lo + 1 < t_hi) load_next_tile(kbuf(I1{}), vbuf(I1{}));
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      // the first tile of the range holds the first key that any row of the
      // range sees (a causal row sees a prefix of the keys)
      qk(kbuf(I0{}), sA);
    }
    // Step t (t % 4 == J): pass the barrier (tile t+1, whose loads went out
    // in step t-1, is then visible, and every wave is done with step t-1);
    // issue the loads of tile t+2 into slot (t+2) % 4, last read in step
    // t-2; then the tile body on each of the tile's SUB sub-tiles: softmax
    // of the sub-tile, whose scores were computed in the previous body,
    // while the scores of the next sub-tile (the second half of this tile,
    // or the first of tile t+1) are computed, and P V of the sub-tile.
    auto step = [&](int t, auto J, f32x16 (&s0)[KB], f32x16 (&s1)[KB]) {
      constexpr int j = decltype(J)::value;
      using Next = std::integral_constant<int, (j + 1) & 3>;
      using Pre2 = std::integral_constant<int, (j + 2) & 3>;
      // unconditional (redundant at t = 0), so that every path into the
      // transpose reads below passes a wait for the loads of step t-1
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile t+1 has landed
      __syncthreads();
      if (t + 2 < t_hi) load_next_tile(kbuf(Pre2{}), vbuf(Pre2{}));
      const int u = t * SUB;
      if (live(u)) {
        mask_scores(u, s0);
        tile_body(SUB == 1 ? kbuf(Next{}) : kbuf(J) + CB * DP, vbuf(J), s0, s1, u == u_lo);
      }
      if constexpr (SUB == 2) {
        if (live(u + 1)) {
          mask_scores(u + 1, s1);
          tile_body(kbuf(Next{}), vbuf(J) + CB * DP, s1, s0, u + 1 == u_lo);
        }
      }
    };
    // The guards nest so that step t+2 is only reached through step t+1 (and
    // its wait for the loads of step t); with flat guards the compiler sees a
    // path that skips it and makes the transpose reads of step t+2 wait for
    // those loads.  The score registers alternate per sub-tile: with two
    // sub-tiles per tile every step starts on sA.
    auto& sC = SUB == 1 ? sB : sA;  // the first score set of odd steps
    auto& sD = SUB == 1 ? sA : sB;
    for (int t = t_lo; t < t_hi; t += 4) {
      step(t, I0{}, sA, sB);
      if (t + 1 < t_hi) {
        step(t + 1, I1{}, sC, sD);
        if (t + 2 < t_hi) {
          step(t + 2, I2{}, sA, sB);
          if (t + 3 < t_hi) step(t + 3, I3{}, sC, sD);
        }
      }
    }
  } else if constexpr (KS == 2) {
    // Two key groups over pairs of tiles.  K slot j holds K tiles 2p, 2p+1
    // of pair p in arrays k(2j), k(2j+1), V slot j likewise in v(2j),
    // v(2j+1); the K pairs run one ahead of the V pairs.  Step s (j = s % 2)
    // passes the barrier (K pair s+1 and V pair s, loaded in step s-1, have
    // landed; every wave is done with step s-1), loads K pair s+2 into K
    // slot j (it held pair s, last read in step s-1) and V pair s+1 into V
    // slot j+1 (it held pair s-1), then runs the tile body on the wave's
    // tile t_lo + 2s + kgrp: its softmax, the scores of its tile two ahead
    // (K pair s+1), P V with V pair s.  Tile indices are relative to t_lo.
    auto load_k_pair = [&](int u0, auto J) {  // tiles t_lo+u0, t_lo+u0+1
      constexpr int j = decltype(J)::value;
      if (t_lo + u0 < t_hi) load_k_tile(kbuf(std::integral_constant<int, 2 * j>{}));
      if (t_lo + u0 + 1 < t_hi) load_k_tile(kbuf(std::integral_constant<int, 2 * j + 1>{}));
    };
    auto load_v_pair = [&](int u0, auto J) {
      constexpr int j = decltype(J)::value;
      if (t_lo + u0 < t_hi) load_v_tile(vbuf(std::integral_constant<int, 2 * j>{}));
      if (t_lo + u0 + 1 < t_hi) load_v_tile(vbuf(std::integral_constant<int, 2 * j + 1>{}));
    };
    // this wave's tile of the pair in slot J
    auto my_k = [&](auto J) -> uint16_t* {
      constexpr int j = decltype(J)::value;
      return kgrp ? kbuf(std::integral_constant<int, 2 * j + 1>{}) : kbuf(std::integral_constant<int, 2 * j>{});
    };
    auto my_v = [&](auto J) -> uint16_t* {
      constexpr int j = decltype(J)::value;
      return kgrp ? vbuf(std::integral_constant<int, 2 * j + 1>{}) : vbuf(std::integral_constant<int, 2 * j>{});
    };
    const int nsteps = (t_hi - t_lo + 1) / 2;
    if (nsteps > 0) {
      load_k_pair(0, I0{});
      load_k_pair(2, I1{});
      load_v_pair(0, I0{});
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      qk(my_k(I0{}), sA);
    }
    auto pstep = [&](int st, auto J, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      constexpr int j = decltype(J)::value;
      using Nx = std::integral_constant<int, (j + 1) & 1>;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      load_k_pair(2 * st + 4, J);
      load_v_pair(2 * st + 2, Nx{});
      const int t = t_lo + 2 * st + kgrp;
      if (live(t)) {
        mask_scores(t, sc);
        tile_body(my_k(Nx{}), my_v(J), sc, sn, st == 0);
      }
    };
    for (int st = 0; st < nsteps; st += 2) {
      pstep(st, I0{}, sA, sB);
      if (st + 1 < nsteps) pstep(st + 1, I1{}, sB, sA);
    }

    // Merge of the two groups by the rescaling rule of the online softmax:
    // with a_g = exp2((m_g - M) c), M = max(m_0, m_1), O = a_0 O_0 + a_1 O_1
    // and l = a_0 l_0 + a_1 l_1 (a group that saw no key has m = -inf,
    // O = 0, l = 0 and weight 0).  Both waves of a row block hold the same
    // rows in the same lanes, so group 1 leaves its accumulators, its
    // denominator shares and m in LDS lane by lane and group 0 combines
    // them.  Accumulator block (db, rb) takes 4 KiB of the K arrays (DP/32
    // blocks per array), as 4 x 64 lanes of 16 bytes (whole 16-byte LDS
    // accesses, consecutive lanes on consecutive banks); the shares (16
    // bytes per lane) and m sit in v(0).
    __syncthreads();  // every wave is done with the ring
    constexpr int per_array = DP / 32;
    auto acc_block = [&](int q) -> float* {
      const int arr = q / per_array, off = (q - arr * per_array) * 1024;
      float* base = arr == 0 ? (float*)kbuf(I0{}) : arr == 1 ? (float*)kbuf(I1{})
                  : arr == 2 ? (float*)kbuf(I2{}) : (float*)kbuf(I3{});
      return base + off;
    };
    float* const mlb = (float*)vbuf(I0{}) + rb * 5 * 64;
    f32x4* const shares = (f32x4*)mlb + lane;
    float* const m_at = mlb + 4 * 64 + lane;
    if (kgrp == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4* blk = (f32x4*)acc_block(db * NWR + rb) + lane;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          blk[e4 * 64] = f32x4{oacc[db][4 * e4], oacc[db][4 * e4 + 1], oacc[db][4 * e4 + 2], oacc[db][4 * e4 + 3]};
      }
      *shares = f32x4{lp[0], lp[1], lp[2], lp[3]};
      *m_at = m_run;
    }
    __syncthreads();
    if (kgrp == 1) return;
    const float m1 = *m_at;
    const float M = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - M) * c);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - M) * c);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4* blk = (const f32x4*)acc_block(db * NWR + rb) + lane;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4 x = blk[e4 * 64];
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][4 * e4 + i] = oacc[db][4 * e4 + i] * a0 + x[i] * a1;
      }
    }
    const f32x4 sh = *shares;
#pragma unroll
    for (int i = 0; i < 4; ++i) lp[i] = lp[i] * a0 + sh[i] * a1;
    m_run = M;
    mc = M == -INFINITY ? 0.f : M * c;
  } else {
    // Four key groups over quads of 32-key tiles, for grids whose one- and
    // two-group shapes leave a SIMD one wave: the workgroup's 8 waves are 2
    // row blocks x 4 groups, two waves per SIMD.  K slot j (of two) holds
    // the K tiles 4p .. 4p+3 of quad p in arrays k(4j) .. k(4j+3), V slot j
    // likewise; the K quads run one ahead of the V quads, step by step as
    // the pairs of two groups do.  Group g takes tile 4s + g of step s.
    auto load_k_quad = [&](int u0, auto J) {  // tiles t_lo+u0 .. t_lo+u0+3
      constexpr int j = decltype(J)::value;
      if (t_lo + u0 < t_hi) load_k_tile(kbuf(std::integral_constant<int, 4 * j>{}));
      if (t_lo + u0 + 1 < t_hi) load_k_tile(kbuf(std::integral_constant<int, 4 * j + 1>{}));
      if (t_lo + u0 + 2 < t_hi) load_k_tile(kbuf(std::integral_constant<int, 4 * j + 2>{}));
      if (t_lo + u0 + 3 < t_hi) load_k_tile(kbuf(std::integral_constant<int, 4 * j + 3>{}));
    };
    auto load_v_quad = [&](int u0, auto J) {
      constexpr int j = decltype(J)::value;
      if (t_lo + u0 < t_hi) load_v_tile(vbuf(std::integral_constant<int, 4 * j>{}));
      if (t_lo + u0 + 1 < t_hi) load_v_tile(vbuf(std::integral_constant<int, 4 * j + 1>{}));
      if (t_lo + u0 + 2 < t_hi) load_v_tile(vbuf(std::integral_constant<int, 4 * j + 2>{}));
      if (t_lo + u0 + 3 < t_hi) load_v_tile(vbuf(std::integral_constant<int, 4 * j + 3>{}));
    };
    // this wave's tile of the quad in slot J (a wave-uniform select)
    auto my_k = [&](auto J) -> uint16_t* {
      constexpr int j = decltype(J)::value;
      uint16_t* const a0 = kbuf(std::integral_constant<int, 4 * j>{});
      uint16_t* const a1 = kbuf(std::integral_constant<int, 4 * j + 1>{});
      uint16_t* const a2 = kbuf(std::integral_constant<int, 4 * j + 2>{});
      uint16_t* const a3 = kbuf(std::integral_constant<int, 4 * j + 3>{});
      return kgrp == 0 ? a0 : kgrp == 1 ? a1 : kgrp == 2 ? a2 : a3;
    };
    auto my_v = [&](auto J) -> uint16_t* {
      constexpr int j = decltype(J)::value;
      uint16_t* const a0 = vbuf(std::integral_constant<int, 4 * j>{});
      uint16_t* const a1 = vbuf(std::integral_constant<int, 4 * j + 1>{});
      uint16_t* const a2 = vbuf(std::integral_constant<int, 4 * j + 2>{});
      uint16_t* const a3 = vbuf(std::integral_constant<int, 4 * j + 3>{});
      return kgrp == 0 ? a0 : kgrp == 1 ? a1 : kgrp == 2 ? a2 : a3;
    };
    const int nsteps = (t_hi - t_lo + 3) / 4;
    if (nsteps > 0) {
      load_k_quad(0, I0{});
      load_k_quad(4, I1{});
      load_v_quad(0, I0{});
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      qk(my_k(I0{}), sA);
    }
    auto qstep = [&](int st, auto J, f32x16 (&sc)[KB], f32x16 (&sn)[KB]) {
      constexpr int j = decltype(J)::value;
      using Nx = std::integral_constant<int, (j + 1) & 1>;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      load_k_quad(4 * st + 8, J);
      load_v_quad(4 * st + 4, Nx{});
      const int t = t_lo + 4 * st + kgrp;
      if (live(t)) {
        mask_scores(t, sc);
        tile_body(my_k(Nx{}), my_v(J), sc, sn, st == 0);
      }
    };
    for (int st = 0; st < nsteps; st += 2) {
      qstep(st, I0{}, sA, sB);
      if (st + 1 < nsteps) qstep(st + 1, I1{}, sB, sA);
    }

    // Merge of the four groups by the same rescaling rule: groups 1-3 leave
    // their accumulators (4 KiB blocks in the ring arrays k0..k7, v1..v7,
    // 16 bytes per lane access), denominator shares and m (mlbuf) in LDS,
    // lane by lane; group 0 takes
    // M = max_g m_g and a_g = exp2((m_g - M) c), O = sum_g a_g O_g and
    // l = sum_g a_g l_g (a group that saw no key has weight 0).
    __shared__ __attribute__((aligned(16))) float mlbuf[3 * NWR * 5 * 64];
    __syncthreads();  // every wave is done with the ring
    constexpr int per_array = TILE * 2 / 4096;  // 4 KiB blocks per ring array
    static_assert(per_array >= 1 && 3 * DB * NWR <= 15 * per_array, "merge blocks fit the ring");
    auto acc_block = [&](int q) -> float* {
      const int arr = q / per_array, off = (q - arr * per_array) * 1024;
      uint16_t* base;
      switch (arr) {
        case 0: base = kbuf(I0{}); break;
        case 1: base = kbuf(I1{}); break;
        case 2: base = kbuf(I2{}); break;
        case 3: base = kbuf(I3{}); break;
        case 4: base = kbuf(std::integral_constant<int, 4>{}); break;
        case 5: base = kbuf(std::integral_constant<int, 5>{}); break;
        case 6: base = kbuf(std::integral_constant<int, 6>{}); break;
        case 7: base = kbuf(std::integral_constant<int, 7>{}); break;
        case 8: base = vbuf(I1{}); break;
        case 9: base = vbuf(I2{}); break;
        case 10: base = vbuf(I3{}); break;
        case 11: base = vbuf(std::integral_constant<int, 4>{}); break;
        case 12: base = vbuf(std::integral_constant<int, 5>{}); break;
        case 13: base = vbuf(std::integral_constant<int, 6>{}); break;
        default: base = vbuf(std::integral_constant<int, 7>{}); break;
      }
      return (float*)base + off;
    };
    // group g's shares (16 bytes per lane) and m
    auto shares = [&](int g) -> f32x4* { return (f32x4*)(mlbuf + ((g - 1) * NWR + rb) * 5 * 64) + lane; };
    auto m_at = [&](int g) -> float* { return mlbuf + ((g - 1) * NWR + rb) * 5 * 64 + 4 * 64 + lane; };
    if (kgrp != 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4* blk = (f32x4*)acc_block(((kgrp - 1) * DB + db) * NWR + rb) + lane;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          blk[e4 * 64] = f32x4{oacc[db][4 * e4], oacc[db][4 * e4 + 1], oacc[db][4 * e4 + 2], oacc[db][4 * e4 + 3]};
      }
      *shares(kgrp) = f32x4{lp[0], lp[1], lp[2], lp[3]};
      *m_at(kgrp) = m_run;
    }
    __syncthreads();
    if (kgrp != 0) return;
    float mo[3];
    float M = m_run;
#pragma unroll
    for (int g = 1; g < 4; ++g) {
      mo[g - 1] = *m_at(g);
      M = fmaxf(M, mo[g - 1]);
    }
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - M) * c);
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= a0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lp[i] *= a0;
#pragma unroll
    for (int g = 1; g < 4; ++g) {
      const float ag = mo[g - 1] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mo[g - 1] - M) * c);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4* blk = (const f32x4*)acc_block(((g - 1) * DB + db) * NWR + rb) + lane;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const f32x4 x = blk[e4 * 64];
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[db][4 * e4 + i] += x[i] * ag;
        }
      }
      const f32x4 sh = *shares(g);
#pragma unroll
      for (int i = 0; i < 4; ++i) lp[i] += sh[i] * ag;
    }
    m_run = M;
    mc = M == -INFINITY ? 0.f : M * c;
  }

  // Epilogue: divide by the row's denominator once, round, store.
  const float l = half_sum((lp[0] + lp[1]) + (lp[2] + lp[3]));
  const float inv = l > 0.f ? 1.f / l : 0.f;
  // log-sum-exp of the scaled scores: ln(sum_j exp(scale*s_j)) =
  // ln 2 * (m*c + log2 l); -inf when the range held no key of the row
  const float lse = l > 0.f ? (mc + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
  if (a.splits > 1) {
    if (qrow < N) {
      const size_t row = ((size_t)split * (a.total_tiles / per_head) + bh) * N + qrow;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * hi;
          const float4 out = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                              oacc[db][4 * g + 3] * inv};
          *(float4*)(a.part_o + row * D + d0) = out;
        }
      if (hi == 0) a.part_lse[row] = lse;
    }
    return;
  }
  if (a.lse != nullptr && qrow < N && hi == 0) a.lse[(size_t)bh * N + qrow] = lse;
  if constexpr (KS == 1 && !CAUSAL) {
    // One key group, no mask: every wave gets here after the same work,
    // and the ring is free once all of them have.  Each wave stages its
    // 32 x D tile of O (16-bit) in a region of the ring, then stores it row
    // by row: each store instruction writes 512 contiguous bytes of a dense
    // O, where storing from the accumulator layout writes 16 bytes into
    // each of 32 rows (8 MB of O by a full grid: 3.0 against 4.6 us).
    // (Causal waves finish at different times; making the early ones wait
    // at the barrier costs more than the stores gain.)
    __syncthreads();
    constexpr int REGION = 32 * D;      // elements per wave
    constexpr int WPA = TILE / REGION;  // regions per ring array
    constexpr int CPR8 = D / 4;         // 8-byte chunks per row
    static_assert(WPA >= 1 && (NW + WPA - 1) / WPA <= 8, "O staging fits the ring");
    const int arr = wave / WPA;
    uint16_t* base = arr == 0 ? kbuf(I0{}) : arr == 1 ? kbuf(I1{}) : arr == 2 ? kbuf(I2{}) : arr == 3 ? kbuf(I3{})
                   : arr == 4 ? vbuf(I0{}) : arr == 5 ? vbuf(I1{}) : arr == 6 ? vbuf(I2{}) : vbuf(I3{});
    base += (wave - arr * WPA) * REGION;
    // 8-byte chunk c8 of row r sits at chunk pchunk(r, c8) of the row: the
    // 32 rows that one write instruction touches (one chunk each) and the
    // rows that one read instruction covers fall on distinct banks
    auto pchunk = [](int r, int c8) {
      if constexpr (D == 64) return c8 ^ ((r >> 1) & 15);
      else if constexpr (D == 96) return (c8 & ~7) | ((c8 ^ (r >> 2)) & 7);
      else return c8 ^ (r & 31);
    };
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // elements 4g..4g+3 are columns 32 db + 8 g + 4 hi .. +3 of row l32
        const int c8 = 8 * db + 2 * g + hi;
        const u32x2 out = {Ops<T>::pack(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                           Ops<T>::pack(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *(u32x2*)(base + 4 * (l32 * CPR8 + pchunk(l32, c8))) = out;
      }
    // the wave's own writes, read back by other lanes of the wave
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < CPR8 / 2; ++i) {
      const int ci = 64 * i + lane, r = ci / CPR8, c8 = ci - r * CPR8;
      const u32x2 v = *(const u32x2*)(base + 4 * (r * CPR8 + pchunk(r, c8)));
      if (q0 + r < N) *(u32x2*)(O + (size_t)(q0 + r) * ldo + 4 * c8) = v;
    }
  } else if (qrow < N) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // elements 4g..4g+3 are columns d0..d0+3 of row qrow
        const int d0 = 32 * db + 8 * g + 4 * hi;
        u32x2 out = {Ops<T>::pack(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                     Ops<T>::pack(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *(u32x2*)(O + (size_t)qrow * ldo + d0) = out;
      }
  }
}

template <typename T, int D, bool CAUSAL, bool SPLIT_P, int NW, int OCC, int KS = 1, int BN = kBlockN>
hipError_t launch_one(const Args& base, int64_t BH, hipStream_t stream) {
  using S = Shape<D, NW, BN>;
  constexpr int BM = 32 * NW / KS;
  Args a = base;
  a.num_qtiles = (a.N + BM - 1) / BM;
  a.total_tiles = (int)(BH * a.num_qtiles * a.splits);
  void* args[] = {&a};
  const bool full = !CAUSAL && a.N % BN == 0;
  const void* kernel = full ? (const void*)fa_forward_kernel<T, D, CAUSAL, SPLIT_P, NW, OCC, KS, BN, !CAUSAL>
                            : (const void*)fa_forward_kernel<T, D, CAUSAL, SPLIT_P, NW, OCC, KS, BN, false>;
  return hipLaunchKernel(kernel, dim3(a.total_tiles), dim3(S::NT), args, 0, stream);
}

inline Args make_args(const Problem& p) {
  Args a;
  a.q = (const uint16_t*)p.q;
  a.k = (const uint16_t*)p.k;
  a.v = (const uint16_t*)p.v;
  a.o = (uint16_t*)p.o;
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.lo = p.lo;
  a.H = p.H;
  a.group = p.group;
  a.N = p.N;
  a.num_qtiles = 0;
  a.total_tiles = 0;
  a.splits = p.splits;
  a.part_o = p.part_o;
  a.part_lse = p.part_lse;
  a.lse = p.lse;
  // A zero (or vanishing) scale becomes 2^-120: the weights stay uniform to
  // within 1e-6 for any finite score, and masked scores (-inf) still give
  // exp2(-inf) = 0 without a special case.
  a.c = fmaxf(__builtin_fabsf(p.scale) * 1.4426950408889634f, 0x1p-120f);
  a.qxor = p.scale < 0.f ? 0x80008000u : 0u;
  return a;
}

// Workgroup shape per head dimension and mask: mfma_waves and mfma_block_n
// (measured on MI355X).  D = 64 causal runs two workgroups per CU (waves_per_eu 2).  With
// two key groups (p.key_groups == 2, chosen by the host for grids that leave
// CUs idle) the workgroup is p.ks_waves waves: 2 or 4 row blocks x 2 key
// groups.  For causal grids the host may name another one-group shape
// (p.waves1, p.block_n1): 32-key tiles at D = 64 and 96, 8 waves at D = 64,
// or 2 or 4 waves with 32-key tiles at D = 128.
template <typename T, bool SPLIT_P>
hipError_t launch(const Problem& p, hipStream_t stream) {
  const Args a = make_args(p);
  if (p.key_groups == 4) {
    // four groups of two 32-row blocks, 32-key tiles (the host's choice for
    // grids whose two-group shape leaves a SIMD one wave)
    switch (p.D) {
      case 64:
        return p.causal ? launch_one<T, 64, true, SPLIT_P, 8, 1, 4, 32>(a, p.BH, stream)
                        : launch_one<T, 64, false, SPLIT_P, 8, 1, 4, 32>(a, p.BH, stream);
      case 96:
        return p.causal ? launch_one<T, 96, true, SPLIT_P, 8, 1, 4, 32>(a, p.BH, stream)
                        : launch_one<T, 96, false, SPLIT_P, 8, 1, 4, 32>(a, p.BH, stream);
      case 128:
        return p.causal ? launch_one<T, 128, true, SPLIT_P, 8, 1, 4, 32>(a, p.BH, stream)
                        : launch_one<T, 128, false, SPLIT_P, 8, 1, 4, 32>(a, p.BH, stream);
      default:
        return hipErrorInvalidValue;
    }
  }
  if (p.key_groups == 2) {
    // the 8-wave shapes the host may choose: non-causal D = 64 and 128,
    // causal at every D
    constexpr int W = mfma_ks_waves;
    const bool w8 = p.ks_waves == 8;
    switch (p.D) {
      case 64:
        if (p.causal)
          return w8 ? launch_one<T, 64, true, SPLIT_P, 8, 1, 2>(a, p.BH, stream)
                    : launch_one<T, 64, true, SPLIT_P, W, mfma_ks_occupancy(64), 2>(a, p.BH, stream);
        return w8 ? launch_one<T, 64, false, SPLIT_P, 8, 1, 2>(a, p.BH, stream)
                  : launch_one<T, 64, false, SPLIT_P, W, mfma_ks_occupancy(64), 2>(a, p.BH, stream);
      case 96:
        if (!p.causal) return launch_one<T, 96, false, SPLIT_P, W, mfma_ks_occupancy(96), 2>(a, p.BH, stream);
        return w8 ? launch_one<T, 96, true, SPLIT_P, 8, 1, 2>(a, p.BH, stream)
                  : launch_one<T, 96, true, SPLIT_P, W, mfma_ks_occupancy(96), 2>(a, p.BH, stream);
      case 128:
        if (p.causal)
          return w8 ? launch_one<T, 128, true, SPLIT_P, 8, 1, 2>(a, p.BH, stream)
                    : launch_one<T, 128, true, SPLIT_P, W, mfma_ks_occupancy(128), 2>(a, p.BH, stream);
        return w8 ? launch_one<T, 128, false, SPLIT_P, 8, 1, 2>(a, p.BH, stream)
                  : launch_one<T, 128, false, SPLIT_P, W, mfma_ks_occupancy(128), 2>(a, p.BH, stream);
      default:
        return hipErrorInvalidValue;
    }
  }
  // the host's causal one-group shapes (p.waves1, p.block_n1)
  if (p.causal && p.D == 64 && p.waves1 == 8 && p.block_n1 == 0)
    return launch_one<T, 64, true, SPLIT_P, 8, 1, 1, 64>(a, p.BH, stream);
  if (p.causal && p.block_n1 == 32) {
    if (p.D == 64 && p.waves1 == 0) return launch_one<T, 64, true, SPLIT_P, 4, 2, 1, 32>(a, p.BH, stream);
    if (p.D == 96 && p.waves1 == 0) return launch_one<T, 96, true, SPLIT_P, 4, 1, 1, 32>(a, p.BH, stream);
    if (p.D == 128 && p.waves1 == 2) return launch_one<T, 128, true, SPLIT_P, 2, 1, 1, 32>(a, p.BH, stream);
    if (p.D == 128 && p.waves1 == 4) return launch_one<T, 128, true, SPLIT_P, 4, 1, 1, 32>(a, p.BH, stream);
    return hipErrorInvalidValue;
  }
  if (p.waves1 != 0 || p.block_n1 != 0) return hipErrorInvalidValue;
  switch (p.D) {
    case 64:
      return p.causal ? launch_one<T, 64, true, SPLIT_P, mfma_waves(64, true), 2>(a, p.BH, stream)
                      : launch_one<T, 64, false, SPLIT_P, mfma_waves(64, false), 1>(a, p.BH, stream);
    case 96:
      return p.causal ? launch_one<T, 96, true, SPLIT_P, mfma_waves(96, true), 1>(a, p.BH, stream)
                      : launch_one<T, 96, false, SPLIT_P, mfma_waves(96, false), 1>(a, p.BH, stream);
    case 128:
      return p.causal
                 ? launch_one<T, 128, true, SPLIT_P, mfma_waves(128, true), 1, 1, mfma_block_n(128, SPLIT_P)>(
                       a, p.BH, stream)
                 : launch_one<T, 128, false, SPLIT_P, mfma_waves(128, false), 1, 1, mfma_block_n(128, SPLIT_P)>(
                       a, p.BH, stream);
    default:
      return hipErrorInvalidValue;
  }
}

#ifdef FA_TILE_SWEEP
// Every workgroup shape of the calibration sweep (the tuning library only):
// (waves per workgroup, waves_per_eu hint, key groups, keys per LDS tile).
// Two workgroups per CU need a 64-element LDS row (D = 64) and four waves per
// workgroup (two waves of two workgroups sit on two SIMDs only); with D = 96
// or 128 one workgroup fills the LDS, so those sizes take the one-workgroup
// shapes only.  128-key tiles take 128 KiB of LDS at D = 64 (one workgroup
// per CU) and do not fit at D = 96 or 128; two key groups take 64-key
// tiles, four take 32-key tiles.
template <typename T, bool SPLIT_P, int D, bool CAUSAL, int BN>
hipError_t launch_shape_bn(const Args& a, int64_t BH, int nw, int occ, int ks, hipStream_t s) {
  if (ks == 1) {
    if (nw == 2 && occ == 1) return launch_one<T, D, CAUSAL, SPLIT_P, 2, 1, 1, BN>(a, BH, s);
    if (nw == 4 && occ == 1) return launch_one<T, D, CAUSAL, SPLIT_P, 4, 1, 1, BN>(a, BH, s);
    if (nw == 8 && occ == 1) return launch_one<T, D, CAUSAL, SPLIT_P, 8, 1, 1, BN>(a, BH, s);
    if constexpr (D == 64 && BN <= 64) {
      if (nw == 4 && occ == 2) return launch_one<T, D, CAUSAL, SPLIT_P, 4, 2, 1, BN>(a, BH, s);
    }
  } else if (ks == 2 && BN == 64) {
    if (nw == 4 && occ == 1) return launch_one<T, D, CAUSAL, SPLIT_P, 4, 1, 2>(a, BH, s);
    if (nw == 8 && occ == 1) return launch_one<T, D, CAUSAL, SPLIT_P, 8, 1, 2>(a, BH, s);
    if constexpr (D == 64) {
      if (nw == 4 && occ == 2) return launch_one<T, D, CAUSAL, SPLIT_P, 4, 2, 2>(a, BH, s);
    }
  } else if (ks == 4 && BN == 32) {
    if (nw == 8 && occ == 1) return launch_one<T, D, CAUSAL, SPLIT_P, 8, 1, 4, 32>(a, BH, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, bool SPLIT_P, int D, bool CAUSAL>
hipError_t launch_shape_d(const Args& a, int64_t BH, int nw, int occ, int ks, int bn, hipStream_t s) {
  switch (bn) {
    case 32: return launch_shape_bn<T, SPLIT_P, D, CAUSAL, 32>(a, BH, nw, occ, ks, s);
    case 64: return launch_shape_bn<T, SPLIT_P, D, CAUSAL, 64>(a, BH, nw, occ, ks, s);
    case 128:
      if constexpr (D == 64) return launch_shape_bn<T, SPLIT_P, D, CAUSAL, 128>(a, BH, nw, occ, ks, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool SPLIT_P>
hipError_t launch_shape(const Problem& p, int nw, int occ, int ks, int bn, hipStream_t s) {
  const Args a = make_args(p);
  switch (p.D) {
    case 64:
      return p.causal ? launch_shape_d<T, SPLIT_P, 64, true>(a, p.BH, nw, occ, ks, bn, s)
                      : launch_shape_d<T, SPLIT_P, 64, false>(a, p.BH, nw, occ, ks, bn, s);
    case 96:
      return p.causal ? launch_shape_d<T, SPLIT_P, 96, true>(a, p.BH, nw, occ, ks, bn, s)
                      : launch_shape_d<T, SPLIT_P, 96, false>(a, p.BH, nw, occ, ks, bn, s);
    case 128:
      return p.causal ? launch_shape_d<T, SPLIT_P, 128, true>(a, p.BH, nw, occ, ks, bn, s)
                      : launch_shape_d<T, SPLIT_P, 128, false>(a, p.BH, nw, occ, ks, bn, s);
    default:
      return hipErrorInvalidValue;
  }
}
#endif

}  // namespace mfma
}  // namespace fa
