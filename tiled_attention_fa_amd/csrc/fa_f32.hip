// FlashAttention forward for fp32 storage on the matrix cores: scores in
// fp64 (v_mfma_f64_16x16x4f64: the products of two fp32 values are exact in
// fp64 and the sums run in fp64, so large logits keep their absolute
// precision), the weights P in fp32, and O in fp32 (v_mfma_f32_16x16x4f32).
//
// Same tile loop as the 16-bit kernel ("Android Transformer Optimization:
// Attention and Mobile GPU Bottlenecks", section "A Complete Tile Loop"): per
// tile the scores are formed, the running maximum and denominator are
// updated, the accumulator is rescaled by exp(m_old - m_new) and
// exp(S - m_new) V is added; O is divided by the denominator once at the end.
//
// A workgroup owns 16 * RW query rows (RW waves of 16 rows) in KG key groups
// of RW waves each (KG = 1, 2 or 4); group g takes the key tiles (32 keys)
// g, g + KG, ... and the groups' results are merged at the end by the same
// rescaling rule.  The host takes 64-row workgroups (RW = 4) on grids that
// fill the device and fewer rows in more groups on small ones, so that
// more SIMDs share the rows' chains of key tiles.  A wave
// forms S^T = K Q^T for 16 keys x its 16 rows per block: lane l holds the
// scores of row l & 15 for keys (l >> 4) + 4e, e = 0..3.  Those four scores
// are exactly the P^T operand of the four k-steps of O^T += V^T P^T (k-step e
// takes keys (l >> 4) + 4e of every lane group), so P never moves between
// lanes; V is read from LDS in the matching key order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace f32k {

constexpr int kBlockN = 32;  // keys per LDS tile: two blocks of 16
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

// n consecutive floats from p in 16-byte accesses (p 16-byte aligned).
template <int n>
__device__ __forceinline__ void load_run(const float* p, float (&out)[n]) {
  static_assert(n % 4 == 0, "run length");
#pragma unroll
  for (int i = 0; i < n / 4; ++i) {
    const f32x4 x = *(const f32x4*)(p + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * i + j] = x[j];
  }
}
// Row m (0..15) of O^T block db is head dim 64 i + 4 m + j for db = 4 i + j
// (groups of four blocks), and 64 i + 2 m + j for a last pair of blocks
// (D = 96).  A lane's operands of every block (its row m) are then DB/4
// runs of 4 dims and maybe one of 2, and the 16 lanes of one key row read
// 16 consecutive runs: distinct banks.
template <int DB>
__device__ __forceinline__ void load_vrow(const float* row, int m, float (&out)[DB]) {
#pragma unroll
  for (int i = 0; i < DB / 4; ++i) {
    const f32x4 x = *(const f32x4*)(row + 64 * i + 4 * m);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * i + j] = x[j];
  }
  if constexpr (DB % 4 != 0) {
    const f32x2 x = *(const f32x2*)(row + 64 * (DB / 4) + 2 * m);
    out[DB - 2] = x[0];
    out[DB - 1] = x[1];
  }
}
template <int DB>
__device__ __forceinline__ void store_orow(float* row, int m, const float (&in)[DB]) {
#pragma unroll
  for (int i = 0; i < DB / 4; ++i)
    *(f32x4*)(row + 64 * i + 4 * m) = f32x4{in[4 * i], in[4 * i + 1], in[4 * i + 2], in[4 * i + 3]};
  if constexpr (DB % 4 != 0) *(f32x2*)(row + 64 * (DB / 4) + 2 * m) = f32x2{in[DB - 2], in[DB - 1]};
}

// LDS row pitches (floats).  Lane l reads the K operands of a block as one
// run of D/4 floats of row l & 15 (16-byte reads): a pitch of 4 (mod 64)
// words starts the 16 rows 4 banks apart, so the 16 lanes of one read of
// the run cover all 64 banks.  The V operands are runs within one row per
// 16 lanes (load_vrow); a pitch of 16 (mod 64) words puts the rows that the
// four lane groups read on different banks.  D = 96 takes the D = 128
// pitches.
template <int D>
constexpr int k_pitch() { return D <= 64 ? 68 : 132; }
template <int D>
constexpr int v_pitch() { return D <= 64 ? 80 : 144; }

struct Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  Layout lq, lk, lv, lo;  // element strides of each tensor
  int H;                  // query heads per batch
  int group;              // query heads per key/value head
  int N;
  int num_qtiles;
  int total_tiles;  // BH * num_qtiles * splits
  double c;         // |scale| * log2(e)
  float qsign;      // -1 when scale < 0 (exact sign flip of Q), else +1
  int splits;       // key-range splits per query block (1: O written directly)
  float* part_o;    // splits > 1: [splits, BH, N, D] normalised partial O
  float* part_lse;  // splits > 1: [splits, BH, N] partial log-sum-exp
  float* lse;       // splits == 1, optional: [BH, N] log-sum-exp
};

__device__ __forceinline__ double lanes_max(double x) {  // over lanes l, l ^ 16, l ^ 32, l ^ 48
  x = fmax(x, __shfl_xor(x, 16));
  return fmax(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float lanes_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// LDS of a workgroup: a K tile and a V tile (padded rows) per key group;
// after the loop the same bytes carry groups 1 .. KG-1's O, m and
// denominator shares (lane by lane) to group 0.
template <int D, int RW, int KG>
struct Smem {
  static constexpr int NT = 64 * RW;  // threads of one key group
  static constexpr int K_FLOATS = KG * kBlockN * k_pitch<D>();
  static constexpr int TILES = 4 * (K_FLOATS + KG * kBlockN * v_pitch<D>());
  static constexpr int MO = 0;                               // f32x4 [KG-1][D/16][NT]
  static constexpr int MM = MO + (KG - 1) * (D / 16) * NT * 16;  // double [KG-1][NT]
  static constexpr int ML = MM + (KG - 1) * NT * 8;           // float [KG-1][NT]
  static constexpr int MERGE = ML + (KG - 1) * NT * 4;
  static constexpr int BYTES = TILES > MERGE ? TILES : MERGE;
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// 64-row workgroups at D = 64 are held to 128 VGPRs, four waves per SIMD, so
// that two 8-wave workgroups fit on a CU (full grids run that way).
template <int D, int RW>
constexpr int f32_waves_per_eu() { return D == 64 && RW == 4 ? 4 : 1; }

template <int D, bool CAUSAL, int RW, int KG>
__global__ __launch_bounds__(64 * RW * KG) __attribute__((amdgpu_waves_per_eu(f32_waves_per_eu<D, RW>())))
void fa_forward_f32_kernel(Args a) {
  constexpr int BN = kBlockN, PK = k_pitch<D>(), PV = v_pitch<D>();
  constexpr int BM = 16 * RW;         // query rows per workgroup
  constexpr int NT = 64 * RW;         // threads of one key group
  constexpr int DS = D / 4;           // k-steps of S^T = K Q^T (4 head dims each)
  constexpr int DB = D / 16;          // 16-column blocks of O
  constexpr int CH = BN * D / 4 / NT; // 16-byte loads per thread, operand and tile
  using Lds = Smem<D, RW, KG>;
  static_assert(RW == 1 || RW == 2 || RW == 4, "row waves");
  static_assert(KG == 1 || KG == 2 || KG == 4, "key groups");
  static_assert(D % 32 == 0 && D <= 128 && CH * NT * 4 == BN * D, "head dim");
  __shared__ __attribute__((aligned(16))) char smem[Lds::BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int kgrp = KG == 1 ? 0 : wave / RW;  // key group
  const int rw = wave - kgrp * RW;           // 16-row block
  const int gtid = tid - kgrp * NT;                 // thread within the key group
  const int c16 = lane & 15, lg = lane >> 4;

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
  const float* __restrict__ Q = a.q + b * a.lq.sb + h * a.lq.sh;
  const float* __restrict__ K = a.k + b * a.lk.sb + hk * a.lk.sh;
  const float* __restrict__ V = a.v + b * a.lv.sb + hk * a.lv.sh;
  float* __restrict__ O = a.o + b * a.lo.sb + h * a.lo.sh;
  const int ldq = a.lq.sn, ldk = a.lk.sn, ldv = a.lv.sn, ldo = a.lo.sn;  // row strides
  const double cd = a.c;
  const int q0 = qt * BM + 16 * rw;  // first query row of this wave
  const int row = q0 + c16;               // this lane's query row

  // Q^T operand: k-step s takes head dims DS j + s, j = 0..3; lane l holds
  // row q0 + (l & 15), dim DS (l >> 4) + s, so that each lane's DS dims are
  // one contiguous run; widened to fp64 once (exact).
  double qd[DS];
  {
    float qr[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = 0.f;
    if (row < N) load_run(Q + (size_t)row * ldq + DS * lg, qr);
#pragma unroll
    for (int s = 0; s < DS; ++s) qd[s] = (double)(qr[s] * a.qsign);
  }

  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  double m_run = -INFINITY;  // running maximum of the raw scores of the row
  float l_part = 0.f;        // this lane's share of the row's denominator

  const int kv_end = CAUSAL ? min(N, qt * BM + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  // this workgroup's share of the key tiles (all of them when splits == 1)
  const int t_lo = split * ntiles / a.splits;
  const int t_hi = (split + 1) * ntiles / a.splits;

  // Tile t of the key group: loaded by its threads into registers (16 bytes
  // each, zero past key N), then stored to the group's LDS tile.
  float* const Ks = (float*)smem + kgrp * BN * PK;              // this group's K tile
  float* const Vs = (float*)smem + Lds::K_FLOATS + kgrp * BN * PV;  // and V tile
  f32x4 kr[CH], vr[CH];
  auto fetch = [&](int t) {
    const int k0 = t * BN;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = i * NT + gtid, r = idx / (D / 4), c4 = idx - r * (D / 4);
      kr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      vr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k0 + r < N) {
        kr[i] = *(const f32x4*)(K + (size_t)(k0 + r) * ldk + 4 * c4);
        vr[i] = *(const f32x4*)(V + (size_t)(k0 + r) * ldv + 4 * c4);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = i * NT + gtid, r = idx / (D / 4), c4 = idx - r * (D / 4);
      *(f32x4*)(&Ks[r * PK + 4 * c4]) = kr[i];
      *(f32x4*)(&Vs[r * PV + 4 * c4]) = vr[i];
    }
  };

  auto tile = [&](int t) {
    const int k0 = t * BN;
    const float* ks = Ks;
    const float* vs = Vs;
    // S^T for the two 16-key blocks: element e of block kb is the score of
    // key k0 + 16 kb + (l >> 4) + 4e against this lane's row
    double sc[2][4];
    double mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // the K operand in the Q operand's dim order: one contiguous run
      float kr_[DS];
      load_run(ks + (16 * kb + c16) * PK + DS * lg, kr_);
      f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int s = 0; s < DS; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kr_[s], qd[s], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = k0 + 16 * kb + lg + 4 * e;
        sc[kb][e] = (key >= N || (CAUSAL && key > row)) ? -INFINITY : acc[e];
        mx = fmax(mx, sc[kb][e]);
      }
    }
    const double m_new = fmax(m_run, lanes_max(mx));
    // exp(scale (s - m)) = exp2(c (s - m)), the difference formed in fp64
    // before rounding to fp32; a row with no visible key so far keeps -inf
    const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((float)((m_run - m_new) * cd));
    m_run = m_new;
    float p[2][4];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[kb][e] = sc[kb][e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((float)((sc[kb][e] - m_new) * cd));
        ps += p[kb][e];
      }
    l_part = l_part * alpha + ps;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    // O^T += V^T P^T: k-step (kb, e) takes keys 16 kb + j + 4e, j = 0..3,
    // the j-th from lane group j, which holds it as its element e (lane l
    // supplies row m = l & 15 of every block, load_vrow's dims)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float vr_[DB];
        load_vrow(vs + (16 * kb + lg + 4 * e) * PV, c16, vr_);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr_[db], p[kb][e], o[db], 0, 0, 0);
      }
  };

  // Every key group runs the same number of steps, so the barriers match.
  const int steps = (t_hi - t_lo + KG - 1) / KG;
  int t = t_lo + kgrp;
  if (t < t_hi) fetch(t);
  for (int st = 0; st < steps; ++st, t += KG) {
    __syncthreads();  // every wave is done with the previous tiles
    if (t < t_hi) stash();
    __syncthreads();
    if (t + KG < t_hi) fetch(t + KG);
    // a causal tile whose first key lies past the wave's last row holds
    // nothing for it
    if (t < t_hi && (!CAUSAL || t * BN <= q0 + 15)) tile(t);
  }

  if constexpr (KG > 1) {
    // groups 1 .. KG-1 leave O, m and their denominator shares in LDS, lane
    // by lane (16-byte accesses), over the tiles once every group is done
    // with them; group 0 merges by the rescaling rule
    f32x4* const mo = (f32x4*)(smem + Lds::MO);
    double* const mm = (double*)(smem + Lds::MM);
    float* const ml = (float*)(smem + Lds::ML);
    __syncthreads();
    if (kgrp > 0) {
      const int j = kgrp - 1;
#pragma unroll
      for (int db = 0; db < DB; ++db) mo[(j * DB + db) * NT + gtid] = o[db];
      mm[j * NT + gtid] = m_run;
      ml[j * NT + gtid] = l_part;
    }
    __syncthreads();
    if (kgrp > 0) return;
    double M = m_run;
#pragma unroll
    for (int j = 0; j < KG - 1; ++j) M = fmax(M, mm[j * NT + gtid]);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((float)((m_run - M) * cd));
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= a0;
    l_part *= a0;
#pragma unroll
    for (int j = 0; j < KG - 1; ++j) {
      const double mj = mm[j * NT + gtid];
      const float aj = mj == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((float)((mj - M) * cd));
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] += mo[(j * DB + db) * NT + gtid] * aj;
      l_part += ml[j * NT + gtid] * aj;
    }
    m_run = M;
  }

  // Epilogue: the row's denominator over the four lane groups, one
  // reciprocal; O^T element r of every block is row m = 4 (l >> 4) + r of
  // the blocks, store_orow's dims of O[row].
  const float L = lanes_sum(l_part);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  // log-sum-exp of the row's scaled scores, ln 2 * (M*c + log2 L); -inf
  // when this key range held no key of the row
  const float lse = L > 0.f ? (float)((m_run * cd + (double)__builtin_amdgcn_logf(L)) * 0.6931471805599453) : -INFINITY;
  const bool part = a.splits > 1;
  if (row < N) {
    float* dst = part ? a.part_o + ((size_t)split * (a.total_tiles / per_head) + bh) * N * D + (size_t)row * D
                      : O + (size_t)row * ldo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float run[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) run[db] = o[db][r] * inv;
      store_orow(dst, 4 * lg + r, run);
    }
    if (lg == 0) {
      if (part)
        a.part_lse[((size_t)split * (a.total_tiles / per_head) + bh) * N + row] = lse;
      else if (a.lse != nullptr)
        a.lse[(size_t)bh * N + row] = lse;
    }
  }
}

}  // namespace f32k

namespace {
f32k::Args f32_args(const Problem& p, int block_m) {
  using namespace f32k;
  Args a;
  a.q = (const float*)p.q;
  a.k = (const float*)p.k;
  a.v = (const float*)p.v;
  a.o = (float*)p.o;
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.lo = p.lo;
  a.H = p.H;
  a.group = p.group;
  a.N = p.N;
  a.num_qtiles = (p.N + block_m - 1) / block_m;
  a.splits = p.splits;
  a.total_tiles = (int)(p.BH * a.num_qtiles * a.splits);
  a.c = __builtin_fabs((double)p.scale) * 1.4426950408889634;
  a.qsign = p.scale < 0.f ? -1.f : 1.f;
  a.part_o = p.part_o;
  a.part_lse = p.part_lse;
  a.lse = p.lse;
  return a;
}

template <int RW, int KG>
hipError_t launch_f32_groups(const Problem& p, hipStream_t stream) {
  using namespace f32k;
  Args a = f32_args(p, 16 * RW);
  void (*kern)(Args) = nullptr;
  switch (p.D) {
    case 64: kern = p.causal ? fa_forward_f32_kernel<64, true, RW, KG> : fa_forward_f32_kernel<64, false, RW, KG>; break;
    case 96: kern = p.causal ? fa_forward_f32_kernel<96, true, RW, KG> : fa_forward_f32_kernel<96, false, RW, KG>; break;
    case 128:
      kern = p.causal ? fa_forward_f32_kernel<128, true, RW, KG> : fa_forward_f32_kernel<128, false, RW, KG>;
      break;
    default: return hipErrorInvalidValue;
  }
  void* args[] = {&a};
  return hipLaunchKernel((const void*)kern, dim3(a.total_tiles), dim3(64 * RW * KG), args, 0, stream);
}

// The workgroup shapes: (waves per key group, key groups).  More than one
// key group only with one key range (splits == 1).
hipError_t launch_f32_rw_kg(const Problem& p, int row_waves, int key_groups, hipStream_t stream) {
  if (key_groups > 1 && p.splits != 1) return hipErrorInvalidValue;
  switch (row_waves * 8 + key_groups) {
    case 4 * 8 + 1: return launch_f32_groups<4, 1>(p, stream);
    case 4 * 8 + 2: return launch_f32_groups<4, 2>(p, stream);
    case 2 * 8 + 2: return launch_f32_groups<2, 2>(p, stream);
    case 2 * 8 + 4: return launch_f32_groups<2, 4>(p, stream);
    case 1 * 8 + 4: return launch_f32_groups<1, 4>(p, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

// The host's shape (p.f32_row_waves, p.key_groups); split ranges run the
// 64-row one-group shape.
hipError_t launch_f32(const Problem& p, hipStream_t stream) {
  if (p.splits != 1) return launch_f32_groups<4, 1>(p, stream);
  return launch_f32_rw_kg(p, p.f32_row_waves, p.key_groups, stream);
}

#ifdef FA_TILE_SWEEP
// The fp32 kernel with the shape given (the tuning library only).
hipError_t launch_f32_shape(const Problem& p, int row_waves, int key_groups, hipStream_t stream) {
  return launch_f32_rw_kg(p, row_waves, key_groups, stream);
}
#endif

}  // namespace fa
