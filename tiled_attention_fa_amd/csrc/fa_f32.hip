// FlashAttention forward for fp32 storage, on the vector ALUs (scores in
// fp64, everything else in fp32).
//
// Same tile loop as the matrix-core kernel ("Android Transformer
// Optimization: Attention and Mobile GPU Bottlenecks", section "A Complete
// Tile Loop"): per tile the scores are formed, the running maximum and
// denominator are updated, the accumulator is rescaled by exp(m_old - m_new)
// and exp(S - m_new) V is added; O is divided by the denominator once at the
// end.
//
// A workgroup owns 64 query rows, one per lane, and has eight waves (four
// for D > 64).  The key tiles (16 keys) are dealt round-robin to the waves:
// each wave keeps its own running maximum, denominator and accumulator for
// the 64 rows over its share of the keys, staging its tiles in an LDS region
// of its own (so the waves never wait for each other inside the loop).  At
// the end the waves' partial results are merged with the same rescaling
// rule: with M the largest of the waves' maxima, O = sum_w exp(m_w - M)
// acc_w / sum_w exp(m_w - M) l_w.  Every K and V element a wave reads is the
// same for all its lanes, which LDS serves as a broadcast.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace f32k {

constexpr int kBlockM = kF32BlockM;  // query rows per workgroup (= lanes)
constexpr int kBlockN = 16;          // keys per tile
// waves per workgroup, each a share of the keys: eight while their merge
// areas (64 rows x D floats each) fit in LDS, else four
template <int D>
constexpr int waves_for() { return D <= 64 ? 8 : 4; }
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

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

// LDS writes of one wave made visible to all its lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, bool CAUSAL, int W = waves_for<D>()>
__global__ __launch_bounds__(kBlockM * W) void fa_forward_f32_kernel(Args a) {
  constexpr int BN = kBlockN;
  constexpr int kWaves = W;
  static_assert((D / W) % 4 == 0, "each wave merges whole 16-byte column groups");
  static_assert(D % 16 == 0 && D <= 128, "head dim");
  // Per wave: a K tile and a V tile; after the loop the same memory holds
  // the waves' accumulators (64 rows x D) for the merge.
  __shared__ __attribute__((aligned(16))) float tiles[kWaves][kBlockM * D];
  __shared__ double m_part[kWaves][kBlockM];
  __shared__ float l_part[kWaves][kBlockM];
  static_assert(3 * BN * D <= kBlockM * D, "tiles fit in the merge area");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // D > 64: K is staged already widened to fp64, each element converted
  // once instead of once per query row (15-16% faster at D = 96 and 128);
  // at D = 64 the doubled LDS reads cost more than the conversions saved
  constexpr bool KW = D > 64;
  float* Ks = tiles[wave];
  [[maybe_unused]] double* Kd = (double*)tiles[wave];
  float* Vs = tiles[wave] + (KW ? 2 : 1) * BN * D;

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
  const int qrow = qt * kBlockM + lane;

  float q[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (qrow < N) x = *(const f32x4*)(Q + (size_t)qrow * ldq + d);
    q[d] = x[0] * a.qsign;
    q[d + 1] = x[1] * a.qsign;
    q[d + 2] = x[2] * a.qsign;
    q[d + 3] = x[3] * a.qsign;
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  double m_run = -INFINITY;
  float l_run = 0.f;

  const int kv_end = CAUSAL ? min(N, qt * kBlockM + kBlockM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  // this workgroup's share of the key tiles (all of them when splits == 1)
  const int t_lo = split * ntiles / a.splits;
  const int t_hi = (split + 1) * ntiles / a.splits;
  for (int t = t_lo + wave; t < t_hi; t += kWaves) {
    const int k0 = t * BN;
    // this wave's tile: 16 rows of K and of V, 16 bytes per lane per load
    for (int idx = lane; idx < BN * D / 4; idx += 64) {
      const int r = idx / (D / 4), c4 = idx - r * (D / 4);
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (k0 + r < N) {
        kx = *(const f32x4*)(K + (size_t)(k0 + r) * ldk + 4 * c4);
        vx = *(const f32x4*)(V + (size_t)(k0 + r) * ldv + 4 * c4);
      }
      if constexpr (KW) {
        *(f64x2*)(Kd + r * D + 4 * c4) = f64x2{(double)kx[0], (double)kx[1]};
        *(f64x2*)(Kd + r * D + 4 * c4 + 2) = f64x2{(double)kx[2], (double)kx[3]};
      } else {
        *(f32x4*)(Ks + r * D + 4 * c4) = kx;
      }
      *(f32x4*)(Vs + r * D + 4 * c4) = vx;
    }
    wave_sync();

    // Scores in fp64: the products of two fp32 values are exact in fp64 and
    // the D-term sum keeps ~1e-16 relative error, so large logits do not
    // lose absolute precision before the exponential.  Two partial sums
    // per key halve the dependent chain.
    double s[BN];
    double mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      double d0 = 0.0, d1 = 0.0;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        f32x4 qx = {q[d], q[d + 1], q[d + 2], q[d + 3]};
        if constexpr (KW) {
          // the widened Q row (2 D registers) would not fit beside the
          // accumulator: an opaque copy keeps its widening per use
          asm volatile("" : "+v"(qx));
          const f64x2 k01 = *(const f64x2*)(Kd + j * D + d);
          const f64x2 k23 = *(const f64x2*)(Kd + j * D + d + 2);
          d0 = __builtin_fma((double)qx[0], k01[0], d0);
          d1 = __builtin_fma((double)qx[1], k01[1], d1);
          d0 = __builtin_fma((double)qx[2], k23[0], d0);
          d1 = __builtin_fma((double)qx[3], k23[1], d1);
        } else {
          const f32x4 kx = *(const f32x4*)(Ks + j * D + d);
          d0 = __builtin_fma((double)qx[0], (double)kx[0], d0);
          d1 = __builtin_fma((double)qx[1], (double)kx[1], d1);
          d0 = __builtin_fma((double)qx[2], (double)kx[2], d0);
          d1 = __builtin_fma((double)qx[3], (double)kx[3], d1);
        }
      }
      double dot = d0 + d1;
      const int key = k0 + j;
      if (key >= N || (CAUSAL && key > qrow)) dot = -INFINITY;
      s[j] = dot;
      mx = dot > mx ? dot : mx;
    }
    const double m_new = m_run > mx ? m_run : mx;
    // exp(scale * (s - m)) = exp2(c * (s - m)); the difference is formed in
    // fp64 before rounding to fp32, so its error is relative to |s - m|.
    // A row with no visible key in this tile keeps m_new = m_run.
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((float)((m_run - m_new) * cd));
    m_run = m_new;
    float pr[BN];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float p = __builtin_amdgcn_exp2f((float)((s[j] - m_new) * cd));
      if (s[j] == -INFINITY) p = 0.f;  // masked; also right when c == 0
      pr[j] = p;
      psum += p;
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const f32x4 vx = *(const f32x4*)(Vs + j * D + d);
        acc[d] = __builtin_fmaf(pr[j], vx[0], acc[d]);
        acc[d + 1] = __builtin_fmaf(pr[j], vx[1], acc[d + 1]);
        acc[d + 2] = __builtin_fmaf(pr[j], vx[2], acc[d + 2]);
        acc[d + 3] = __builtin_fmaf(pr[j], vx[3], acc[d + 3]);
      }
    }
    wave_sync();  // all lanes are done with the tile before the next one lands
  }

  // Merge the waves' partial results.  Each wave publishes its maximum,
  // denominator and accumulator (row-major, 64 rows x D); then each wave
  // merges D / kWaves of the columns for all 64 rows.
  __syncthreads();  // every wave is out of its tile loop (the areas are reused)
  float* accs = tiles[wave];
#pragma unroll
  for (int d = 0; d < D; d += 4)
    *(f32x4*)(accs + lane * D + d) = f32x4{acc[d], acc[d + 1], acc[d + 2], acc[d + 3]};
  m_part[wave][lane] = m_run;
  l_part[wave][lane] = l_run;
  __syncthreads();

  double M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = m_part[w][lane] > M ? m_part[w][lane] : M;
  float f[kWaves];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const double mw = m_part[w][lane];
    f[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((float)((mw - M) * cd));
    L += f[w] * l_part[w][lane];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  // log-sum-exp of the row's scaled scores, ln 2 * (M*c + log2 L); -inf
  // when this key range held no key of the row
  const float lse = L > 0.f ? (float)((M * cd + (double)__builtin_amdgcn_logf(L)) * 0.6931471805599453) : -INFINITY;
  constexpr int DQ = D / kWaves;  // columns merged by this wave
  const bool part = a.splits > 1;
  float* dst = part ? a.part_o + ((size_t)split * (a.total_tiles / per_head) * N + (size_t)bh * N) * D : nullptr;
  if (qrow < N) {
#pragma unroll
    for (int d = 0; d < DQ; d += 4) {
      const int col = wave * DQ + d;
      f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const f32x4 x = *(const f32x4*)(tiles[w] + lane * D + col);
        out += f[w] * x;
      }
      if (part)
        *(f32x4*)(dst + (size_t)qrow * D + col) = out * inv;
      else
        *(f32x4*)(O + (size_t)qrow * ldo + col) = out * inv;
    }
    if (wave == 0) {
      if (part)
        a.part_lse[((size_t)split * (a.total_tiles / per_head) + bh) * N + qrow] = lse;
      else if (a.lse != nullptr)
        a.lse[(size_t)bh * N + qrow] = lse;
    }
  }
}

}  // namespace f32k

namespace {
f32k::Args f32_args(const Problem& p) {
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
  a.num_qtiles = (p.N + kBlockM - 1) / kBlockM;
  a.splits = p.splits;
  a.total_tiles = (int)(p.BH * a.num_qtiles * a.splits);
  a.c = __builtin_fabs((double)p.scale) * 1.4426950408889634;
  a.qsign = p.scale < 0.f ? -1.f : 1.f;
  a.part_o = p.part_o;
  a.part_lse = p.part_lse;
  a.lse = p.lse;
  return a;
}
}  // namespace

hipError_t launch_f32(const Problem& p, hipStream_t stream) {
  using namespace f32k;
  Args a = f32_args(p);
  void (*kern)(Args) = nullptr;
  int waves = 0;
  if (p.D == 64) {
    kern = p.causal ? fa_forward_f32_kernel<64, true> : fa_forward_f32_kernel<64, false>;
    waves = waves_for<64>();
  }
  if (p.D == 96) {
    kern = p.causal ? fa_forward_f32_kernel<96, true> : fa_forward_f32_kernel<96, false>;
    waves = waves_for<96>();
  }
  if (p.D == 128) {
    kern = p.causal ? fa_forward_f32_kernel<128, true> : fa_forward_f32_kernel<128, false>;
    waves = waves_for<128>();
  }
  if (!kern) return hipErrorInvalidValue;
  void* args[] = {&a};
  return hipLaunchKernel((const void*)kern, dim3(a.total_tiles), dim3(kBlockM * waves), args, 0, stream);
}

#ifdef FA_TILE_SWEEP
// The fp32 kernel with the wave count given (the tuning library only): 2, 4
// or 8 waves at D = 64 (8 fill 128 KiB of LDS), 2 or 4 at D = 96 and 128.
hipError_t launch_f32_shape(const Problem& p, int waves, hipStream_t stream) {
  using namespace f32k;
  Args a = f32_args(p);
  void (*kern)(Args) = nullptr;
  if (p.D == 64) {
    if (waves == 2) kern = p.causal ? fa_forward_f32_kernel<64, true, 2> : fa_forward_f32_kernel<64, false, 2>;
    if (waves == 4) kern = p.causal ? fa_forward_f32_kernel<64, true, 4> : fa_forward_f32_kernel<64, false, 4>;
    if (waves == 8) kern = p.causal ? fa_forward_f32_kernel<64, true, 8> : fa_forward_f32_kernel<64, false, 8>;
  } else if (p.D == 96) {
    if (waves == 2) kern = p.causal ? fa_forward_f32_kernel<96, true, 2> : fa_forward_f32_kernel<96, false, 2>;
    if (waves == 4) kern = p.causal ? fa_forward_f32_kernel<96, true, 4> : fa_forward_f32_kernel<96, false, 4>;
  } else if (p.D == 128) {
    if (waves == 2) kern = p.causal ? fa_forward_f32_kernel<128, true, 2> : fa_forward_f32_kernel<128, false, 2>;
    if (waves == 4) kern = p.causal ? fa_forward_f32_kernel<128, true, 4> : fa_forward_f32_kernel<128, false, 4>;
  }
  if (!kern) return hipErrorInvalidValue;
  void* args[] = {&a};
  return hipLaunchKernel((const void*)kern, dim3(a.total_tiles), dim3(kBlockM * waves), args, 0, stream);
}
#endif

}  // namespace fa
