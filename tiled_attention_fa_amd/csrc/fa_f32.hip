// FlashAttention forward for fp32 storage, on the vector ALUs (scores in
// fp64, everything else in fp32).
//
// Same tile loop as the matrix-core kernel ("Android Transformer
// Optimization: Attention and Mobile GPU Bottlenecks", section "A Complete
// Tile Loop"): a workgroup owns a block of query rows and walks over all
// key/value tiles; per tile it forms the scores, updates the running maximum
// and denominator, rescales the accumulator by exp(m_old - m_new) and adds
// exp(S - m_new) V; O is divided by the denominator once at the end.
//
// One wave64 per workgroup, one query row per lane: the lane keeps its Q row
// and its O accumulator in registers (D <= 128 floats each).  K and V tiles
// of 32 keys are staged in LDS; every lane reads the same K/V element at the
// same time, which LDS serves as a broadcast.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace f32k {

constexpr int kBlockM = kF32BlockM;  // query rows per workgroup (= lanes)
constexpr int kBlockN = 32;          // keys per LDS tile
constexpr int kXcds = 8;
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  int N;
  int num_qtiles;
  int total_tiles;
  double c;     // |scale| * log2(e)
  float qsign;  // -1 when scale < 0 (exact sign flip of Q), else +1
};

__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int per = total / kXcds, extra = total % kXcds;
  const int x = wg % kXcds, slot = wg / kXcds;
  return x * per + (x < extra ? x : extra) + slot;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBlockM) void fa_forward_f32_kernel(Args a) {
  constexpr int BN = kBlockN;
  static_assert(D % 4 == 0 && D <= 128, "head dim");
  __shared__ __attribute__((aligned(16))) float Ks[BN * D];
  __shared__ __attribute__((aligned(16))) float Vs[BN * D];

  const int tid = threadIdx.x;
  const int logical = xcd_remap(blockIdx.x, a.total_tiles);
  const int bh = logical / a.num_qtiles;
  int qt = logical - bh * a.num_qtiles;
  if (CAUSAL) qt = a.num_qtiles - 1 - qt;
  const int N = a.N;
  const size_t head = (size_t)bh * (size_t)N * D;
  const float* __restrict__ Q = a.q + head;
  const float* __restrict__ K = a.k + head;
  const float* __restrict__ V = a.v + head;
  float* __restrict__ O = a.o + head;
  const double cd = a.c;
  const int qrow = qt * kBlockM + tid;

  float q[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (qrow < N) x = *(const f32x4*)(Q + (size_t)qrow * D + d);
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
  for (int k0 = 0; k0 < kv_end; k0 += BN) {
    __syncthreads();
    for (int idx = tid; idx < BN * D / 4; idx += kBlockM) {
      const int r = idx / (D / 4), c4 = idx - r * (D / 4);
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (k0 + r < N) {
        kx = *(const f32x4*)(K + (size_t)(k0 + r) * D + 4 * c4);
        vx = *(const f32x4*)(V + (size_t)(k0 + r) * D + 4 * c4);
      }
      *(f32x4*)(Ks + r * D + 4 * c4) = kx;
      *(f32x4*)(Vs + r * D + 4 * c4) = vx;
    }
    __syncthreads();

    // Scores in fp64: the products of two fp32 values are exact in fp64 and
    // the D-term sum keeps ~1e-16 relative error, so large logits do not
    // lose absolute precision before the exponential.
    double s[BN];
    double mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      double dot = 0.0;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const f32x4 kx = *(const f32x4*)(Ks + j * D + d);
        dot = __builtin_fma((double)q[d], (double)kx[0], dot);
        dot = __builtin_fma((double)q[d + 1], (double)kx[1], dot);
        dot = __builtin_fma((double)q[d + 2], (double)kx[2], dot);
        dot = __builtin_fma((double)q[d + 3], (double)kx[3], dot);
      }
      const int key = k0 + j;
      if (key >= N || (CAUSAL && key > qrow)) dot = -INFINITY;
      s[j] = dot;
      mx = dot > mx ? dot : mx;
    }
    const double m_new = m_run > mx ? m_run : mx;
    // exp(scale * (s - m)) = exp2(c * (s - m)); the difference is formed in
    // fp64 before rounding to fp32, so its error is relative to |s - m|.
    const float alpha =
        (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((float)((m_run - m_new) * cd));
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
  }

  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (qrow < N) {
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      f32x4 x = {acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
      *(f32x4*)(O + (size_t)qrow * D + d) = x;
    }
  }
}

}  // namespace f32k

hipError_t launch_f32(const Problem& p, hipStream_t stream) {
  using namespace f32k;
  Args a;
  a.q = (const float*)p.q;
  a.k = (const float*)p.k;
  a.v = (const float*)p.v;
  a.o = (float*)p.o;
  a.N = p.N;
  a.num_qtiles = (p.N + kBlockM - 1) / kBlockM;
  a.total_tiles = (int)(p.BH * a.num_qtiles);
  a.c = __builtin_fabs((double)p.scale) * 1.4426950408889634;
  a.qsign = p.scale < 0.f ? -1.f : 1.f;
  void (*kern)(Args) = nullptr;
  if (p.D == 64) kern = p.causal ? fa_forward_f32_kernel<64, true> : fa_forward_f32_kernel<64, false>;
  if (p.D == 96) kern = p.causal ? fa_forward_f32_kernel<96, true> : fa_forward_f32_kernel<96, false>;
  if (p.D == 128) kern = p.causal ? fa_forward_f32_kernel<128, true> : fa_forward_f32_kernel<128, false>;
  if (!kern) return hipErrorInvalidValue;
  void* args[] = {&a};
  return hipLaunchKernel((const void*)kern, dim3(a.total_tiles), dim3(kBlockM), args, 0, stream);
}

}  // namespace fa
