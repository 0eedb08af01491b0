// Merge of split-KV partials.
//
// When the keys of a query block are cut into ranges (one workgroup each),
// every range r leaves a partial result normalised by its own denominator,
// O_r, and the log-sum-exp of its scaled scores, lse_r = m_r + ln l_r.  The
// whole row follows by the rescaling rule of the online softmax ("Android
// Transformer Optimization: Attention and Mobile GPU Bottlenecks", sections
// "The Essence of FlashAttention: Reordering the Computation" and "A
// Complete Tile Loop": partial sums taken against different maxima are
// brought to a common one by exp(m_old - m_new)):
//
//   lse = M + ln sum_r exp(lse_r - M),   M = max_r lse_r
//   O   = sum_r exp(lse_r - lse) O_r
//
// A range that held no visible key of the row has lse_r = -inf, O_r = 0 and
// weight 0.  A row that no range saw (every lse_r = -inf, so the total
// weight L is 0) is written as 0 with lse = -inf, as the fused epilogue
// writes a row whose denominator is 0.
// One thread per 4 consecutive columns of a row; the partials are fp32,
// [splits, rows, D] and [splits, rows].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

namespace fa {
namespace split {

constexpr int kThreads = 256;
constexpr int64_t kMaxWgs = 1 << 20;  // grid cap; the threads stride over the work
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <typename OutT>
__device__ __forceinline__ void store4(void* o, size_t at, f32x4 x) {
  if constexpr (sizeof(OutT) == 4) {
    *(f32x4*)((float*)o + at) = x;
  } else {
    typedef OutT v4 __attribute__((ext_vector_type(4)));
    v4 y;
    y[0] = (OutT)x[0];  // round to nearest even
    y[1] = (OutT)x[1];
    y[2] = (OutT)x[2];
    y[3] = (OutT)x[3];
    *(v4*)((OutT*)o + at) = y;
  }
}

template <typename OutT>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeProblem p) {
  const int G = p.D / 4;
  const int64_t work = p.rows * G;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < work;
       idx += (int64_t)gridDim.x * kThreads) {
    const int64_t row = idx / G;
    const int g = (int)(idx - row * G);
    float M = -INFINITY;
#pragma unroll 4
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.part_lse[s * p.rows + row]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // unrolled so that the loads of several ranges are in flight at once; a
    // range with no visible key (lse_r = -inf, O_r = 0) gets weight 0
#pragma unroll 4
    for (int s = 0; s < p.splits; ++s) {
      const float ls = p.part_lse[s * p.rows + row];
      const f32x4 o = *(const f32x4*)(p.part_o + ((size_t)s * p.rows + row) * p.D + 4 * g);
      const float w = ls == -INFINITY ? 0.f : expf(ls - M);
      L += w;
      acc += w * o;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    store4<OutT>(p.o, (size_t)row * p.D + 4 * g, acc * inv);
    if (p.lse != nullptr && g == 0) p.lse[row] = L > 0.f ? M + logf(L) : -INFINITY;
  }
}

}  // namespace split

hipError_t launch_split_merge(const MergeProblem& p, hipStream_t stream) {
  using namespace split;
  const int64_t work = p.rows * (p.D / 4);
  const int64_t wgs = (work + kThreads - 1) / kThreads < kMaxWgs ? (work + kThreads - 1) / kThreads : kMaxWgs;
  if (wgs == 0) return hipSuccess;
  MergeProblem x = p;
  void* args[] = {&x};
  const void* k = p.dtype == FA_F16    ? (const void*)merge_kernel<_Float16>
                  : p.dtype == FA_BF16 ? (const void*)merge_kernel<__bf16>
                                       : (const void*)merge_kernel<float>;
  return hipLaunchKernel(k, dim3((unsigned)wgs), dim3(kThreads), args, 0, stream);
}

}  // namespace fa
