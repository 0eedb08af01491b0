// Internal interface between the C ABI (fa_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One validated forward problem: [BH, N, D] tensors (B and H folded).
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
};

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

// Smallest number of query rows per workgroup of each kernel family: the
// host bounds grid sizes with these (larger blocks only mean fewer
// workgroups).
constexpr int kMfmaBlockM = 128;
constexpr int kF32BlockM = 64;

// Kernel launchers.  Each returns the launch status and touches nothing
// else.  D must be 64, 96 or 128 and N >= 1 (checked by the caller).
hipError_t launch_mfma_f16(const Problem& p, hipStream_t stream);
hipError_t launch_mfma_bf16(const Problem& p, hipStream_t stream);
hipError_t launch_f32(const Problem& p, hipStream_t stream);
hipError_t launch_naive_f16(const NaiveProblem& p, hipStream_t stream);
hipError_t launch_naive_bf16(const NaiveProblem& p, hipStream_t stream);

}  // namespace fa
