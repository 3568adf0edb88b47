// Fixed-order sums of per-chunk partial arrays (weight gradients summed
// over many row chunks): two passes that spread the work over the whole
// chip, in an order that does not depend on timing, so the results are
// reproducible.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace e3k {

// Pass 1 of adding n_chunks partial arrays part[c][0..n): the sum of the
// cpg consecutive chunks of group blockIdx.y, in chunk order, written over
// the group's first chunk (which this thread read first).
static __global__ void __launch_bounds__(256)
    k_sum_chunk_groups(int n_chunks, int cpg, int64_t n, float* __restrict__ part) {
  const int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (i >= n) return;
  const int c0 = int(blockIdx.y) * cpg;
  const int c1 = min(n_chunks, c0 + cpg);
  float s = 0.0f;
  for (int c = c0; c < c1; ++c) s += part[int64_t(c) * n + i];
  part[int64_t(c0) * n + i] = s;
}

// Pass 2: out[i] (+)= the group sums in group order.
static __global__ void __launch_bounds__(256)
    k_sum_group_totals(int n_groups, int cpg, int64_t n, const float* __restrict__ part,
                       float* __restrict__ out, int accumulate) {
  const int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (i >= n) return;
  float s = accumulate ? out[i] : 0.0f;
  for (int g = 0; g < n_groups; ++g) s += part[int64_t(g) * cpg * n + i];
  out[i] = s;
}

// out (+)= sum over the n_chunks partials part[c][0..n) in a fixed order
// (groups of 32 chunks, then the groups in order); part is overwritten.
inline hipError_t sum_partials_fixed(int n_chunks, int64_t n, float* part, float* out,
                                     int accumulate, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  constexpr int kCpg = 32;
  const unsigned bx = unsigned((n + 255) / 256);
  const int groups = (n_chunks + kCpg - 1) / kCpg;
  if (groups > 0) {
    hipLaunchKernelGGL(k_sum_chunk_groups, dim3(bx, unsigned(groups)), dim3(256), 0, s, n_chunks,
                       kCpg, n, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_sum_group_totals, dim3(bx), dim3(256), 0, s, groups, kCpg, n, part, out,
                     accumulate);
  return hipGetLastError();
}

}  // namespace e3k
