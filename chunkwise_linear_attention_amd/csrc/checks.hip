// Device-side check of a log-decay tensor: counts the values the chunkwise
// entry points do not accept.  Those calls take the decays on trust (a check
// in every call would cost a pass over the tensor and a synchronization);
// this call lets a caller who cannot vouch for its inputs look first.
//
// What the chunkwise forms allow ("Parallel scan", zerotofrontier.app,
// section "The chunkwise algorithm"; "Lightning Attention-2", Eq. 10): the
// in-chunk decay products are formed as exponentials of differences of
// cumulative log decays, which a NaN or +inf poisons for every later token.
// The scalar form takes l = -inf as an exact reset (a_t = 0); the form with
// one decay per key dimension factors each 16-token block through
// exp(+-cumulative log), which stays bounded only for decays a_t <= 1, i.e.
// l <= 0, and has no reset.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace cla {

namespace {

constexpr int CK_THR = 256;

__global__ __launch_bounds__(1) void zero_counts_kernel(uint32_t *counts) {
  for (int i = 0; i < 4; ++i) counts[i] = 0u;
}

// counts[0] NaN, [1] +inf, [2] finite and > 0, [3] -inf; each workgroup adds
// its own tallies once (integer sums: the result does not depend on order)
__global__ __launch_bounds__(CK_THR) void count_log_decay_kernel(const float *l, int64_t n,
                                                                 uint32_t *counts) {
  __shared__ uint32_t red[4][CK_THR / 64];
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * CK_THR;
  for (int64_t i = (int64_t)blockIdx.x * CK_THR + threadIdx.x; i < n; i += stride) {
    const float x = l[i];
    c[0] += x != x ? 1u : 0u;
    c[1] += x == INFINITY ? 1u : 0u;
    c[2] += (x > 0.f && x < INFINITY) ? 1u : 0u;
    c[3] += x == -INFINITY ? 1u : 0u;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t v = c[k];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[k][w] = v;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    uint32_t v = 0u;
#pragma unroll
    for (int u = 0; u < CK_THR / 64; ++u) v += red[threadIdx.x][u];
    if (v) atomicAdd(counts + threadIdx.x, v);
  }
}

}  // namespace

hipError_t launch_check_log_decay(const float *l, int64_t n, uint32_t *counts,
                                  hipStream_t stream) {
  CLA_LAUNCH("check_log_decay_zero", zero_counts_kernel, dim3(1), dim3(1), stream, counts);
  if (n == 0) return hipSuccess;
  const int64_t want = (n + CK_THR - 1) / CK_THR;
  const unsigned grid = (unsigned)(want < 2048 ? want : 2048);
  CLA_LAUNCH("check_log_decay", count_log_decay_kernel, dim3(grid), dim3(CK_THR), stream, l, n,
             counts);
  return hipSuccess;
}

}  // namespace cla
