// Internal interface of the selective-scan kernels (sscan.hip) for the C-ABI
// layer.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cla {
namespace sscan {

constexpr int kChannels = 64;  // channels per workgroup
constexpr int kTile = 32;      // steps per time tile of the forward
constexpr int kCkpt = 16;      // checkpoint interval = steps per tile of the backward

__host__ __device__ inline int64_t num_tiles(int64_t T) { return (T + kTile - 1) / kTile; }
__host__ __device__ inline int64_t num_ckpts(int64_t T) { return (T + kCkpt - 1) / kCkpt; }
__host__ __device__ inline int64_t num_groups(int64_t D) { return (D + kChannels - 1) / kChannels; }

// fp32 states before every 16th step, [B, ceil(T/16), D, N]
inline size_t ckpt_bytes(int64_t B, int64_t T, int64_t D, int64_t N) {
  return (size_t)(B * num_ckpts(T) * D * N) * sizeof(float);
}

struct FwdArgs {
  const float *x, *delta, *A, *Bm, *Cm, *h0;
  float *y, *hT, *ckpt;  // any may be null
  int64_t B, T, D, N;
};

struct BwdArgs {
  const float *x, *delta, *A, *Bm, *Cm, *ckpt, *dy, *dhT;
  float *dx, *ddelta, *dA, *dB, *dC, *dh0;
  float *part;  // [B, groups, T, 2N] per-workgroup sums over its channels of dB, dC
  float *dAp;   // [B, D, N] per-sequence dA
  int64_t B, T, D, N;
};

// Workspace of the backward: per-workgroup partials, per-sequence dA, and
// (when the forward's checkpoints are not given) room for them.
inline size_t part_bytes(int64_t B, int64_t T, int64_t D, int64_t N) {
  return (size_t)(B * num_groups(D) * T * 2 * N) * sizeof(float);
}
inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t bwd_ws_bytes(int64_t B, int64_t T, int64_t D, int64_t N, bool need_ckpt) {
  return round256(part_bytes(B, T, D, N)) + round256((size_t)(B * D * N) * sizeof(float)) +
         (need_ckpt ? round256(ckpt_bytes(B, T, D, N)) : 0);
}

hipError_t fwd_dispatch(const FwdArgs &a, hipStream_t stream);
hipError_t bwd_dispatch(const BwdArgs &a, hipStream_t stream);

}  // namespace sscan
}  // namespace cla
