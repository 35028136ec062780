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

// How time is split over workgroups: P segments of seg_tiles 32-step tiles
// (the last one shorter).  P = 1 when B * channel groups alone give 512
// workgroups.
struct Plan {
  int64_t P, seg_tiles;
};
inline Plan plan(int64_t B, int64_t T, int64_t D) {
  const int64_t units = B * num_groups(D), nt = num_tiles(T);
  Plan p{1, nt > 0 ? nt : 1};
  if (units >= 512 || nt < 4) return p;
  const int64_t want = (512 + units - 1) / units;
  p.seg_tiles = (nt + want - 1) / want;
  p.P = (nt + p.seg_tiles - 1) / p.seg_tiles;
  return p;
}

struct FwdArgs {
  const float *x, *delta, *A, *Bm, *Cm, *h0;
  float *y, *hT, *ckpt;  // any may be null
  int64_t B, T, D, N;
  int64_t P, seg_tiles;  // the plan
  // P > 1: each segment's local state from zero and its decay product
  // ([P-1, B, D, N] each); scanned in place, Hloc slot p - 1 then holds the
  // state segment p starts from
  float *Hloc, *Aprod;
};

struct BwdArgs {
  const float *x, *delta, *A, *Bm, *Cm, *ckpt, *dy, *dhT;
  float *dx, *ddelta, *dA, *dB, *dC, *dh0;
  float *part;  // [B, groups, T, 2N] per-workgroup sums over its channels of dB, dC
  float *dAp;   // [P, B, D, N] dA per (segment, sequence)
  int64_t B, T, D, N;
  int64_t P, seg_tiles;  // the plan
  // P > 1: per segment q >= 1 the local adjoint at its start (times the
  // first step's decay) and its decay product ([P, B, D, N] each); the
  // reverse scan leaves in Gloc slot p + 1 the adjoint segment p ends with
  float *Gloc, *Aprod;
};

inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t part_bytes(int64_t B, int64_t T, int64_t D, int64_t N) {
  return (size_t)(B * num_groups(D) * T * 2 * N) * sizeof(float);
}
// Workspace of the forward: Hloc and Aprod when time is split, else 0.
inline size_t fwd_ws_bytes(int64_t B, int64_t T, int64_t D, int64_t N) {
  const Plan p = plan(B, T, D);
  return p.P > 1 ? 2 * round256((size_t)((p.P - 1) * B * D * N) * sizeof(float)) : 0;
}
// Workspace of the backward: per-workgroup partials, dA per (segment,
// sequence), Gloc and Aprod when time is split, and, when the forward's
// checkpoints are not given, room for them and for the forward's workspace.
inline size_t bwd_ws_bytes(int64_t B, int64_t T, int64_t D, int64_t N, bool need_ckpt) {
  const Plan p = plan(B, T, D);
  const size_t bdn = (size_t)(B * D * N) * sizeof(float);
  return round256(part_bytes(B, T, D, N)) + round256(p.P * bdn) +
         (p.P > 1 ? 2 * round256(p.P * bdn) : 0) +
         (need_ckpt ? round256(ckpt_bytes(B, T, D, N)) + fwd_ws_bytes(B, T, D, N) : 0);
}

hipError_t fwd_dispatch(const FwdArgs &a, hipStream_t stream);
hipError_t bwd_dispatch(const BwdArgs &a, hipStream_t stream);

}  // namespace sscan
}  // namespace cla
