// Internal declarations shared by the C-ABI layer (api.cpp) and the kernel
// translation units.  Not part of the public interface (include/cla.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cla {

// Kernel timing hooks (no-ops unless cla_timing_enable(1) was called).
namespace timing {
void before(hipStream_t stream);
void after(hipStream_t stream, const char *name);
void cancel(hipStream_t stream);  // drop the start event of a failed launch
}  // namespace timing

// Launch a kernel between the timing hooks and return the launch error, if
// any, from the enclosing function (which returns hipError_t) before anything
// else is enqueued, so that no later call can hide it.
#define CLA_LAUNCH(name, kernel, grid, block, stream, ...)                       \
  do {                                                                           \
    ::cla::timing::before(stream);                                               \
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);             \
    const hipError_t cla_launch_err_ = hipGetLastError();                       \
    if (cla_launch_err_ != hipSuccess) {                                         \
      ::cla::timing::cancel(stream);                                             \
      return cla_launch_err_;                                                    \
    }                                                                            \
    ::cla::timing::after(stream, name);                                          \
  } while (0)

// ---------------------------------------------------------------------------
// diagonal scan
// ---------------------------------------------------------------------------

// How a diagonal scan is split over the GPU.  Channels are grouped 64 at a
// time (16 lanes x float4); each group sweeps the whole time axis unless the
// batch and channel count alone give too few groups, in which case the time
// axis is cut into P segments whose composed pairs go through the workspace.
struct ScanPlan {
  int64_t P = 1;         // segments along time
  int64_t seg_len = 0;   // steps per segment (multiple of the block length)
  size_t ws_bytes = 0;   // workspace bytes (P - 1 pairs per channel)
};

ScanPlan plan_scan(int64_t B, int64_t T, int64_t D);

hipError_t launch_scan_fwd(const float *a, const float *b, const float *h0,
                           float *h, float *hT, int64_t B, int64_t T,
                           int64_t D, const ScanPlan &plan, void *ws,
                           hipStream_t stream);

hipError_t launch_scan_bwd(const float *a, const float *h, const float *h0,
                           const float *dh, const float *dhT, float *da,
                           float *db, float *dh0, int64_t B, int64_t T,
                           int64_t D, const ScanPlan &plan, void *ws,
                           hipStream_t stream);

// Bytes of the fixed device array behind launch_scan_fwd_noalloc (the
// largest workspace plan_scan can ask for fits in it).
constexpr size_t kScanNoAllocScratchBytes = 262144;

// launch_scan_fwd with the segment pairs in the library's fixed device array
// instead of a workspace (on the current device; no allocation).
hipError_t launch_scan_fwd_noalloc(const float *a, const float *b, const float *h0,
                                   float *h, float *hT, int64_t B, int64_t T,
                                   int64_t D, const ScanPlan &plan,
                                   hipStream_t stream);

// counts[0..3] = the numbers of NaN, +inf, finite positive and -inf values
// among l[0..n) (counts zeroed by a kernel of its own first).
hipError_t launch_check_log_decay(const float *l, int64_t n, uint32_t *counts,
                                  hipStream_t stream);

// dst[i] = src ? src[i] : 0 for i < n (empty-sequence final states).
hipError_t launch_copy_or_zero(float *dst, const float *src, int64_t n,
                               hipStream_t stream);

// ---------------------------------------------------------------------------
// chunkwise linear attention
// ---------------------------------------------------------------------------

struct ChunkPlan {
  int64_t P = 1;            // forward: segments along time per (batch, head)
  int64_t seg_chunks = 0;   // forward: chunks per segment
  int64_t P_b = 1;          // backward: segments (at most kMaxBwdSegChunks each)
  int64_t seg_chunks_b = 0; // backward: chunks per segment
  size_t ws_fwd = 0;        // workspace bytes, forward
  size_t ws_bwd = 0;        // workspace bytes, backward
  size_t saved_bytes = 0;   // states at the backward's segment ends (P_b - 1 of them)
};

ChunkPlan plan_chunk(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV);

// The chunk kernels run on a grid (B*H, segments): at most 2^31 - 1
// sequence-heads and 65535 segments (T up to 16 * 65535 chunks of 64 tokens).
inline bool chunk_plan_launchable(const ChunkPlan &plan, int64_t nh) {
  return nh <= 0x7fffffff && plan.P <= 65535 && plan.P_b <= 65535;
}

// saved (optional): receives S after every plan.seg_chunks_b chunks, the
// states the backward's segments start from ([P_b - 1, B*H, DK, DV]).
hipError_t launch_chunk_fwd(const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const float *l,
                            const float *S0, uint16_t *o, float *ST,
                            float *saved, int64_t B, int64_t H, int64_t T,
                            int64_t DK, int64_t DV, const ChunkPlan &plan,
                            void *ws, hipStream_t stream);

// saved (optional): the states written by launch_chunk_fwd; the dQ pass then
// starts its segments from them instead of recomputing them.
hipError_t launch_chunk_bwd(const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const float *l,
                            const float *S0, const uint16_t *dO,
                            const float *dST, const float *saved, uint16_t *dq,
                            uint16_t *dk, uint16_t *dv, float *dl, float *dS0,
                            int64_t B, int64_t H, int64_t T, int64_t DK,
                            int64_t DV, const ChunkPlan &plan, void *ws,
                            hipStream_t stream);

}  // namespace cla
