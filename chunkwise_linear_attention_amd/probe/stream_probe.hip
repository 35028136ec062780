// Streaming probe for the benchmark (not part of libcla's C ABI): the
// diagonal scan backward's memory traffic with none of its arithmetic, to
// measure the HBM rate that traffic pattern reaches on the GPU at hand.
//
// Per element it reads three fp32 arrays and writes two (the backward's
// 3 reads and 2 writes), in the scan kernels' order: a workgroup owns 64
// channels (16 lanes x float4) of one batch row and walks its rows of D
// floats in time; lane = 16 channel lanes x 4 time slots, NW waves, K rows
// per slot per block, all K rows loaded before any is written; workgroups
// are spread over the 8 XCDs as the scan kernels spread them.  Of the orders
// and depths measured (linear grid-stride with 1-8 float4 per array in
// flight, this order at NW x K = 2x1 .. 4x4), NW = 4, K = 2 moved the most
// bytes per second on MI355X.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kNW = 4;
constexpr int kK = 2;

__global__ __launch_bounds__(64 * kNW) void stream_3r2w(const float *a, const float *b,
                                                         const float *c, float *o1, float *o2,
                                                         int64_t T, int64_t D) {
  const int64_t ng = gridDim.x, gpb = D / 64;
  // consecutive workgroup ids go to the 8 XCDs in turn: give each XCD a
  // contiguous range of channel groups (ng is a multiple of 8)
  const int64_t g = (int64_t)(blockIdx.x % 8) * (ng / 8) + blockIdx.x / 8;
  const int64_t row = g / gpb, c0 = (g % gpb) * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cq = lane & 15, s = lane >> 4;
  const int64_t base = row * T * D + c0 + cq * 4;
  for (int64_t t0 = 0; t0 < T; t0 += 4 * kNW * kK) {
    f32x4 x[kK], y[kK], z[kK];
#pragma unroll
    for (int k = 0; k < kK; ++k) {
      const int64_t t = t0 + (w * 4 + s) * kK + k;
      if (t < T) {
        const int64_t off = base + t * D;
        x[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a + off));
        y[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(b + off));
        z[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(c + off));
      }
    }
#pragma unroll
    for (int k = 0; k < kK; ++k) {
      const int64_t t = t0 + (w * 4 + s) * kK + k;
      if (t < T) {
        const int64_t off = base + t * D;
        __builtin_nontemporal_store(x[k] * y[k] + z[k], reinterpret_cast<f32x4 *>(o1 + off));
        __builtin_nontemporal_store(x[k] - z[k], reinterpret_cast<f32x4 *>(o2 + off));
      }
    }
  }
}

}  // namespace

// a, b, c, o1, o2: device arrays of B*T*D fp32 (16-byte aligned), laid out
// [B, T, D].  Requires D % 64 == 0 and B * D / 64 a multiple of 8.  Returns
// 0, -1 for arguments it does not take, or the hipError_t of the launch.
// Launches on `stream`; never allocates or synchronizes.
extern "C" int cla_probe_stream_3r2w(const float *a, const float *b, const float *c, float *o1,
                                     float *o2, int64_t B, int64_t T, int64_t D,
                                     hipStream_t stream) {
  if (!a || !b || !c || !o1 || !o2 || B <= 0 || T <= 0 || D <= 0 || D % 64 != 0 ||
      (B * (D / 64)) % 8 != 0 || B * (D / 64) > 0x7fffffff)
    return -1;
  for (const void *p : {(const void *)a, (const void *)b, (const void *)c, (const void *)o1,
                        (const void *)o2})
    if (reinterpret_cast<uintptr_t>(p) & 15u) return -1;
  hipLaunchKernelGGL(stream_3r2w, dim3((unsigned)(B * (D / 64))), dim3(64 * kNW), 0, stream,
                     a, b, c, o1, o2, T, D);
  return (int)hipGetLastError();
}
