// Device helpers shared by the chunkwise kernels: bf16 MFMA fragments, LDS
// tile layouts with an XOR swizzle, and the staging of 64-token chunks.
//
// MFMA: v_mfma_f32_16x16x32_bf16 computes C(16x16) += A(16x32) B(32x16).
// Lane l = 16 * lg + li holds
//   A: row li, the 8 k-values of k-group lg;
//   B: column li, the 8 k-values of k-group lg;
//   C: column li, rows 4 * lg + 0..3.
// Only the row/column assignment matters for correctness: A and B pair their
// k-values by (lg, element), so any permutation of k applied to both is
// allowed.  The kernels use that freedom to feed an accumulator tile straight
// back in as an operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cla {
namespace chunk {

constexpr int TC = 64;       // chunk length
constexpr int NWAVE = 4;     // waves per workgroup
constexpr int NTHR = 64 * NWAVE;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950)
__device__ __forceinline__ __bf16 tobf(float x) { return (__bf16)x; }

__device__ __forceinline__ float tof(__bf16 x) { return (float)x; }

__device__ __forceinline__ bf16x8 cvt8(const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = tobf(x[e]);
  return r;
}

__device__ __forceinline__ bf16x8 cvt8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = tobf(lo[e]);
    r[e + 4] = tobf(hi[e]);
  }
  return r;
}

// ---------------------------------------------------------------------------
// LDS tiles.  16-byte chunks of a row are XOR-swizzled with the row index so
// that the 16 lanes of an MFMA fragment read (different rows, same logical
// chunk) hit different banks.
//   row-major tile  [64 tokens][D]   : D/8 chunks per row, swizzle row % (D/8)
//   transposed tile [D][64 tokens]   : 8 chunks per row,   swizzle row % 8
// ---------------------------------------------------------------------------

template <int NCH>
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * (NCH * 16) + ((chunk ^ (row & (NCH - 1))) * 16);
}

template <int NCH>
__device__ __forceinline__ bf16x8 lds_frag(const unsigned char *base, int row, int chunk) {
  return *reinterpret_cast<const bf16x8 *>(base + swz_off<NCH>(row, chunk));
}

// 8 bytes (4 bf16) at element offset `col` (a multiple of 4) of a row
template <int NCH>
__device__ __forceinline__ bf16x4 lds_half(const unsigned char *base, int row, int col) {
  return *reinterpret_cast<const bf16x4 *>(base + swz_off<NCH>(row, col >> 3) + (col & 7) * 2);
}

// ---------------------------------------------------------------------------
// Staging of a [64 x D] bf16 chunk (rows = tokens, row stride D elements in
// global memory; rows >= n are zero).  Thread tid < 2D handles token quad
// sq = tid % 16 (tokens 4sq .. 4sq+3) and column chunk dc = tid / 16
// (columns 8dc .. 8dc+7): four 16-byte global loads.
// ---------------------------------------------------------------------------

template <int D>
struct TileRegs {
  uint4 r[4];
  bool active;
};

template <int D>
__device__ __forceinline__ void tile_load(const uint16_t *src, int n, int tid, TileRegs<D> &t) {
  t.active = tid < 2 * D;
  const int sq = tid & 15, dc = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * sq + i;
    if (t.active && row < n) {
      t.r[i] = *reinterpret_cast<const uint4 *>(src + (int64_t)row * D + dc * 8);
    } else {
      t.r[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// row-major copy: 4 x 16-byte LDS writes
template <int D>
__device__ __forceinline__ void tile_store_rows(unsigned char *dst, int tid, const TileRegs<D> &t) {
  if (!t.active) return;
  const int sq = tid & 15, dc = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4 *>(dst + swz_off<D / 8>(4 * sq + i, dc)) = t.r[i];
}

__device__ __forceinline__ uint32_t bf16_at(const uint4 &v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// transposed copy: for each of the 8 columns, the 4 tokens as one 8-byte write
template <int D>
__device__ __forceinline__ void tile_store_cols(unsigned char *dst, int tid, const TileRegs<D> &t) {
  if (!t.active) return;
  const int sq = tid & 15, dc = tid >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * dc + e;
    const uint32_t lo = bf16_at(t.r[0], e) | (bf16_at(t.r[1], e) << 16);
    const uint32_t hi = bf16_at(t.r[2], e) | (bf16_at(t.r[3], e) << 16);
    *reinterpret_cast<uint2 *>(dst + swz_off<8>(d, sq >> 1) + (sq & 1) * 8) = make_uint2(lo, hi);
  }
}

}  // namespace chunk
}  // namespace cla
