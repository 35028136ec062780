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

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its global loads, stores or LDS DMA in flight (which
// __syncthreads() would drain through its release fence).  For exchanging
// data written with ds_write between waves.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

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

// ---------------------------------------------------------------------------
// Item-level staging: an item is 4 token rows x 8 columns (four 16-byte
// pieces) of a [64 x D] chunk; item ids 0 .. 2D-1, token quad sq = id % 16
// (tokens 4sq .. 4sq+3), column chunk dc = id / 16 (columns 8dc .. 8dc+7).
// Consecutive ids of one wave cover 16 token quads x 4 column chunks.
// ---------------------------------------------------------------------------

// Loads are unconditional (rows past the chunk's n tokens re-read row n-1,
// which exists because n >= 1) so that no load waits on another; the stores
// zero those rows.
template <int D>
__device__ __forceinline__ void item_load(const uint16_t *src, int n, int id, uint4 (&r)[4]) {
  const int sq = id & 15, dc = id >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = min(4 * sq + i, n - 1);
    r[i] = *reinterpret_cast<const uint4 *>(src + (int64_t)row * D + dc * 8);
  }
}

// Same with a run-time row stride D (elements); columns 8 dc .. 8 dc + 7.
__device__ __forceinline__ void item_load_rt(const uint16_t *src, int D, int n, int id,
                                             uint4 (&r)[4]) {
  const int sq = id & 15, dc = id >> 4;
  const uint16_t *p = src + dc * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = min(4 * sq + i, n - 1);
    r[i] = *reinterpret_cast<const uint4 *>(p + (int64_t)row * D);
  }
}

__device__ __forceinline__ void zero_tail(int sq, int n, uint4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (4 * sq + i >= n) r[i] = make_uint4(0u, 0u, 0u, 0u);
}

template <int D>
__device__ __forceinline__ void item_store_rows(unsigned char *dst, int id, int n, uint4 (&r)[4]) {
  const int sq = id & 15, dc = id >> 4;
  zero_tail(sq, n, r);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4 *>(dst + swz_off<D / 8>(4 * sq + i, dc)) = r[i];
}

template <int D>
__device__ __forceinline__ void item_store_cols(unsigned char *dst, int id, int n, uint4 (&r)[4]) {
  const int sq = id & 15, dc = id >> 4;
  zero_tail(sq, n, r);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * dc + e;
    const uint32_t lo = bf16_at(r[0], e) | (bf16_at(r[1], e) << 16);
    const uint32_t hi = bf16_at(r[2], e) | (bf16_at(r[3], e) << 16);
    *reinterpret_cast<uint2 *>(dst + swz_off<8>(d, sq >> 1) + (sq & 1) * 8) = make_uint2(lo, hi);
  }
}

// The lower-triangular 16 x 16 score tiles (row tile rt >= column tile st) of
// a 64 x 64 chunk, then the two strictly-upper tiles that the k-blocks of 32
// read and that must hold zeros: (0, 1) and (2, 3).  Wave w of NW handles
// tiles w, w + NW, ...
// (Packed 2 bits per tile in an immediate, so that no table is read from
// memory.)  rt: 0,1,1,2,2,2,3,3,3,3,0,2   st: 0,0,1,0,1,2,0,1,2,3,1,3
__device__ __forceinline__ int tile_rt(int t) { return (0x8FFA94u >> (2 * t)) & 3; }
__device__ __forceinline__ int tile_st(int t) { return (0xDE4910u >> (2 * t)) & 3; }

// In-chunk cumulative log decay and the three decays, by one wave:
// c_r = l_1 + .. + l_r (rows past the chunk add 0), lambda_r = exp(c_r),
// gamma_r = exp(c_63 - c_r), alpha = exp(c_63).
__device__ __forceinline__ void chunk_decays(float lv, int lane, float *CS, float *LAM,
                                             float *GAM, float *ALPHA) {
  float c = lv;
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    const float p = __shfl_up(c, sh, 64);
    if (lane >= sh) c += p;
  }
  const float cl = __shfl(c, 63, 64);
  CS[lane] = c;
  LAM[lane] = expf(c);
  GAM[lane] = expf(cl - c);
  if (lane == 0) ALPHA[0] = expf(cl);
}

// ---------------------------------------------------------------------------
// Asynchronous staging: global -> LDS copies that bypass registers
// (global_load_lds, 16 bytes per lane; lane i of a wave writes bytes
// 16 i .. 16 i + 15 of a 1 KB LDS block).  Block b of a row-major swizzled
// [64 x D] tile holds rows RPB b .. RPB b + RPB - 1 (RPB = 64 / (D / 8)); lane
// i lands at row RPB b + i / NCH, physical chunk i % NCH, so it fetches the
// logical chunk (i % NCH) ^ (row % NCH).  Rows past the chunk's n tokens
// re-read row n - 1 (finite data the kernels mask out).
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;

template <int D>
__device__ __forceinline__ void dma_block(const uint16_t *chunk_src, int n, unsigned char *tile,
                                          int block, int lane) {
  constexpr int NCH = D / 8;
  constexpr int RPB = 64 / NCH;
  const int row = block * RPB + lane / NCH;
  const int c = (lane % NCH) ^ (row & (NCH - 1));
  const int grow = min(row, n - 1);
  __builtin_amdgcn_global_load_lds(chunk_src + (int64_t)grow * D + c * 8,
                                   (lds_void *)(tile + block * 1024), 16, 0, 0);
}

// ---------------------------------------------------------------------------
// Transposed fragment reads (ds_read_b64_tr_b16).  Within each 16-lane group
// the hardware returns result[i][e] = src[4 e + i / 4][i % 4], where src[j] is
// the 4 elements at lane j's address.  Pointing lane j at row s0 + j / 4,
// columns d0 + 4 (j % 4) .. + 3 of a row-major tile therefore gives lane i the
// column d0 + i for rows s0 .. s0 + 3.
// tr_frag returns, for lane (li, lg), the 8 values X[s0 + 8 lg + e][d0 + li],
// e = 0..7: an MFMA fragment whose k index runs over rows.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int NCH>
__device__ __forceinline__ bf16x4 tr_read4(const unsigned char *tile, int s0, int d0, int li) {
  const int row = s0 + (li >> 2);
  const int col = d0 + 4 * (li & 3);
  const unsigned char *p = tile + swz_off<NCH>(row, col >> 3) + (col & 7) * 2;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
}

template <int NCH>
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char *tile, int s0, int d0, int li,
                                          int lg) {
  const bf16x4 lo = tr_read4<NCH>(tile, s0 + 8 * lg, d0, li);
  const bf16x4 hi = tr_read4<NCH>(tile, s0 + 8 * lg + 4, d0, li);
  return cat8(lo, hi);
}

}  // namespace chunk
}  // namespace cla
