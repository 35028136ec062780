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

// log2(e) in fp32: exp(x) = exp2(x * kLog2e)
constexpr float kLog2e = 1.44269504088896341f;

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
// LDS tiles: row-major [rows][NCH 16-byte pieces] (NCH = 8 or 16), the pieces
// of a row XOR-permuted by a 3-bit pattern of the row index:
//   pattern(row) = (row & 3) << 1 | (row >> 2) & 1
// Eight consecutive rows get eight different patterns, so a 16-byte fragment
// read of 8 rows at one piece hits every bank once; four consecutive rows
// (row & 3 = 0..3) get patterns 2k | const, so a transposed read of two
// adjacent pieces in 4 rows does too.  Because the pattern leaves the piece
// index's top bit alone and touches the next two bits only through row & 3,
// a lane's addresses for pieces 2 dt + b, dt = 0..7, take four distinct
// values plus immediates.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int swz_pat(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

template <int NCH>
__device__ __forceinline__ int swz_off(int row, int chunk) {
  static_assert(NCH == 8 || NCH == 16, "row of 8 or 16 pieces");
  return row * (NCH * 16) + ((chunk ^ swz_pat(row)) * 16);
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

// In-chunk decays of one chunk, one token per lane; every wave computes them
// for itself and reads other tokens' values with cross-lane shuffles.  A step
// with l = -inf (a = 0, an exact reset) clears the state before its write:
// its log enters the sums as 0, and the count of resets so far tells which
// tokens it separates, so no -inf is ever formed, added or subtracted.
//   c = finite part of l_1 + .. + l_r (this lane's token r; lanes past the
//       chunk read l = 0), k = resets among steps 1..r
// A segment product a_{r:s} = prod_{s < u <= r} a_u is exp(c_r - c_s) when
// k_r == k_s and 0 otherwise.
struct ChunkDecay {
  float c, c_last;  // this lane's and the chunk's last cumulative log
  int k, k_last;    // this lane's and the chunk's reset count
  bool any;         // the chunk holds a reset (wave-uniform)
};

// x + (the x of the lane DPP control CTRL selects), rows outside ROW_MASK and
// sources outside the row adding 0
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_addf(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, true));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_addi(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum across the 64 lanes by DPP: within every 16-lane row
// by shifts of 1, 2, 4 and 8 lanes, then across rows by the broadcasts of
// lanes 15 and 31 (the cross-lane scan of AMD's GCN documentation); no LDS.
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x = dpp_addf<0x111, 0xF>(x);  // row_shr:1
  x = dpp_addf<0x112, 0xF>(x);  // row_shr:2
  x = dpp_addf<0x114, 0xF>(x);  // row_shr:4
  x = dpp_addf<0x118, 0xF>(x);  // row_shr:8
  x = dpp_addf<0x142, 0xA>(x);  // row_bcast:15 into rows 1, 3
  return dpp_addf<0x143, 0xC>(x);  // row_bcast:31 into rows 2, 3
}
__device__ __forceinline__ int wave_prefix_sum(int x) {
  x = dpp_addi<0x111, 0xF>(x);
  x = dpp_addi<0x112, 0xF>(x);
  x = dpp_addi<0x114, 0xF>(x);
  x = dpp_addi<0x118, 0xF>(x);
  x = dpp_addi<0x142, 0xA>(x);
  return dpp_addi<0x143, 0xC>(x);
}

__device__ __forceinline__ ChunkDecay chunk_decay(float l, int lane) {
  ChunkDecay d;
  const bool rst = l < -3.0e38f;  // -inf
  d.any = __ballot(rst) != 0;
  const float c = wave_prefix_sum(rst ? 0.f : l);
  const int k = d.any ? wave_prefix_sum(rst ? 1 : 0) : 0;
  d.c = c;
  d.k = k;
  d.c_last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c), 63));
  d.k_last = d.any ? __builtin_amdgcn_readlane(k, 63) : 0;
  return d;
}

// The lower-triangular 16 x 16 score tiles (row tile rt >= column tile st) of
// a 64 x 64 chunk, then the two strictly-upper tiles that the k-blocks of 32
// read and that must hold zeros: (0, 1) and (2, 3).  Wave w of NW handles
// tiles w, w + NW, ...
// (Packed 2 bits per tile in an immediate, so that no table is read from
// memory.)  rt: 0,1,1,2,2,2,3,3,3,3,0,2   st: 0,0,1,0,1,2,0,1,2,3,1,3
__device__ __forceinline__ int tile_rt(int t) { return (0x8FFA94u >> (2 * t)) & 3; }
__device__ __forceinline__ int tile_st(int t) { return (0xDE4910u >> (2 * t)) & 3; }

// x = hi + lo to about 2^-16 relative: hi = bf16(x) (round to nearest even),
// lo = bf16(x - hi).  The fp32 value of each hi element is read back from its
// packed pair (a shift or a mask) rather than converted a second time.
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, bf16x8 &hi, bf16x8 &lo) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  hi = cvt8(a, b);
  const u32x4 hw = __builtin_bit_cast(u32x4, hi);
  float r[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x0 = w < 2 ? a[2 * w] : b[2 * w - 4];
    const float x1 = w < 2 ? a[2 * w + 1] : b[2 * w - 3];
    r[2 * w] = x0 - __builtin_bit_cast(float, hw[w] << 16);
    r[2 * w + 1] = x1 - __builtin_bit_cast(float, hw[w] & 0xffff0000u);
  }
  lo = cvt8(r);
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Asynchronous staging: global -> LDS copies that bypass registers
// (global_load_lds, 16 bytes per lane; lane i of a wave writes bytes
// 16 i .. 16 i + 15 of a 1 KB LDS block).  Block b of a row-major swizzled
// [64 x D] tile holds rows RPB b .. RPB b + RPB - 1 (RPB = 64 / (D / 8)); lane
// i lands at row RPB b + i / NCH, physical chunk i % NCH, so it fetches the
// logical chunk (i % NCH) ^ swz_pat(row).  Rows past the chunk's n tokens
// re-read row n - 1 (finite data the kernels mask out).
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;

template <int D>
__device__ __forceinline__ void dma_block(const uint16_t *chunk_src, int n, unsigned char *tile,
                                          int block, int lane) {
  constexpr int NCH = D / 8;
  constexpr int RPB = 64 / NCH;
  const int row = block * RPB + lane / NCH;
  const int c = (lane % NCH) ^ swz_pat(row);
  const int grow = min(row, n - 1);
  __builtin_amdgcn_global_load_lds(chunk_src + (int64_t)grow * D + c * 8,
                                   (lds_void *)(tile + block * 1024), 16, 0, 0);
}

// The global address of the 16 bytes lane `lane` copies for block `block`
// of such a tile (the address dma_block fetches).
template <int D>
__device__ __forceinline__ const uint16_t *bf16_block_src(const uint16_t *chunk_src, int n,
                                                          int block, int lane) {
  constexpr int NCH = D / 8;
  constexpr int RPB = 64 / NCH;
  const int row = block * RPB + lane / NCH;
  const int c = (lane % NCH) ^ swz_pat(row);
  const int grow = min(row, n - 1);
  return chunk_src + (int64_t)grow * D + c * 8;
}

// The same copies as global_load_lds (16 or 4 bytes per lane into an LDS
// block, lane i at byte offset i times the size), issued from inline assembly
// with the block's LDS address passed in M0.  The compiler does not see these
// loads, so it inserts no wait for them: not in front of LDS accesses it
// cannot tell apart from the target (where the builtin gets a vmcnt(0) that
// holds all later work until the copy lands), nor anywhere else.  The caller
// waits (vmcnt(0)) and synchronizes the workgroup before any lane touches the
// target.  Loads the compiler does track stay correctly waited for: vector
// memory operations complete in issue order, so one it does not count only
// makes its counted waits (vmcnt(N)) wait longer.
// (M0 takes the LDS byte address of the block, a wave-uniform value.)
__device__ __forceinline__ void lds_copy16_untracked(const void *src, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_addr)
               : "memory");
}

__device__ __forceinline__ void lds_copy4_untracked(const void *src, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(src), "{m0}"(lds_addr)
               : "memory");
}

__device__ __forceinline__ void lds_copy16_untracked(const void *src, unsigned char *lds_block) {
  lds_copy16_untracked(
      src, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)lds_block));
}

// The LDS byte address of a staging buffer, re-derived behind an empty asm at
// each staging call: the block addresses added to it are then formed next to
// their copies instead of being computed once and kept live (in SGPRs, which
// then spill) across the chunk loop.
__device__ __forceinline__ uint32_t staging_base(const unsigned char *buf) {
  uint32_t x = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void *)buf);
  asm volatile("" : "+s"(x));
  return x;
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
