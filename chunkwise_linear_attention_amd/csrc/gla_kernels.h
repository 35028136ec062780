// Argument blocks and launchers of the kernels with one decay per key
// dimension (gla.hip, gla_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "chunk_common.h"

namespace cla {
namespace gla {

// The [64 x DK] fp32 cumulative logs in LDS: row r's 16-byte pieces are
// XOR-swizzled by r & 15 (piece p held at p ^ (r & 15)), so that the 16 rows
// a 16-lane group reads at one column fall in different banks (the plain
// layout put all of them, 512 bytes apart, in the same bank).  Index of
// element (r, d):
template <int DK>
__host__ __device__ __forceinline__ int csx(int r, int d) {
  static_assert(DK >= 64, "at least 16 pieces per row");
  return r * DK + ((((d >> 2) ^ (r & 15)) << 2) | (d & 3));
}

// dst[r][d] = src[r][d] * F[r / 16][d] over a swizzled [64 x DK] bf16 tile
// (dst may be src; F: 4 rows of DK fp32 factors, one per 16-token block), by
// all NTH threads of a workgroup: operands that every wave reads, formed once
// instead of by each wave.
template <int DK, int NTH>
__device__ __forceinline__ void scale_rows_by_block(const unsigned char *src, unsigned char *dst,
                                                    const float *F, int tid) {
  using namespace cla::chunk;
  constexpr int NCK = DK / 8;
  static_assert((64 * NCK) % NTH == 0, "whole rounds");
#pragma unroll
  for (int g0 = 0; g0 < 64 * NCK; g0 += NTH) {
    const int g = g0 + tid;
    const int r = g / NCK, c8 = g % NCK;
    const int off = swz_off<NCK>(r, c8);
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(src + off);
    const f32x4 f0 = *reinterpret_cast<const f32x4 *>(F + (r >> 4) * DK + 8 * c8);
    const f32x4 f1 = *reinterpret_cast<const f32x4 *>(F + (r >> 4) * DK + 8 * c8 + 4);
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[e] = tof(x[e]) * f0[e];
      y[e + 4] = tof(x[e + 4]) * f1[e];
    }
    *reinterpret_cast<bf16x8 *>(dst + off) = cvt8(y);
  }
}

// x + (x of the lane DPP control CTRL selects), rows outside ROW_MASK and
// sources outside the row adding 0
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, true));
}

// exp of a difference of cumulative logs, which the kernels keep in base-2
// units (c log2 e): a single v_exp_f32
__device__ __forceinline__ float exp_c(float x2) { return __builtin_amdgcn_exp2f(x2); }

// The in-chunk cumulative logs, in place in the [64 x DK] fp32 tile (csx
// layout), in base-2 units: c_r[d] = log2(e) * (sum of l_t[d] over t <= r,
// t < n) (rows past the chunk's n tokens repeat its total).  One lane per row: wave w takes the columns
// [w CPW, (w + 1) CPW), reads its row's pieces of them, forms each column's
// inclusive prefix sum across the 64 lanes by DPP (within every 16-lane row by
// shifts of 1, 2, 4 and 8 lanes, then across rows by the broadcasts of lanes 15
// and 31: the cross-lane scan of AMD's GCN documentation), and writes them
// back.  The caller synchronizes the workgroup before and after.
template <int DK, int NTH>
__device__ __forceinline__ void cumsum_rows_dpp(float *CS, int n, int tid) {
  using namespace cla::chunk;
  constexpr int NW = NTH / 64, CPW = DK / NW;  // columns per wave
  static_assert(CPW % 4 == 0 && NW * CPW == DK, "whole 16-byte pieces per wave");
  const int r = tid & 63;
  const int c0 = __builtin_amdgcn_readfirstlane(tid >> 6) * CPW;
  float x[CPW];
#pragma unroll
  for (int p = 0; p < CPW / 4; ++p) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(CS + csx<DK>(r, c0 + 4 * p));
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * p + e] = r < n ? v[e] : 0.f;
  }
#pragma unroll
  for (int c = 0; c < CPW; ++c) x[c] = dpp_add<0x111, 0xF>(x[c]);  // row_shr:1
#pragma unroll
  for (int c = 0; c < CPW; ++c) x[c] = dpp_add<0x112, 0xF>(x[c]);  // row_shr:2
#pragma unroll
  for (int c = 0; c < CPW; ++c) x[c] = dpp_add<0x114, 0xF>(x[c]);  // row_shr:4
#pragma unroll
  for (int c = 0; c < CPW; ++c) x[c] = dpp_add<0x118, 0xF>(x[c]);  // row_shr:8
#pragma unroll
  for (int c = 0; c < CPW; ++c) x[c] = dpp_add<0x142, 0xA>(x[c]);  // row_bcast:15 into rows 1, 3
#pragma unroll
  for (int c = 0; c < CPW; ++c) x[c] = dpp_add<0x143, 0xC>(x[c]);  // row_bcast:31 into rows 2, 3
#pragma unroll
  for (int p = 0; p < CPW / 4; ++p) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x[4 * p + e] * kLog2e;  // base-2 units
    *reinterpret_cast<f32x4 *>(CS + csx<DK>(r, c0 + 4 * p)) = v;
  }
}

// x[e] = the log tile's element (r, 8 c8 + e), e < 8: two 16-byte pieces of
// row r, read as such (the compiler does not see through csx's XOR that each
// group of 4 columns is contiguous, and would read single words)
template <int DK>
__device__ __forceinline__ void cs_read8(const float *CS, int r, int c8, float (&x)[8]) {
  using namespace cla::chunk;
  const f32x4 lo = *reinterpret_cast<const f32x4 *>(CS + csx<DK>(r, 8 * c8));
  const f32x4 hi = *reinterpret_cast<const f32x4 *>(CS + csx<DK>(r, 8 * c8 + 4));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = lo[e];
    x[e + 4] = hi[e];
  }
}

// The backward's decay gradient sums q.dq - k.dk backwards inside blocks of
// this many chunks, each started from the boundary term <S, G>.  Segments of
// the sequence that run on separate workgroups are whole multiples of it.
constexpr int64_t kSegChunks = 16;

// How a sequence is split over workgroups: P segments of seg_chunks chunks
// (the last one shorter).  P = 1 when B*H alone fills the GPU.
struct GlaPlan {
  int64_t P, seg_chunks;
};
GlaPlan plan_gla(int64_t nh, int64_t T);

struct GlaFwdArgs {
  const uint16_t *q, *k;  // [nh, T, DK] bf16
  const uint16_t *v;      // [nh, T, DV] bf16
  const float *l;         // [nh, T, DK] log decays
  const float *S0;        // [nh, DK, DV] or NULL (zeros)
  uint16_t *o;            // [nh, T, DV] bf16
  float *ST;              // [nh, DK, DV] or NULL (not written)
  int64_t nh, T;
  int64_t P, seg_chunks;  // the plan
  // P > 1: each segment's local state from zero (Sloc [P-1, nh, DK, DV]) and
  // total decay (Aseg [P-1, nh, DK]), then, scanned in place, the state each
  // segment starts from (segment p >= 1 reads slot p - 1)
  float *Sloc, *Aseg;
};

// Workspace of the forward: Sloc and Aseg (256-byte aligned), 0 when P = 1.
size_t gla_fwd_ws_bytes(int64_t nh, int64_t T, int64_t DK, int64_t DV);

hipError_t gla_fwd_dispatch(const GlaFwdArgs &args, int DK, int DV, hipStream_t stream);

struct GlaBwdArgs {
  const uint16_t *q, *k;  // [nh, T, DK] bf16
  const uint16_t *v, *dO; // [nh, T, DV] bf16
  const float *l;         // [nh, T, DK] log decays
  const float *S0;        // [nh, DK, DV] or NULL
  const float *dST;       // [nh, DK, DV] or NULL
  uint16_t *dq, *dk;      // [nh, T, DK] bf16
  uint16_t *dv;           // [nh, T, DV] bf16
  float *dl;              // [nh, T, DK]
  float *dS0;             // [nh, DK, DV] or NULL
  float *r1;              // workspace [nh, T, DK]: q (.) dq (fp32, from the dQ pass)
  float *Sseg;            // workspace [nblk, nh, DK, DV]: S at the end of each 16-chunk block
  int64_t nh, T;
  int64_t P, seg_chunks;  // the plan (segments on separate workgroups)
  // P > 1, workspace: the state each segment starts from (slot p - 1 for
  // segment p, from the state pass and its scan); per segment p >= 1 its
  // local adjoint state sum_t diag(A_t) q_t dO_t^T (A_t the decay from the
  // segment's start) and total decay, from the dQ pass, which the reverse
  // scan turns into the adjoint state at each segment's end (slot p + 1 for
  // segment p; the last segment starts from dS_T)
  const float *Sin;
  float *Gloc, *Aq;
};

// Workspace of the backward: r1, Sseg and, for P > 1, the state pass's
// buffers (as the forward's), Gloc [P, nh, DK, DV] and Aq [P, nh, DK], each
// 256-byte aligned.
size_t gla_bwd_ws_bytes(int64_t nh, int64_t T, int64_t DK, int64_t DV);

// The forward's state pass and scan alone (args.Sloc, args.Aseg filled).
hipError_t gla_states_dispatch(const GlaFwdArgs &args, int DK, int DV, hipStream_t stream);

hipError_t gla_bwd_dispatch(const GlaBwdArgs &args, int DK, int DV, hipStream_t stream);

}  // namespace gla
}  // namespace cla
