// Chunkwise linear attention with one decay per key dimension (gated linear
// attention), forward pass, for gfx950.
//
// Citations (page title, then section):
//   ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
//
// Recurrence (ZTF "The chunkwise algorithm", the GLA form): row d of the
// state decays by its own a_t[d] = exp(l_t[d]),
//   S_t = diag(a_t) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t.
// Chunks of 64 tokens; inside a chunk c_r[d] = l_1[d] + .. + l_r[d] is summed
// in fp32 over the chunk's own logs only (ZTF "Long products without
// underflow": short windows, no long cumulative sums).  The three segment
// products become per-dimension:
//   scores   A[r, s] = sum_d q_r[d] k_s[d] exp(c_r[d] - c_s[d])   (s <= r)
//   read     O_r    += sum_d q_r[d] exp(c_r[d]) S[d, :]
//   update   S[d, :] = exp(c_n[d]) S[d, :] + sum_s k_s[d] exp(c_n[d] - c_s[d]) v_s
// The scores no longer factor through one matrix product with an elementwise
// mask, and exp(c_r) exp(-c_s) overflows for strong decays.  The chunk is cut
// into four sub-blocks of 16 tokens; with cb_R / ce_R the cumulative logs at
// the start / end of block R (cb_0 = 0, cb_R = ce_{R-1}):
//   Qh[r, d] = q_r[d] exp(c_r[d] - cb_R[d])     (r in block R; factor <= 1)
//   Kh[s, d] = k_s[d] exp(ce_S[d] - c_s[d])     (s in block S; factor <= 1)
// For S < R,  A[r, s] = sum_d Qh[r, d] Kh[s, d] exp(cb_R[d] - ce_S[d]), where
// the last factor (the decay between the two blocks) is <= 1 as well: every
// factor lies in (0, 1], so nothing overflows and a factor that underflows
// only drops a product that is itself below fp32 range.  For S = R the middle
// factor is exp(cb_R - ce_R) >= 1, the inverse of the block's own decay; while
// that decay stays above exp(-60) in every dimension the same product form is
// used (all factors within exp(+-60)); a block whose decay falls below it in
// some dimension has its diagonal scores computed elementwise, exactly, from
// the raw q and k rows.  The read and the update use
//   QL[r, d] = Qh[r, d] exp(cb_R[d]),   KG[s, d] = Kh[s, d] exp(c_n[d] - ce_S[d]),
// both products of factors <= 1.
//
// Workgroup = 4 waves on one (batch*head); wave w owns value columns
// [w DV/4, (w+1) DV/4) of the state, held in MFMA accumulators.  LDS holds the
// chunk's Q, K, V (bf16, swizzled rows) and its log decays (fp32, then the
// cumulative logs), 80 KB at DK = DV = 128, so two workgroups share a CU.
#include "chunk_common.h"
#include "gla_kernels.h"
#include "internal.h"

namespace cla {
namespace gla {

using namespace cla::chunk;

namespace {

// Sub-block whose own decay is below e^-60 in some dimension: its diagonal
// scores are computed elementwise.  (The threshold is in the base-2 units the
// cumulative logs are kept in.)
constexpr float kBadLog = 60.f * kLog2e;

// DMA of the [64 x D] fp32 log tile in the swizzled layout of csx: 1 KB
// blocks of RPB rows; rows past the chunk re-read row n - 1.
template <int D>
__device__ __forceinline__ void dma_f32_block(const float *chunk_src, int n, unsigned char *tile,
                                              int block, int lane) {
  constexpr int PPR = D / 4;     // 16-byte pieces per row
  constexpr int RPB = 64 / PPR;  // rows per 1 KB block
  const int row = block * RPB + lane / PPR;
  const int grow = min(row, n - 1);
  // this lane lands at piece lane % PPR of the row: it fetches the piece the
  // row's swizzle (csx) puts there
  __builtin_amdgcn_global_load_lds(chunk_src + (int64_t)grow * D + (((lane % PPR) ^ (row & 15)) * 4),
                                   (lds_void *)(tile + block * 1024), 16, 0, 0);
}

// value of lane n of this lane's 16-lane row (DPP row_newbcast; n must be a
// compile-time constant once the caller's loops are unrolled)
__device__ __forceinline__ float row_bcast(float v, int n) {
  switch (n) {
#define CLA_RB(N) \
  case N:         \
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N, 0xF, 0xF, false));
    CLA_RB(0) CLA_RB(1) CLA_RB(2) CLA_RB(3) CLA_RB(4) CLA_RB(5) CLA_RB(6) CLA_RB(7)
    CLA_RB(8) CLA_RB(9) CLA_RB(10) CLA_RB(11) CLA_RB(12) CLA_RB(13) CLA_RB(14) CLA_RB(15)
#undef CLA_RB
  }
  return v;
}

// OUT: the full forward over segment blockIdx.y of the plan, from S0 or the
// scanned state of the segments before it.  !OUT: the state pass -- segment
// blockIdx.y (of the first P - 1) from a zero state, writing its local state
// and total decay for the scan across segments.
template <int DK, int DV, bool OUT>
__global__ __launch_bounds__(NTHR, 2) void gla_fwd_kernel(GlaFwdArgs a) {
  constexpr int NJ = DV / 64;   // 16-column tiles of the state per wave
  constexpr int NDT = DK / 16;  // 16-row tiles of the state
  constexpr int NCK = DK / 8, NCV = DV / 8;
  constexpr int B_KS = 64 * DK * 2;
  constexpr int B_VS = B_KS + 64 * DK * 2;
  constexpr int B_CS = B_VS + 64 * DV * 2;
  constexpr int BUF = B_CS + 64 * DK * 4;
  constexpr int NBQ = DK / 8, NBV = DV / 8, NBL = DK / 4;
  constexpr int NBLK = 2 * NBQ + NBV + NBL;
  // Once the scores are formed, the score tile P [64][64] bf16 (8 KB) reuses
  // the first rows of the cumulative logs and the per-block factors the rest
  // of the chunk needs go to rows 50..58 (interior rows of block 3).
  constexpr int P_ROWS = 8192 / (DK * 4);  // rows of the logs P covers
  static_assert(P_ROWS <= 32 && BUF <= 80 * 1024, "LDS layout");
  constexpr int R_FQ = 50, R_FK = 54, R_AL = 58;
  __shared__ __attribute__((aligned(1024))) unsigned char buf[BUF];
  unsigned char *QS = buf;
  unsigned char *KS = buf + B_KS;
  unsigned char *VS = buf + B_VS;
  float *CS = reinterpret_cast<float *>(buf + B_CS);
  unsigned char *PS = buf + B_CS;

  const int tid0 = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  // Lane coordinates are re-derived behind an empty asm at the start of each
  // phase, so that the compiler forms LDS addresses next to their use instead
  // of hoisting them all out of the chunk loop (which exhausts registers).
  int tid = tid0, lane = tid0 & 63, li = lane & 15, lg = lane >> 4;
#define FRESH_LANE()             \
  do {                           \
    int t_ = tid0;               \
    asm volatile("" : "+v"(t_)); \
    tid = t_;                    \
    lane = t_ & 63;              \
    li = lane & 15;              \
    lg = lane >> 4;              \
  } while (0)
  const int64_t bh = blockIdx.x;
  const int64_t seg = blockIdx.y;
  const int64_t T = a.T;
  const int64_t nchunks = (T + TC - 1) / TC;
  const int64_t c_begin = seg * a.seg_chunks;
  const int64_t c_end = min(nchunks, c_begin + a.seg_chunks);
  const int j0 = w * (DV / 4);
  const uint16_t *qh = a.q + bh * T * DK;
  const uint16_t *kh = a.k + bh * T * DK;
  const uint16_t *vh = a.v + bh * T * DV;
  const float *lh = a.l + bh * T * DK;

  // S_acc[dt][jt][i] = S[16 dt + 4 lg + i][j0 + 16 jt + li]
  f32x4 S_acc[NDT][NJ];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) S_acc[dt][jt] = zero4();
  const float *src = !OUT ? nullptr
                     : seg == 0 ? (a.S0 ? a.S0 + bh * DK * DV : nullptr)
                                : a.Sloc + ((seg - 1) * a.nh + bh) * DK * DV;
  if (src) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S_acc[dt][jt][i] = src[(16 * dt + 4 * lg + i) * DV + j0 + 16 * jt + li];
  }

  float lsum = 0.f;  // state pass: the segment's summed log decay of dimension tid

  for (int64_t ci = c_begin; ci < c_end; ++ci) {
    const int64_t t0 = ci * TC;
    const int n = (int)min<int64_t>(TC, T - t0);

    // ---- stage: Q, K, V, l of the chunk into LDS ----
    lds_barrier();  // the previous chunk's LDS reads are done
    FRESH_LANE();
    for (int b = OUT ? w : NBQ + w; b < NBLK; b += NWAVE) {  // the state pass needs no q
      if (b < NBQ)
        dma_block<DK>(qh + t0 * DK, n, QS, b, lane);
      else if (b < 2 * NBQ)
        dma_block<DK>(kh + t0 * DK, n, KS, b - NBQ, lane);
      else if (b < 2 * NBQ + NBV)
        dma_block<DV>(vh + t0 * DV, n, VS, b - 2 * NBQ, lane);
      else
        dma_f32_block<DK>(lh + t0 * DK, n, buf + B_CS, b - 2 * NBQ - NBV, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();

    // ---- cumulative logs, in place ----
    cumsum_rows_dpp<DK, NTHR>(CS, n, tid);
    lds_barrier();

    // ---- Qh, Kh in place (8 elements per step) ----
    FRESH_LANE();
    // each thread takes RPT rows of one 16-row block (one 8-column group), so
    // it reads the block's boundary logs once
    {
      constexpr int RPT = 64 * NCK / NTHR, SPB = 16 / RPT;
      static_assert(RPT * NTHR == 64 * NCK && SPB * RPT == 16, "whole rounds in one block");
      const int c8 = tid % NCK, q = tid / NCK;
      const int B = q / SPB, i0 = q % SPB;
      const int re = 16 * B + 15, rb = 16 * B - 1;  // rb read only when B > 0
      float ce8[8], cb8[8];
      cs_read8<DK>(CS, re, c8, ce8);
      if (B > 0) {
        cs_read8<DK>(CS, rb, c8, cb8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) cb8[e] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int r = 16 * B + i0 + k * SPB;
        const int off = swz_off<NCK>(r, c8);
        float cr8[8];
        cs_read8<DK>(CS, r, c8, cr8);
        bf16x8 kv = *reinterpret_cast<const bf16x8 *>(KS + off);
        float yk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) yk[e] = r < n ? tof(kv[e]) * exp_c(ce8[e] - cr8[e]) : 0.f;
        *reinterpret_cast<bf16x8 *>(KS + off) = cvt8(yk);
        if (OUT) {
          bf16x8 qv = *reinterpret_cast<const bf16x8 *>(QS + off);
          float yq[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) yq[e] = tof(qv[e]) * exp_c(cr8[e] - cb8[e]);
          *reinterpret_cast<bf16x8 *>(QS + off) = cvt8(yq);
        }
      }
    }
    lds_barrier();

    f32x4 sc[3];
    int tR[3], tS[3];
    int ntile = 0;
    if constexpr (OUT) {
    // ---- scores: tile (R, S), S <= R, as acc[i] = A[16R + li][16S + 4lg + i] ----
    // wave w: the diagonal tile (w, w) and the off-diagonal tiles w, w + 4 of
    // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
    {
      const int offR = 0x122333, offS = 0x001012;  // packed (R, S) of the six
      tR[0] = w;
      tS[0] = w;
      ntile = 1;
      for (int t = w; t < 6; t += NWAVE) {
        tR[ntile] = (offR >> (4 * (5 - t))) & 15;
        tS[ntile] = (offS >> (4 * (5 - t))) & 15;
        ++ntile;
      }
    }
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      if (x >= ntile) break;
      FRESH_LANE();
      const int R = tR[x], S = tS[x];
      f32x4 acc = zero4();
      // a diagonal block whose decay falls below e^-60 in some
      // dimension is done elementwise (wave-uniform decision)
      bool exact = false;
      if (R == S) {
        bool bad = false;
        for (int d = lane; d < DK; d += 64) {
          const float cbd = R > 0 ? CS[csx<DK>(16 * R - 1, d)] : 0.f;
          bad |= cbd - CS[csx<DK>(16 * R + 15, d)] > kBadLog;
        }
        exact = __ballot(bad) != 0;
      }
      if (!exact) {
        // The 16 lanes of a row use the same DK / 2 factors exp(cb_R - ce_S)
        // (dimensions 32 kk + 8 lg + e): each lane forms two of them and the
        // row shares them by DPP broadcast.
        float fpair[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int idx = 2 * li + h;  // (kk, e) = (idx / 8, idx % 8)
          const int d = 32 * (idx >> 3) + 8 * lg + (idx & 7);
          if (idx < DK / 4) {
            const float cb = R > 0 ? CS[csx<DK>(16 * R - 1, d)] : 0.f;
            fpair[h] = exp_c(cb - CS[csx<DK>(16 * S + 15, d)]);
          } else {
            fpair[h] = 0.f;
          }
        }
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
          const bf16x8 kv = lds_frag<NCK>(KS, 16 * S + li, 4 * kk + lg);
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            y[e] = tof(kv[e]) * row_bcast((8 * kk + e) & 1 ? fpair[1] : fpair[0], (8 * kk + e) >> 1);
          acc = mfma(cvt8(y), lds_frag<NCK>(QS, 16 * R + li, 4 * kk + lg), acc);
        }
      } else {
        // exact: sum_d q_r[d] k_s[d] exp(c_r[d] - c_s[d]) from the raw rows
        const int r = 16 * R + li;
        const int rr = min(r, n - 1);
        const uint16_t *qrow = qh + (t0 + rr) * DK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * R + 4 * lg + i;
          const uint16_t *krow = kh + (t0 + min(s, n - 1)) * DK;
          float sum = 0.f;
          if (s <= r) {
            for (int d0 = 0; d0 < DK; d0 += 8) {
              const bf16x8 qv = *reinterpret_cast<const bf16x8 *>(qrow + d0);
              const bf16x8 kv = *reinterpret_cast<const bf16x8 *>(krow + d0);
#pragma unroll
              for (int e = 0; e < 8; ++e)
                sum += tof(qv[e]) * tof(kv[e]) *
                       exp_c(CS[csx<DK>(r, d0 + e)] - CS[csx<DK>(s, d0 + e)]);
            }
          }
          acc[i] = sum;
        }
      }
      // causal and chunk-length masks
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * R + li, s = 16 * S + 4 * lg + i;
        if (s > r || s >= n || r >= n) acc[i] = 0.f;
      }
      sc[x] = acc;
    }
    }
    lds_barrier();  // every read of the cumulative logs' interior rows is done

    // ---- per-block factors (from the block-end rows, before P covers them) ----
    FRESH_LANE();
    for (int d = tid; d < DK; d += NTHR) {
      float ce[4];
#pragma unroll
      for (int B = 0; B < 4; ++B) ce[B] = CS[csx<DK>(16 * B + 15, d)];
      const float cl = ce[3];  // the chunk's last cumulative log (rows past n add 0)
      if (!OUT) lsum += cl;
#pragma unroll
      for (int B = 0; B < 4; ++B) {
        CS[(R_FQ + B) * DK + d] = B > 0 ? exp_c(ce[B - 1]) : 1.f;  // exp(cb_B)
        CS[(R_FK + B) * DK + d] = exp_c(cl - ce[B]);
      }
      CS[R_AL * DK + d] = exp_c(cl);
    }
    lds_barrier();
    // KG = Kh (.) exp(c_n - ce_S) and QL = Qh (.) exp(cb_R) in place: the
    // update's and the output's operands, which every wave reads in full
    FRESH_LANE();
    scale_rows_by_block<DK, NTHR>(KS, KS, CS + R_FK * DK, tid);
    if constexpr (OUT) scale_rows_by_block<DK, NTHR>(QS, QS, CS + R_FQ * DK, tid);
    if constexpr (!OUT) lds_barrier();
    if constexpr (OUT) {
    // ---- P[r][s] (bf16) over the first rows of the logs ----
    FRESH_LANE();
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      if (x >= ntile) break;
      const int R = tR[x], S = tS[x];
      bf16x4 pv;
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = tobf(sc[x][i]);
      // P row r = 16R + li, columns 16S + 4lg .. + 3
      *reinterpret_cast<bf16x4 *>(PS + swz_off<8>(16 * R + li, 2 * S + (lg >> 1)) + (lg & 1) * 8) =
          pv;
    }
    // the output reads P in 32-column steps up to the diagonal, which covers
    // the two tiles (0, 1) and (2, 3) above it: they hold zeros
    if (w >= 2) {
      const int R = w == 2 ? 0 : 2;
      const bf16x4 z = {tobf(0.f), tobf(0.f), tobf(0.f), tobf(0.f)};
      *reinterpret_cast<bf16x4 *>(PS + swz_off<8>(16 * R + li, 2 * (R + 1) + (lg >> 1)) +
                                  (lg & 1) * 8) = z;
    }
    lds_barrier();

    // ---- output: O^T[j][r] = (V^T P^T)[j][r] + (S^T QL^T)[j][r] ----
    {
      FRESH_LANE();
      bf16x8 vfrag[NJ][2];
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) vfrag[jt][kb] = tr_frag<NCV>(VS, 32 * kb, j0 + 16 * jt, li, lg);
      bf16x8 sfrag[DK / 32][NJ];
#pragma unroll
      for (int kk = 0; kk < DK / 32; ++kk)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) sfrag[kk][jt] = cvt8(S_acc[2 * kk][jt], S_acc[2 * kk + 1][jt]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int rr = 16 * rt + li;
        bf16x8 qfrag[DK / 32];  // QL^T B operands, k = {32kk + 4lg + 0..3, +16}
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
          const int da = 32 * kk + 4 * lg, db = da + 16;
          qfrag[kk] = cat8(lds_half<NCK>(QS, rr, da), lds_half<NCK>(QS, rr, db));
        }
        bf16x8 pfrag[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) pfrag[kb] = lds_frag<8>(PS, rr, 4 * kb + lg);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < DK / 32; ++kk) acc = mfma(sfrag[kk][jt], qfrag[kk], acc);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            if (kb <= (rt >> 1)) acc = mfma(vfrag[jt][kb], pfrag[kb], acc);
          if (rr < n) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = tobf(acc[i]);
            *reinterpret_cast<bf16x4 *>(a.o + (bh * T + t0 + rr) * DV + j0 + 16 * jt + 4 * lg) = ov;
          }
        }
      }
    }

    }

    // ---- state update: S <- diag(alpha) S + KG^T V ----
    {
      FRESH_LANE();
      const float *al = CS + R_AL * DK;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const f32x4 av = *reinterpret_cast<const f32x4 *>(al + 16 * dt + 4 * lg);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
          for (int i = 0; i < 4; ++i) S_acc[dt][jt][i] *= av[i];
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 vb[NJ];  // V B operands: k = s, column j
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) vb[jt] = tr_frag<NCV>(VS, 32 * kb, j0 + 16 * jt, li, lg);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 ka = tr_frag<NCK>(KS, 32 * kb, 16 * dt, li, lg);  // KG^T: row d, k = s
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) S_acc[dt][jt] = mfma(ka, vb[jt], S_acc[dt][jt]);
        }
      }
    }
  }

  FRESH_LANE();
  if (!OUT) {
    float *dst = a.Sloc + (seg * a.nh + bh) * DK * DV;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(16 * dt + 4 * lg + i) * DV + j0 + 16 * jt + li] = S_acc[dt][jt][i];
    if (tid < DK) a.Aseg[(seg * a.nh + bh) * DK + tid] = exp_c(lsum);
  } else if (a.ST && seg == a.P - 1) {
    float *dst = a.ST + bh * DK * DV;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(16 * dt + 4 * lg + i) * DV + j0 + 16 * jt + li] = S_acc[dt][jt][i];
  }
}

#undef FRESH_LANE

// The state each segment starts from (ZTF "Splitting one sequence across
// devices", with a decay per key dimension): S_in(0) = S0 and
// S_in(p) = diag(A(p-1)) S_in(p-1) + S_loc(p-1), one thread per state entry,
// written over S_loc(p-1) once read.
__global__ __launch_bounds__(256) void gla_segment_scan_kernel(const float *S0, float *Sloc,
                                                               const float *Aseg, int64_t nh,
                                                               int64_t DK, int64_t DV, int64_t P) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= nh * DK * DV) return;
  const int64_t bh = e / (DK * DV), d = (e / DV) % DK;
  float s = S0 ? S0[e] : 0.f;
  for (int64_t p = 1; p < P; ++p) {
    float *slot = Sloc + (p - 1) * nh * DK * DV + e;
    s = Aseg[((p - 1) * nh + bh) * DK + d] * s + *slot;
    *slot = s;
  }
}

template <int DK, int DV>
hipError_t gla_states_impl(const GlaFwdArgs &args, hipStream_t stream) {
  CLA_LAUNCH("gla_fwd_segments", (gla_fwd_kernel<DK, DV, false>),
             dim3((unsigned)args.nh, (unsigned)(args.P - 1)), dim3(NTHR), stream, args);
  const int64_t n = args.nh * DK * DV;
  CLA_LAUNCH("gla_segment_scan", gla_segment_scan_kernel, dim3((unsigned)((n + 255) / 256)),
             dim3(256), stream, args.S0, args.Sloc, args.Aseg, args.nh, (int64_t)DK, (int64_t)DV,
             args.P);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t gla_fwd_impl(const GlaFwdArgs &args, hipStream_t stream) {
  if (args.P > 1) {
    const hipError_t e = gla_states_impl<DK, DV>(args, stream);
    if (e != hipSuccess) return e;
  }
  CLA_LAUNCH("gla_fwd", (gla_fwd_kernel<DK, DV, true>),
             dim3((unsigned)args.nh, (unsigned)args.P), dim3(NTHR), stream, args);
  return hipGetLastError();
}

}  // namespace

GlaPlan plan_gla(int64_t nh, int64_t T) {
  // enough segments to give the GPU about 512 workgroups (two per CU), each
  // a whole number of 16-chunk blocks
  const int64_t nchunks = (T + TC - 1) / TC;
  GlaPlan p{1, nchunks > 0 ? nchunks : 1};
  if (nh >= 512 || nchunks <= kSegChunks) return p;
  const int64_t want = (512 + nh - 1) / nh;
  int64_t seg = (nchunks + want - 1) / want;
  seg = ((seg + kSegChunks - 1) / kSegChunks) * kSegChunks;
  p.seg_chunks = seg;
  p.P = (nchunks + seg - 1) / seg;
  return p;
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t gla_fwd_ws_bytes(int64_t nh, int64_t T, int64_t DK, int64_t DV) {
  const GlaPlan p = plan_gla(nh, T);
  if (p.P <= 1) return 0;
  return round256((size_t)((p.P - 1) * nh * DK * DV) * sizeof(float)) +
         round256((size_t)((p.P - 1) * nh * DK) * sizeof(float));
}

hipError_t gla_fwd_dispatch(const GlaFwdArgs &args, int DK, int DV, hipStream_t stream) {
  if (DK == 64 && DV == 64) return gla_fwd_impl<64, 64>(args, stream);
  if (DK == 64 && DV == 128) return gla_fwd_impl<64, 128>(args, stream);
  if (DK == 128 && DV == 64) return gla_fwd_impl<128, 64>(args, stream);
  if (DK == 128 && DV == 128) return gla_fwd_impl<128, 128>(args, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
}  // namespace cla

namespace cla {
namespace gla {

hipError_t gla_states_dispatch(const GlaFwdArgs &args, int DK, int DV, hipStream_t stream) {
  if (DK == 64 && DV == 64) return gla_states_impl<64, 64>(args, stream);
  if (DK == 64 && DV == 128) return gla_states_impl<64, 128>(args, stream);
  if (DK == 128 && DV == 64) return gla_states_impl<128, 64>(args, stream);
  if (DK == 128 && DV == 128) return gla_states_impl<128, 128>(args, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
}  // namespace cla
