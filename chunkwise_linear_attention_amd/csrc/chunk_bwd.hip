// Chunkwise linear attention, backward pass: the reverse-order dK/dV kernel,
// which also forms the decay gradient, for gfx950.  The dQ pass is the forward
// kernel run on (dO, V, K) (chunk.hip).
//
// Citations (page title, then section / equation):
//   ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
//   LA2 = "Lightning Attention-2: A Free Lunch for Handling Unlimited
//         Sequence Lengths in Large Language Models" (paper-graph-ui summary)
//
// ZTF "The backward pass of linear attention": the adjoint state obeys the
// reverse recurrence Sbar_t = q_t dO_t^T + a_{t+1} Sbar_{t+1}; keys and values
// get kbar_t = Sbar_t v_t and vbar_t = Sbar_t^T k_t.  Chunkwise, with G the
// gradient of the state after chunk j (LA2 Eq. 17, 19, 20 with the index
// convention of the per-token Eq. 12):
//   dV_[j] = (Q K^T (.) D)^T dO + diag(gamma) K G
//   dK_[j] = (dO V^T (.) D)^T Q + diag(gamma) V G^T
//   G     <- alpha G + (diag(lambda) Q)^T dO       (state gradient entering j)
// with the same in-chunk decays as the forward.  Chunks run last to first.
//
// Workgroup = 8 waves on one (batch*head, segment).  Waves 0-3 ("dV side")
// each own the columns [w DV/4, (w+1) DV/4) of G in fp32 MFMA accumulators;
// waves 4-7 ("dK side") each own the columns [w' DK/4, (w'+1) DK/4) of G^T.
// Both copies are updated every chunk from the same bf16 operands, so each
// side feeds its state straight back as an MFMA operand without an LDS round
// trip.  The dK side also forms r2_s = k_s . dk_s (fp32, before rounding) for
// the decay gradient.
//
// Decay gradient (ZTF "The backward pass of linear attention", the closed
// form after Yang et al. 2023 Sec. 4.3): dl_u = sum_{t >= u} (q_t . dq_t -
// k_t . dk_t), plus <S_T, dS_T> on every u when the final state has a
// gradient (every path into the final state crosses every step).  A reverse
// cumulative sum per sequence, accumulated in fp64.
#include "chunk_common.h"
#include "chunk_kernels.h"
#include "internal.h"

namespace cla {
namespace chunk {

namespace {

constexpr int BTHR = 512;

// dK, dV, the decay gradient and dS0 of one segment, starting from the G at its end (dS_T
// for the last segment; the segment-local G states come from the dQ pass).
// At DK = DV = 64 two workgroups (16 waves) share a CU, four waves per SIMD:
// the register budget is then 128 per lane.
template <int DK, int DV>
__global__ __launch_bounds__(BTHR, (DK == 64 && DV == 64) ? 4 : 2) void chunk_bwd_kernel(
    BwdArgs a) {
  constexpr int NJ = DV / 64;   // dV side: 16-col tiles of G per wave
  constexpr int NI = DK / 64;   // dK side: 16-col tiles of G^T per wave
  constexpr int NCK = DK / 8, NCV = DV / 8;
  constexpr int RK = 64 * DK * 2, RV = 64 * DV * 2;  // row-major tile bytes
  // Two staging buffers, each [Q | dO | K | V] (the log decays go to
  // registers):
  // the next chunk streams into one by DMA while the other is being used.
  // The copies are issued untracked: with the builtin the compiler waited for
  // the whole DMA at the first score-tile write (it cannot tell the score
  // tiles from the DMA target); the step waits for it at its end instead.
  constexpr int B_DOS = RK;
  constexpr int B_KS = B_DOS + RV;
  constexpr int B_VS = B_KS + RK;
  constexpr int BUF = B_VS + RV;
  // 1 KB DMA blocks per chunk
  constexpr int NBQ = DK / 8, NBD = DV / 8;
  constexpr int NBK = DK / 8, NBV = DV / 8;
  constexpr int NBLK = NBQ + NBD + NBK + NBV;
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[BUF];
  // P1[s][r] = D_rs (q_r . k_s), P2[s][r] = D_rs (dO_r . v_s)
  __shared__ __attribute__((aligned(1024))) unsigned char P1[64 * 128];
  __shared__ __attribute__((aligned(1024))) unsigned char P2[64 * 128];
  // The per-wave k.dk partials of a chunk, R2P[u][s] (u = dK-side wave),
  // live in score-tile pieces that no tile uses: rows s >= 32 of P2, logical
  // pieces 0-3 (the tiles (r, s) with r < 32 <= s are structurally zero and
  // neither written nor read).  With the decays in registers this keeps
  // DK = DV = 64 at 80 KB of LDS, two workgroups per CU.
  auto r2p_at = [&](int u, int s_) __attribute__((always_inline)) -> float * {
    const int idx = u * 64 + s_;  // 0..255: 16-byte piece idx / 4, word idx % 4
    const int q = idx >> 2;
    return reinterpret_cast<float *>(P2 + swz_off<8>(32 + (q >> 2), q & 3) + 4 * (idx & 3));
  };
  auto r2p_sum = [&](int s_) __attribute__((always_inline)) -> float {
    return *r2p_at(0, s_) + *r2p_at(1, s_) + *r2p_at(2, s_) + *r2p_at(3, s_);
  };
  // The same pieces of P1 (never written by a score tile either) hold the
  // chunk's per-token values TOK[u][t] (u = 0: base-2 cumulative log, 1:
  // lambda), written by every wave (the same values) at the start of a step,
  // so that lanes needing 4 or 8 consecutive tokens read them as 16-byte
  // pieces instead of one cross-lane shuffle per token.
  auto tok_at = [&](int u, int t_) __attribute__((always_inline)) -> float * {
    const int idx = u * 64 + t_;
    const int q = idx >> 2;
    return reinterpret_cast<float *>(P1 + swz_off<8>(32 + (q >> 2), q & 3) + 4 * (idx & 3));
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  int li = lane & 15, lg = lane >> 4;
  // Re-derive the lane coordinates behind an empty asm at the start of each
  // phase, so that the compiler forms LDS addresses next to their use instead
  // of hoisting all of them out of the chunk loop (which exhausts registers).
#define FRESH_LANE()                   \
  do {                                 \
    int l_ = lane;                     \
    asm volatile("" : "+v"(l_));       \
    li = l_ & 15;                      \
    lg = l_ >> 4;                      \
  } while (0)
  // a lane-dependent value re-derived behind an empty asm, like FRESH_LANE,
  // so that the 64-bit addresses built from it are formed at their use and
  // not kept live (or spilled) across the chunk loop
  auto fresh = [](int x) __attribute__((always_inline)) {
    asm volatile("" : "+v"(x));
    return x;
  };
  const int side = w >> 2, wv = w & 3;   // side 0: dV / G;  side 1: dK / G^T
  // grid (nh, segments): both indices are workgroup ids, held in scalar
  // registers, so every pointer derived from them stays wave-uniform
  const int64_t bh = blockIdx.x;
  const int64_t seg = blockIdx.y;
  const int64_t T = a.T;
  const int64_t nchunks = (T + TC - 1) / TC;
  const int64_t c_begin = seg * a.seg_chunks;
  const int64_t c_end = min(nchunks, c_begin + a.seg_chunks);
  const int jw0 = wv * (DV / 4);  // side 0: first column j of this wave
  const int dw0 = wv * (DK / 4);  // side 1: first column d of G^T

  const uint16_t *qh = a.q + bh * T * DK;
  const uint16_t *kh = a.k + bh * T * DK;
  const uint16_t *vh = a.v + bh * T * DV;
  const uint16_t *doh = a.dO + bh * T * DV;
  const float *lh = a.l + bh * T;

  // One register array holds either side's state (both have DK*DV/1024
  // tiles of 16 x 16):
  //   side 0: Gs[dt * NJ + jt][i] = G[16 dt + 4 lg + i][jw0 + 16 jt + li]
  //   side 1: Gs[jt * NI + it][i] = G^T[16 jt + 4 lg + i][dw0 + 16 it + li]
  constexpr int NG = DK * DV / 1024;
  static_assert((DK / 16) * NJ == NG && (DV / 16) * NI == NG, "state tiles");
  f32x4 Gs[NG];
#define G0(dt, jt) Gs[(dt) * NJ + (jt)]
#define G1(jt, it) Gs[(jt) * NI + (it)]
  {
    const float *src = nullptr;
    if (seg == a.P - 1) {
      src = a.dST ? a.dST + bh * DK * DV : nullptr;
    } else {
      src = a.Gin + (seg * a.nh + bh) * DK * DV;
    }
#pragma unroll
    for (int x = 0; x < NG; ++x) Gs[x] = zero4();
    if (src) {
      if (side == 0) {
#pragma unroll
        for (int dt = 0; dt < DK / 16; ++dt)
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              G0(dt, jt)[i] = src[(16 * dt + 4 * lg + i) * DV + jw0 + 16 * jt + li];
      } else {
#pragma unroll
        for (int jt = 0; jt < DV / 16; ++jt)
#pragma unroll
          for (int it = 0; it < NI; ++it)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              G1(jt, it)[i] = src[(dw0 + 16 * it + li) * DV + 16 * jt + 4 * lg + i];
      }
    }
  }
  double dl_carry = 0.0;  // wave 0: the decay gradient's running suffix sum
  {
    // Boundary term of the decay gradient: <S, G> at this segment's end, from
    // the fp32 state S^T that the dQ pass held at that boundary (S_T^T for
    // the last segment) and the G just loaded; the read runs along rows
    // (coalesced) through the G^T side, whose copy has the state's layout.
    const bool last = seg == a.P - 1;
    const float *St = last ? (a.STb ? a.STb + bh * DK * DV : nullptr)
                           : a.Sseg + (seg * a.nh + bh) * DK * DV;
    double part = 0.0;
    if (St && side == 1) {
      float pf = 0.f;
#pragma unroll
      for (int jt = 0; jt < DV / 16; ++jt)
#pragma unroll
        for (int it = 0; it < NI; ++it)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pf += G1(jt, it)[i] * St[(16 * jt + 4 * lg + i) * DK + dw0 + 16 * it + li];
      part = pf;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    // (P1 holds no score tile before the chunk loop)
    double *bred = reinterpret_cast<double *>(P1);
    if (lane == 0) bred[w] = part;
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) dl_carry += bred[u];
    }
  }
  int64_t r2_t0 = -1;  // chunk whose k.dk partials sit in the P2 spare pieces
  int r2_n = 0;
  // wave 0: q.dq of the staged chunk (one token per lane), and of the chunk
  // whose decay gradient is formed next
  float r1_next = 0.f, r1_prev = 0.f;

  // Decay gradient of one chunk by wave 0, token t on lane t:
  //   dl_t = carry + sum_{u >= t in the chunk} (r1_u - r2_u),
  // r1 = q.dq (the dQ pass), r2 = k.dk (this pass); the chunk's total then
  // joins the carry, which starts at <S, G> at the segment's end (the sum over
  // all paths that cross it) and runs backwards through the segment's chunks.
  // fp64 accumulation throughout.
  auto chunk_dl = [&](float r1, float r2, int nrows) __attribute__((always_inline)) -> float {
    double sfx = lane < nrows ? (double)r1 - (double)r2 : 0.0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double y = __shfl_down(sfx, o, 64);
      if (lane + o < 64) sfx += y;
    }
    const float out = (float)(dl_carry + sfx);
    dl_carry += __shfl(sfx, 0, 64);
    return out;
  };

  // DMA of chunk cj into a staging buffer: 1 KB row blocks spread over the
  // waves; every wave loads the chunk's log decays, one per lane, into a
  // register for the step that computes the chunk.
  float l_next = 0.f;
  auto stage = [&](int64_t cj, unsigned char *buf) __attribute__((always_inline)) {
    const int64_t tj = cj * TC;
    const int nj = (int)min<int64_t>(TC, T - tj);
    // the per-lane DMA addresses are formed here, at each stage, instead of
    // being kept live (one 64-bit pair per staged tensor) across the loop
    const int ln = fresh(lane);
    const uint32_t lb = staging_base(buf);
    // wave w takes blocks w, w + 8, ...; every tensor's block count is a
    // multiple of 8, so the tensor of each round is known at compile time
    constexpr int NW = BTHR / 64;
    static_assert(NBQ % NW == 0 && NBD % NW == 0 && NBK % NW == 0 && NBV % NW == 0, "rounds");
#pragma unroll
    for (int r0 = 0; r0 < NBLK; r0 += NW) {
      const int b = w + r0;
      // (untracked copies: the step waits for them at its end)
      if (r0 < NBQ) {
        lds_copy16_untracked(bf16_block_src<DK>(qh + tj * DK, nj, b, ln), lb + b * 1024);
      } else if (r0 < NBQ + NBD) {
        lds_copy16_untracked(bf16_block_src<DV>(doh + tj * DV, nj, b - NBQ, ln),
                             lb + B_DOS + (b - NBQ) * 1024);
      } else if (r0 < NBQ + NBD + NBK) {
        lds_copy16_untracked(bf16_block_src<DK>(kh + tj * DK, nj, b - NBQ - NBD, ln),
                             lb + B_KS + (b - NBQ - NBD) * 1024);
      } else {
        lds_copy16_untracked(bf16_block_src<DV>(vh + tj * DV, nj, b - NBQ - NBD - NBK, ln),
                             lb + B_VS + (b - NBQ - NBD - NBK) * 1024);
      }
    }
    // this lane's log decay, used when the chunk is computed (rows past the
    // chunk read l = 0 there)
    l_next = ln < nj ? lh[tj + ln] : 0.f;
    if (w == 0) r1_next = ln < nj ? a.r1[bh * T + tj + ln] : 0.f;
  };

  // One chunk from staging buffer `cur`, while the chunk before it streams
  // into `nxt` (released by the barrier that ended the previous step).
  auto step = [&](int64_t ci, unsigned char *cur, unsigned char *nxt)
                  __attribute__((always_inline)) {
    const int64_t t0 = ci * TC;
    const int n = (int)min<int64_t>(TC, T - t0);
    unsigned char *QS = cur;
    unsigned char *DOS = cur + B_DOS;
    unsigned char *KS = cur + B_KS;
    unsigned char *VS = cur + B_VS;
    const float l_cur = l_next;
    const float r1_cur = r1_next;

    if (ci > c_begin) stage(ci - 1, nxt);
    // the previous chunk's k.dk sums (complete; this step overwrites them):
    // its decay gradient is formed and stored at the end of the step, where
    // wave 0's side waits for the other (a store issued here would also hold
    // its data register while the DMA is in flight)
    const int64_t dl_row = r2_t0;
    const int dl_n = r2_n;
    const float r2_prev = w == 0 && r2_t0 >= 0 && lane < r2_n ? r2p_sum(lane) : 0.f;
    // In-chunk decays, one token per lane, computed by every wave (lanes
    // are then read with cross-lane shuffles).  Rows past the chunk: no
    // decay, and lambda = 0 so that they add nothing to the state gradient.
    const ChunkDecay dc = chunk_decay(l_cur, lane);
    const float c_l = dc.c;
    const float c2_l = c_l * kLog2e;  // base-2 cumulative log
    const float lam_l = lane < n && dc.k == 0 ? expf(c_l) : 0.f;
    const float gam_l = dc.k == dc.k_last ? expf(dc.c_last - c_l) : 0.f;
    const float alpha = dc.k_last == 0 ? expf(dc.c_last) : 0.f;
    *tok_at(0, lane) = c2_l;
    *tok_at(1, lane) = lam_l;

    {
      // ---- masked score tiles, stored transposed: P[s][r] ----
      FRESH_LANE();
      {
        unsigned char *PT = side == 0 ? P1 : P2;
        // A whole chunk without resets needs no mask below the diagonal
        // tiles (r > s there); the decay factor is exp2 of a difference of
        // base-2 cumulative logs.
        const bool plain = n == TC && !dc.any;
#pragma unroll 1
        for (int tt = 0; tt < 3; ++tt) {
          const int t = wv + 4 * tt;
          const int rt = tile_rt(t), st = tile_st(t);
          const int s = 16 * st + li;
          f32x4 acc = zero4();
          if (rt >= st) {
            if (side == 0) {
#pragma unroll
              for (int kk = 0; kk < DK / 32; ++kk)
                acc = mfma(lds_frag<NCK>(QS, 16 * rt + li, 4 * kk + lg),
                           lds_frag<NCK>(KS, s, 4 * kk + lg), acc);
            } else {
#pragma unroll
              for (int kk = 0; kk < DV / 32; ++kk)
                acc = mfma(lds_frag<NCV>(DOS, 16 * rt + li, 4 * kk + lg),
                           lds_frag<NCV>(VS, s, 4 * kk + lg), acc);
            }
          }
          // acc[i] = X[r = 16 rt + 4 lg + i][s]; rows past the chunk are masked
          const float cs = __shfl(c2_l, s, 64);
          // base-2 cumulative logs of this lane's 4 rows r = 16 rt + 4 lg + i
          const f32x4 c2r = *reinterpret_cast<const f32x4 *>(tok_at(0, 16 * rt + 4 * lg));
          bf16x4 pv;
          if (plain && rt > st) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pv[i] = tobf(acc[i] * __builtin_amdgcn_exp2f(c2r[i] - cs));
          } else {
            const int ks = dc.any ? __shfl(dc.k, s, 64) : 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 16 * rt + 4 * lg + i;
              float p = 0.f;
              const float cr = c2r[i];
              const bool sep = dc.any && __shfl(dc.k, r, 64) != ks;  // a reset in (s, r]
              if (r >= s && r < n && !sep) p = acc[i] * __builtin_amdgcn_exp2f(cr - cs);
              pv[i] = tobf(p);
            }
          }
          *reinterpret_cast<bf16x4 *>(PT + swz_off<8>(s, 2 * rt + (lg >> 1)) + (lg & 1) * 8) = pv;
        }
      }
      lds_barrier();  // score tiles visible; next chunk's DMA stays in flight

      if (side == 0) {
        // ---- dV^T[j][s] = gamma_s (G^T K^T)[j][s] + (dO^T P1)[j][s] ----
        FRESH_LANE();
        bf16x8 gfrag[DK / 32][NJ];
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) gfrag[kk][jt] = cvt8(G0(2 * kk, jt), G0(2 * kk + 1, jt));
        bf16x8 dfrag[NJ][2];  // dO^T A operands: row j, k = r
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) dfrag[jt][kb] = tr_frag<NCV>(DOS, 32 * kb, jw0 + 16 * jt, li, lg);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int s = 16 * st + li;
          const float gs = __shfl(gam_l, s, 64);
          bf16x8 kfrag[DK / 32];
#pragma unroll
          for (int kk = 0; kk < DK / 32; ++kk)
            kfrag[kk] = cat8(lds_half<NCK>(KS, s, 32 * kk + 4 * lg),
                             lds_half<NCK>(KS, s, 32 * kk + 16 + 4 * lg));
          bf16x8 pfrag[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) pfrag[kb] = lds_frag<8>(P1, s, 4 * kb + lg);
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) acc = mfma(gfrag[kk][jt], kfrag[kk], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] *= gs;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              if (2 * kb + 1 >= st) acc = mfma(dfrag[jt][kb], pfrag[kb], acc);
            // acc[i] = dV[s][jw0 + 16 jt + 4 lg + i]
            if (s < n) {
              bf16x4 ov;
#pragma unroll
              for (int i = 0; i < 4; ++i) ov[i] = tobf(acc[i]);
              *reinterpret_cast<bf16x4 *>(a.dv + (bh * T + t0 + s) * DV + jw0 + 16 * jt + 4 * lg) = ov;
            }
          }
        }
      } else {
        // ---- dK^T[d][s] = gamma_s (G V^T)[d][s] + (Q^T P2)[d][s] ; r2_s ----
        // G enters the inter-chunk product as G = hi + lo, two bf16 parts
        // (hi = bf16(G), lo = bf16(G - hi), both formed once per chunk), and
        //   r2_s = k_s . dk_s + sum_d ((gamma_s k_s)_bf16 - gamma_s k_s)[d] (G v_s)[d]
        //        = (gamma_s k_s)_bf16 . (G v_s) + k_s . (Q^T P2)[:, s],
        // evaluated in the second form (the in-chunk product on its own
        // accumulator); its inter-chunk part pairs with the bf16-rounded
        // (gamma k) rows of the dQ pass's state update, so that the decay
        // gradient's sums telescope exactly (see the segment length in
        // chunk.hip).
        FRESH_LANE();
        bf16x8 ghi[DV / 32][NI], glo[DV / 32][NI];
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk)
#pragma unroll
          for (int it = 0; it < NI; ++it)
            split8(G1(2 * kk, it), G1(2 * kk + 1, it), ghi[kk][it], glo[kk][it]);
        bf16x8 qfrag[NI][2];  // Q^T A operands: row d, k = r
#pragma unroll
        for (int it = 0; it < NI; ++it)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) qfrag[it][kb] = tr_frag<NCK>(QS, 32 * kb, dw0 + 16 * it, li, lg);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int s = 16 * st + li;
          const float gs = __shfl(gam_l, s, 64);
          bf16x8 vfrag[DV / 32];  // V B operands: column s
#pragma unroll
          for (int kk = 0; kk < DV / 32; ++kk)
            vfrag[kk] = cat8(lds_half<NCV>(VS, s, 32 * kk + 4 * lg),
                             lds_half<NCV>(VS, s, 32 * kk + 16 + 4 * lg));
          bf16x8 pfrag[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) pfrag[kb] = lds_frag<8>(P2, s, 4 * kb + lg);
          float r2p = 0.f;
#pragma unroll
          for (int it = 0; it < NI; ++it) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DV / 32; ++kk) acc = mfma(ghi[kk][it], vfrag[kk], acc);
#pragma unroll
            for (int kk = 0; kk < DV / 32; ++kk) acc = mfma(glo[kk][it], vfrag[kk], acc);
            // in-chunk part on its own accumulator (no wait for the above)
            f32x4 ai = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              if (2 * kb + 1 >= st) ai = mfma(qfrag[it][kb], pfrag[kb], ai);
            const int dc = dw0 + 16 * it + 4 * lg;
            const bf16x4 kv = lds_half<NCK>(KS, s, dc);
            float kf[4];
            bf16x4 kgb;  // bf16(gamma_s k_s), as the dQ pass's state update rounds it
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              kf[i] = tof(kv[i]);
              kgb[i] = tobf(kf[i] * gs);
            }
            // r2_s = bf16(gamma k) . (G v) + k . (in-chunk part), and
            // dk = gamma (G v) + in-chunk part
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              r2p += tof(kgb[i]) * acc[i];
              r2p += kf[i] * ai[i];
              acc[i] = __builtin_fmaf(gs, acc[i], ai[i]);
            }
            if (s < n) {
              bf16x4 ov;
#pragma unroll
              for (int i = 0; i < 4; ++i) ov[i] = tobf(acc[i]);
              *reinterpret_cast<bf16x4 *>(a.dk + (bh * T + t0 + s) * DK + dc) = ov;
            }
          }
          r2p += __shfl_xor(r2p, 16, 64);
          r2p += __shfl_xor(r2p, 32, 64);
          if (lg == 0) *r2p_at(wv, s) = r2p;
        }
      }
    }

    // ---- state-gradient update (both copies): G <- alpha G + Q^T (lambda dO) ----
    FRESH_LANE();
#pragma unroll
    for (int x = 0; x < NG; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) Gs[x][i] *= alpha;
    if (side == 0) {
      // G[d][j] += sum_r Q^T[d][r] (lambda dO)[r][j]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float lam[8];
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4 *>(tok_at(1, 32 * kb + 8 * lg + e));
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) lam[e + e2] = l4[e2];
        }
        bf16x8 db[NJ];  // (lambda dO) B operands: k = r, column j
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
          const bf16x8 x = tr_frag<NCV>(DOS, 32 * kb, jw0 + 16 * jt, li, lg);
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = tof(x[e]) * lam[e];
          db[jt] = cvt8(y);
        }
#pragma unroll
        for (int dt = 0; dt < DK / 16; ++dt) {
          const bf16x8 qa = tr_frag<NCK>(QS, 32 * kb, 16 * dt, li, lg);  // Q^T: row d, k = r
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) G0(dt, jt) = mfma(qa, db[jt], G0(dt, jt));
        }
      }
    } else {
      // G^T[j][d] += sum_r dO^T[j][r] (lambda Q)[r][d]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float lam[8];
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4 *>(tok_at(1, 32 * kb + 8 * lg + e));
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) lam[e + e2] = l4[e2];
        }
        bf16x8 qb[NI];  // (lambda Q) B operands: k = r, column d
#pragma unroll
        for (int it = 0; it < NI; ++it) {
          const bf16x8 x = tr_frag<NCK>(QS, 32 * kb, dw0 + 16 * it, li, lg);
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = tof(x[e]) * lam[e];
          qb[it] = cvt8(y);
        }
#pragma unroll
        for (int jt = 0; jt < DV / 16; ++jt) {
          const bf16x8 da = tr_frag<NCV>(DOS, 32 * kb, 16 * jt, li, lg);  // dO^T: row j, k = r
#pragma unroll
          for (int it = 0; it < NI; ++it) G1(jt, it) = mfma(da, qb[it], G1(jt, it));
        }
      }
    }
    r2_t0 = t0;
    r2_n = n;
    if (w == 0 && dl_row >= 0) {
      const float dl_val = chunk_dl(r1_prev, r2_prev, dl_n);
      if (lane < dl_n) a.dl[bh * T + dl_row + fresh(lane)] = dl_val;
    }
    r1_prev = r1_cur;
    // the next chunk has landed; this chunk's buffer is free
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  stage(c_end - 1, buf0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int64_t ci = c_end - 1; ci >= c_begin; ci -= 2) {
    step(ci, buf0, buf1);
    if (ci - 1 >= c_begin) step(ci - 1, buf1, buf0);
  }
  if (w == 0 && r2_t0 >= 0) {
    const float v = chunk_dl(r1_prev, lane < r2_n ? r2p_sum(lane) : 0.f, r2_n);
    if (lane < r2_n) a.dl[bh * T + r2_t0 + lane] = v;
  }

  // ---- segment outputs ----
  if (seg == 0 && a.dS0 && side == 0) {
    float *dst = a.dS0 + bh * DK * DV;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(16 * dt + 4 * lg + i) * DV + jw0 + 16 * jt + li] = G0(dt, jt)[i];
  }
}

#undef G0
#undef G1
#undef FRESH_LANE

template <int DK, int DV>
hipError_t bwd_kv_impl(BwdArgs args, hipStream_t stream) {
  const int64_t P = args.P;
  if (P > 1) {
    // Gloc/aloc hold each later segment's local G state and total decay (from
    // the dQ pass); the reverse scan turns slot p into the G at the end of
    // segment p
    hipError_t e =
        launch_segment_scan(args.Gloc, args.aloc, args.dST, 0, 1, args.nh, P, DK, DV, stream);
    if (e != hipSuccess) return e;
    args.Gin = args.Gloc;
  }
  CLA_LAUNCH("chunk_dkdv", (chunk_bwd_kernel<DK, DV>), dim3((unsigned)args.nh, (unsigned)P),
             dim3(BTHR), stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t bwd_kv_dispatch(const BwdArgs &args, int DK, int DV, hipStream_t stream) {
  if (DK == 64 && DV == 64) return bwd_kv_impl<64, 64>(args, stream);
  if (DK == 64 && DV == 128) return bwd_kv_impl<64, 128>(args, stream);
  if (DK == 128 && DV == 64) return bwd_kv_impl<128, 64>(args, stream);
  if (DK == 128 && DV == 128) return bwd_kv_impl<128, 128>(args, stream);
  return hipErrorInvalidValue;
}

}  // namespace chunk
}  // namespace cla
