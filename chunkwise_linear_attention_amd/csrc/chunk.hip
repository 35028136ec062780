// Chunkwise linear attention with a scalar decay per step, forward pass and
// the segment machinery shared with the backward, for gfx950.
//
// Citations (page title, then section / equation):
//   ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
//   LA2 = "Lightning Attention-2: A Free Lunch for Handling Unlimited
//         Sequence Lengths in Large Language Models" (paper-graph-ui summary)
//
// Recurrence (ZTF "The chunkwise algorithm"): S_t = a_t S_{t-1} + k_t v_t^T,
// o_t = S_t^T q_t, a_t = exp(l_t).  Chunks of TC = 64 tokens; for chunk j
// starting after token t0, with in-chunk cumulative logs c_r = l_{t0+1} + ...
// + l_{t0+r} (ZTF "Long products without underflow": sums of logs inside a
// short window stay accurate; no long cumulative sums, no ratios):
//   mask     D_rs  = exp(c_r - c_s) for r >= s (diagonal 1), else 0
//   lambda_r       = exp(c_r)          decay from the chunk start
//   gamma_s        = exp(c_n - c_s)    decay to the chunk end
//   alpha          = exp(c_n)
//   O_[j] = (Q K^T (.) D) V + diag(lambda) Q S_[j-1]      (LA2 Eq. 8)
//   S_[j] = alpha S_[j-1] + (diag(gamma) K)^T V           (LA2 Eq. 10)
// The mask is applied elementwise to the fp32 score tile; it is never
// factored into exp(c_r) exp(-c_s), which overflows for strong decays.  A
// step with l = -inf (a = 0) is an exact reset: the sums keep only finite
// parts and a count of resets decides which products vanish (chunk_decay).
//
// Workgroup = 4 waves on one (batch*head, segment).  Per chunk:
//   stage  : Q (row-major), K (row-major and transposed), V (transposed) into
//            LDS; wave 0 computes c, lambda, gamma, alpha.
//   scores : wave w computes the transposed scores for queries 16w..16w+15
//            against the key tiles at or below the diagonal, masks them in
//            fp32 and writes P = bf16(S (.) D) to LDS.
//   output : wave w owns value columns [w DV/4, (w+1) DV/4) and computes
//            O^T = V^T P^T + S^T (lambda Q)^T on MFMA; its slice of the fp32
//            state, held in MFMA accumulators, is fed back (as bf16) as the A
//            operand of the inter-chunk product without leaving registers.
//   update : S <- alpha S + (gamma K)^T V on MFMA into the same accumulators.
// Inputs are bf16, the state and all accumulation fp32.
#include "chunk_common.h"
#include "chunk_kernels.h"
#include "internal.h"

namespace cla {
namespace chunk {
namespace {

// Concurrent workgroups: the forward-type kernel runs two per CU, the dK/dV
// kernel one per CU, on 256 CUs.  Segment counts are chosen so that the
// workgroups fill whole rounds of these slots.
constexpr int64_t kFwdSlots = 512;
constexpr int64_t kBwdSlots = 256;
constexpr int64_t kMinSegChunks = 4;
// The backward's decay gradient sums q.dq - k.dk backwards only inside one
// segment, starting from the boundary term <S, G> of the two segment states.
// The sum telescopes: over a chunk, the inter-chunk parts of q.dq add up to
// <S_[j-1], dG_j> and those of k.dk to <dS_j, G_j>, where dG_j and dS_j are
// the chunk's contributions to the two states as the kernels accumulate them
// (from (lambda q) and (gamma k) rounded to bf16).  The kernels form q.dq and
// k.dk from exactly those rounded operands and from both states split into
// two bf16 parts (hi + lo), so the two sums cancel to fp32 accumulation
// accuracy and no bf16 rounding noise gathers along the sum.  Backward
// segments hold at most 16 chunks (1024 tokens).
constexpr int64_t kMaxBwdSegChunks = 16;

// Outputs o, S_T and (XD) rdot of one segment.  XD marks the backward's dQ
// pass (see launch_chunk_bwd): there the inter-chunk product uses the state
// split into two bf16 parts, rdot carries the correction that pairs it with
// the rounded (lambda q) of the state-gradient update, and the state at the
// end of each segment but the last is written to Send.  With GSUM, also (in
// segments after the first) the segment-local sum Q^T diag(A) X over the
// segment (gloc, galoc), A_t the decay from the segment start through token
// t.  Run as the backward's dQ pass (Q = dO, X = q) this is the local G state
// of the segment: the gradient of the state entering it from the segment's
// own outputs, G_start = sum_t A_t q_t dO_t^T, a plain sum that needs no
// reverse sweep (ZTF "The chunkwise algorithm", the inter-chunk term read
// backwards).
// Four waves; wave w owns value columns [w DV/4, (w+1) DV/4).
template <int DK, int DV, bool GSUM, bool XD>
__global__ __launch_bounds__(NTHR, 2) void chunk_fwd_kernel(FwdArgs a) {
  static_assert(!GSUM || XD, "segment-local sums are formed in the dQ pass only");
  constexpr int NJ = DV / 64;          // 16-column tiles per wave
  constexpr int NDT = DK / 16;         // 16-row tiles of the state
  constexpr int NCK = DK / 8, NCV = DV / 8;  // 16-byte chunks per row
  constexpr int QB = 64 * DK * 2, VB = 64 * DV * 2;
  // Staging buffer [Q | K | V | X | l] (X: the optional xdot rows).  It is
  // double-buffered (the next chunk streams in by DMA while this one is used)
  // when two workgroups per CU still fit in LDS.  The copies are issued
  // untracked (the compiler had waited for them in front of LDS reads it could
  // not tell apart from their target); each staged chunk is waited for
  // explicitly before it is read.
  constexpr int B_KS = QB;
  constexpr int B_VS = B_KS + QB;
  constexpr int B_XS = B_VS + VB;
  constexpr int B_L = B_XS + (XD ? VB : 0);
  constexpr int BUF = B_L + 64 * 4;
  constexpr int PSB = 64 * 128;
  constexpr int RDB = NWAVE * 64;
  constexpr bool DB = 2 * BUF + PSB + 4 * RDB <= 80 * 1024;
  constexpr int NBQ = DK / 8, NBK = DK / 8, NBV = DV / 8;
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[DB ? BUF : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char PS[PSB];
  __shared__ float RD[RDB];  // xdot partial sums [w][row]
  // The output reads P in 32-column steps up to the diagonal, so rows 0-31,
  // columns 32-63 of P are never written or read: they hold the chunk's
  // per-token values TOK[u][t] (u = 0: base-2 cumulative log, 1: gamma, 2:
  // the segment sums' weight), written by every wave (the same values), so
  // that lanes needing 4 or 8 consecutive tokens read them as 16-byte pieces
  // instead of one cross-lane shuffle per token.
  auto tok_at = [&](int u, int t_) __attribute__((always_inline)) -> float * {
    const int idx = u * 64 + t_;
    const int q = idx >> 2;
    return reinterpret_cast<float *>(PS + swz_off<8>(q >> 2, 4 + (q & 3)) + 4 * (idx & 3));
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  int li = lane & 15, lg = lane >> 4;
  // Re-derive the lane coordinates behind an empty asm at the start of each
  // phase, so that the compiler forms LDS addresses next to their use instead
  // of hoisting all of them out of the chunk loop (which exhausts registers).
#define FRESH_LANE()             \
  do {                           \
    int l_ = lane;               \
    asm volatile("" : "+v"(l_)); \
    li = l_ & 15;                \
    lg = l_ >> 4;                \
  } while (0)
  // a lane-dependent value re-derived behind an empty asm, like FRESH_LANE,
  // so that addresses built from it are not kept live across the chunk loop
  auto fresh = [](int x) __attribute__((always_inline)) {
    asm volatile("" : "+v"(x));
    return x;
  };
  // grid (nh, segments): both indices are workgroup ids, held in scalar
  // registers, so every pointer derived from them stays wave-uniform
  const int64_t bh = blockIdx.x;
  const int64_t seg = blockIdx.y;
  const int64_t T = a.T;
  const int64_t nchunks = (T + TC - 1) / TC;
  const int64_t c_begin = seg * a.seg_chunks;
  const int64_t c_end = min(nchunks, c_begin + a.seg_chunks);
  const int j0 = w * (DV / 4);  // first value column of this wave
  constexpr bool has_x = XD;
  const bool do_g = GSUM && seg > 0;  // wave-uniform

  const uint16_t *qh = a.q + bh * T * DK;
  const uint16_t *kh = a.k + bh * T * DK;
  const uint16_t *vh = a.v + bh * T * DV;
  const uint16_t *xh = has_x ? a.xdot + bh * T * DV : nullptr;
  const float *lh = a.l + bh * T;

  // S_acc[dt][jt][i] = S[16 dt + 4 lg + i][j0 + 16 jt + li]; G_acc alike
  f32x4 S_acc[NDT][NJ];
  f32x4 G_acc[GSUM ? NDT : 1][NJ];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) S_acc[dt][jt] = zero4();
  if constexpr (GSUM) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) G_acc[dt][jt] = zero4();
  }
  {
    const float *src = nullptr;
    bool trans = false;
    if (seg == 0) {
      src = a.S0 ? a.S0 + bh * DK * DV : nullptr;
      trans = a.s0_trans;
    } else {
      src = a.Sin + ((seg - 1) * a.nh + bh) * DK * DV;
      trans = a.slot_trans;
    }
    if (src && trans && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
      // stored transposed: this lane's four rows d are contiguous (16 bytes)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
          S_acc[dt][jt] = *reinterpret_cast<const f32x4 *>(src + (j0 + 16 * jt + li) * DK +
                                                            16 * dt + 4 * lg);
    } else if (src) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = 16 * dt + 4 * lg + i, j = j0 + 16 * jt + li;
            S_acc[dt][jt][i] = src[trans ? j * DK + d : d * DV + j];
          }
    }
  }
  float alpha_total = 1.f;
  // saved states: the next one is slot save_slot - 1, taken after chunk
  // save_at - 1 (a counter, so that the chunk loop does no 64-bit division)
  int64_t save_slot = 0, save_at = -1;
  if (!XD && a.saved) {
    save_slot = c_begin / a.save_every + 1;
    save_at = save_slot * a.save_every;
    if (save_at >= nchunks) save_at = -1;  // no state is saved after the last chunk
  }
  int64_t rd_t0 = -1;  // chunk whose xdot partials sit in RD
  int rd_n = 0;

  // DMA of chunk cj into a staging buffer: 1 KB row blocks spread over the
  // waves, the 64 log decays (rows clamped to the chunk) by wave 0.  part 0:
  // everything; 1: Q, X and the log decays; 2: K and V.
  auto stage = [&](int64_t cj, unsigned char *buf, int part = 0) __attribute__((always_inline)) {
    const int64_t tj = cj * TC;
    const int nj = (int)min<int64_t>(TC, T - tj);
    // the per-lane DMA addresses are formed here, at each stage, instead of
    // being kept live (one 64-bit pair per staged tensor) across the loop
    const int ln = fresh(lane);
    const uint32_t lb = staging_base(buf);
    // wave w takes blocks w, w + NWAVE, ...; every tensor's block count is a
    // multiple of NWAVE, so the tensor of each round is known at compile time
    static_assert(NBQ % NWAVE == 0 && NBK % NWAVE == 0 && NBV % NWAVE == 0, "rounds");
#pragma unroll
    for (int r0 = 0; r0 < NBQ + NBK + NBV + (XD ? NBV : 0); r0 += NWAVE) {
      const int b = w + r0;
      const bool early = r0 < NBQ || r0 >= NBQ + NBK + NBV;  // Q or X
      if ((part == 1 && !early) || (part == 2 && early)) continue;
      // (untracked copies: every staged chunk is waited for explicitly)
      if (r0 < NBQ) {
        lds_copy16_untracked(bf16_block_src<DK>(qh + tj * DK, nj, b, ln), lb + b * 1024);
      } else if (r0 < NBQ + NBK) {
        lds_copy16_untracked(bf16_block_src<DK>(kh + tj * DK, nj, b - NBQ, ln),
                             lb + B_KS + (b - NBQ) * 1024);
      } else if (r0 < NBQ + NBK + NBV) {
        lds_copy16_untracked(bf16_block_src<DV>(vh + tj * DV, nj, b - NBQ - NBK, ln),
                             lb + B_VS + (b - NBQ - NBK) * 1024);
      } else {
        lds_copy16_untracked(bf16_block_src<DV>(xh + tj * DV, nj, b - NBQ - NBK - NBV, ln),
                             lb + B_XS + (b - NBQ - NBK - NBV) * 1024);
      }
    }
    if (w == 0 && part != 2) lds_copy4_untracked(lh + tj + min(ln, nj - 1), lb + B_L);
  };

  // the xdot sums of the previous chunk, from RD
  auto rd_sum = [&]() __attribute__((always_inline)) -> float {
    float s = 0.f;
    if (rd_t0 >= 0 && tid < rd_n) {
#pragma unroll
      for (int u = 0; u < NWAVE; ++u) s += RD[u * 64 + tid];
    }
    return s;
  };

  // The work on one staged chunk.
  auto compute = [&](int64_t ci, const unsigned char *cur, auto before_update)
                     __attribute__((always_inline)) {
    const int64_t t0 = ci * TC;
    const int n = (int)min<int64_t>(TC, T - t0);
    const unsigned char *QS = cur;
    const unsigned char *KS = cur + B_KS;
    const unsigned char *VS = cur + B_VS;
    const unsigned char *XS = cur + B_XS;
    const float *LC = reinterpret_cast<const float *>(cur + B_L);

    // In-chunk decays, one token per lane, computed by every wave and read
    // with cross-lane shuffles.  Rows past the chunk: gamma = 0, so that they
    // add nothing to the state.
    const int fl = fresh(lane);
    const ChunkDecay dc = chunk_decay(fl < n ? LC[fl] : 0.f, fl);
    const float c_l = dc.c;
    const float c2_l = c_l * kLog2e;  // base-2 cumulative log
    const float lam_l = dc.k == 0 ? expf(c_l) : 0.f;
    const float gam_l = lane < n && dc.k == dc.k_last ? expf(dc.c_last - c_l) : 0.f;
    const float alpha = dc.k_last == 0 ? expf(dc.c_last) : 0.f;
    *tok_at(0, lane) = c2_l;
    *tok_at(1, lane) = gam_l;

    {
      // ---- masked transposed score tiles -> P[r][s] (bf16) ----
      FRESH_LANE();
      // A whole chunk without resets needs no mask below the diagonal tiles
      // (s < r there); the decay factor is exp2 of a difference of base-2
      // cumulative logs.
      const bool plain = n == TC && !dc.any;
#pragma unroll
      for (int tt = 0; tt < 12 / NWAVE; ++tt) {
        const int t = w + NWAVE * tt;
        const int rt = tile_rt(t), st = tile_st(t);
        const int r = 16 * rt + li;
        f32x4 acc = zero4();
        if (st <= rt) {
#pragma unroll
          for (int kk = 0; kk < DK / 32; ++kk)
            acc = mfma(lds_frag<NCK>(KS, 16 * st + li, 4 * kk + lg),
                       lds_frag<NCK>(QS, r, 4 * kk + lg), acc);
        }
        // acc[i] = (K Q^T)[s = 16 st + 4 lg + i][r]; keys past the chunk are masked
        const float cr = __shfl(c2_l, r, 64);
        // base-2 cumulative logs of this lane's 4 keys s = 16 st + 4 lg + i
        const f32x4 c2s = *reinterpret_cast<const f32x4 *>(tok_at(0, 16 * st + 4 * lg));
        bf16x4 pv;
        if (plain && st < rt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = tobf(acc[i] * __builtin_amdgcn_exp2f(cr - c2s[i]));
        } else {
          const int kr = dc.any ? __shfl(dc.k, r, 64) : 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = 16 * st + 4 * lg + i;
            const float cs = c2s[i];
            const bool sep = dc.any && __shfl(dc.k, s, 64) != kr;  // a reset in (s, r]
            float p = 0.f;
            if (s <= r && s < n && !sep) p = acc[i] * __builtin_amdgcn_exp2f(cr - cs);
            pv[i] = tobf(p);
          }
        }
        *reinterpret_cast<bf16x4 *>(PS + swz_off<8>(r, 2 * st + (lg >> 1)) + (lg & 1) * 8) = pv;
      }
      lds_barrier();

      if constexpr (XD) {
        // ---- dQ pass output: O^T[j][r] = lambda_r (S^T Q^T)[j][r] + (V^T P^T)[j][r] ----
        // (here O = dq, Q = dO, V = k, X = q).  The inter-chunk product takes
        // the state as S = hi + lo, two bf16 parts (hi = bf16(S), lo =
        // bf16(S - hi), both formed once per chunk), so that S enters it to ~2^-16;
        // rdot_r = x_r . o_r plus the correction
        //   sum_j ((lambda_r x_r)_bf16 - lambda_r x_r)[j] (S^T Q^T)[j][r],
        // evaluated as (lambda_r x_r)_bf16 . (S^T Q^T)[:, r] + x_r . (V^T P^T)[:, r]
        // (the in-chunk product on its own accumulator), which makes its
        // inter-chunk part pair with the bf16-rounded (lambda q) rows that the
        // dK/dV pass adds into its state gradient.
        FRESH_LANE();
        bf16x8 vfrag[NJ][2];  // A operands V^T: row j, k = s
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) vfrag[jt][kb] = tr_frag<NCV>(VS, 32 * kb, j0 + 16 * jt, li, lg);
        bf16x8 shi[DK / 32][NJ], slo[DK / 32][NJ];  // the state slice as hi + lo
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt)
            split8(S_acc[2 * kk][jt], S_acc[2 * kk + 1][jt], shi[kk][jt], slo[kk][jt]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int rr = 16 * rt + li;
          const float lam = __shfl(lam_l, rr, 64);
          bf16x8 qfrag[DK / 32];  // Q^T B operands, same k permutation
#pragma unroll
          for (int kk = 0; kk < DK / 32; ++kk)
            qfrag[kk] = cat8(lds_half<NCK>(QS, rr, 32 * kk + 4 * lg),
                             lds_half<NCK>(QS, rr, 32 * kk + 16 + 4 * lg));
          bf16x8 pfrag[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) pfrag[kb] = lds_frag<8>(PS, rr, 4 * kb + lg);
          float rdp = 0.f;
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) acc = mfma(shi[kk][jt], qfrag[kk], acc);
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) acc = mfma(slo[kk][jt], qfrag[kk], acc);
            // in-chunk part on its own accumulator (no wait for the above)
            f32x4 ai = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              if (kb <= (rt >> 1)) ai = mfma(vfrag[jt][kb], pfrag[kb], ai);
            const int jc = j0 + 16 * jt + 4 * lg;
            const bf16x4 xv = lds_half<NCV>(XS, rr, jc);
            float xf[4];
            bf16x4 xlb;  // bf16(lambda_r x_r), as the dK/dV pass's state update rounds it
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              xf[i] = tof(xv[i]);
              xlb[i] = tobf(xf[i] * lam);
            }
            // rdot_r = bf16(lambda x) . (S^T q) + x . (in-chunk part), and
            // o = lambda (S^T q) + in-chunk part
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              rdp += tof(xlb[i]) * acc[i];
              rdp += xf[i] * ai[i];
              acc[i] = __builtin_fmaf(lam, acc[i], ai[i]);
            }
            if (rr < n) {
              bf16x4 ov;
#pragma unroll
              for (int i = 0; i < 4; ++i) ov[i] = tobf(acc[i]);
              *reinterpret_cast<bf16x4 *>(a.o + (bh * T + t0 + rr) * DV + jc) = ov;
            }
          }
          rdp += __shfl_xor(rdp, 16, 64);
          rdp += __shfl_xor(rdp, 32, 64);
          if (lg == 0) RD[w * 64 + rr] = rdp;
        }
        rd_t0 = t0;
        rd_n = n;
      } else {
        // ---- output: O^T[j][r] = lambda_r (S^T Q^T)[j][r] + (V^T P^T)[j][r] ----
        FRESH_LANE();
        bf16x8 vfrag[NJ][2];  // A operands V^T: row j, k = s
  #pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb) vfrag[jt][kb] = tr_frag<NCV>(VS, 32 * kb, j0 + 16 * jt, li, lg);
        // the state slice as bf16 A operands: row j, k-set
        // {32kk + 4lg + 0..3, 32kk + 16 + 4lg + 0..3}
        bf16x8 sfrag[DK / 32][NJ];
  #pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
  #pragma unroll
          for (int jt = 0; jt < NJ; ++jt) sfrag[kk][jt] = cvt8(S_acc[2 * kk][jt], S_acc[2 * kk + 1][jt]);
  #pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int rr = 16 * rt + li;
          const float lam = __shfl(lam_l, rr, 64);
          bf16x8 qfrag[DK / 32];  // Q^T B operands, same k permutation
  #pragma unroll
          for (int kk = 0; kk < DK / 32; ++kk)
            qfrag[kk] = cat8(lds_half<NCK>(QS, rr, 32 * kk + 4 * lg),
                             lds_half<NCK>(QS, rr, 32 * kk + 16 + 4 * lg));
          bf16x8 pfrag[2];
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb) pfrag[kb] = lds_frag<8>(PS, rr, 4 * kb + lg);
  #pragma unroll
          for (int jt = 0; jt < NJ; ++jt) {
            f32x4 acc = zero4();
  #pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) acc = mfma(sfrag[kk][jt], qfrag[kk], acc);
  #pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] *= lam;
  #pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              if (kb <= (rt >> 1)) acc = mfma(vfrag[jt][kb], pfrag[kb], acc);
            // acc[i] = O[row rr][col j0 + 16 jt + 4 lg + i]
            const int jc = j0 + 16 * jt + 4 * lg;
            if (rr < n) {
              bf16x4 ov;
  #pragma unroll
              for (int i = 0; i < 4; ++i) ov[i] = tobf(acc[i]);
              *reinterpret_cast<bf16x4 *>(a.o + (bh * T + t0 + rr) * DV + jc) = ov;
            }
          }
        }
      }
    }

    // ---- segment-local sum: G += Q^T diag(A) X, A_r = alpha_total lambda_r ----
    // (once the decay from the segment start is exactly 0, every later token
    // adds exactly 0)
    if (GSUM && do_g && __builtin_amdgcn_readfirstlane(alpha_total != 0.f ? 1 : 0)) {
      FRESH_LANE();
      *tok_at(2, lane) = lane < n ? alpha_total * lam_l : 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float wg[8];
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          const f32x4 w4 = *reinterpret_cast<const f32x4 *>(tok_at(2, 32 * kb + 8 * lg + e));
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) wg[e + e2] = w4[e2];
        }
        bf16x8 xb[NJ];  // (A X) B operands: k = s, column j
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
          const bf16x8 x = tr_frag<NCV>(XS, 32 * kb, j0 + 16 * jt, li, lg);
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = tof(x[e]) * wg[e];
          xb[jt] = cvt8(y);
        }
#pragma unroll
        for (int dt = 0; dt < (GSUM ? NDT : 0); ++dt) {
          const bf16x8 qa = tr_frag<NCK>(QS, 32 * kb, 16 * dt, li, lg);  // Q^T: row d, k = s
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) G_acc[dt][jt] = mfma(qa, xb[jt], G_acc[dt][jt]);
        }
      }
    }

    before_update();
    // ---- state update: S <- alpha S + K^T (gamma V) ----
    FRESH_LANE();
    alpha_total *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S_acc[dt][jt][i] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float gam[8];
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        const f32x4 g4 = *reinterpret_cast<const f32x4 *>(tok_at(1, 32 * kb + 8 * lg + e));
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) gam[e + e2] = g4[e2];
      }
      bf16x8 vb[NJ];  // (gamma V) B operands: k = s, column j
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        const bf16x8 x = tr_frag<NCV>(VS, 32 * kb, j0 + 16 * jt, li, lg);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = tof(x[e]) * gam[e];
        vb[jt] = cvt8(y);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8 ka = tr_frag<NCK>(KS, 32 * kb, 16 * dt, li, lg);  // K^T: row d, k = s
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) S_acc[dt][jt] = mfma(ka, vb[jt], S_acc[dt][jt]);
      }
    }
    // the state the backward's segment save_slot starts from
    if (!XD && ci + 1 == save_at) {
      float *dst = a.saved + ((save_slot - 1) * a.nh + bh) * DK * DV;
      ++save_slot;
      save_at = ci + 1 + a.save_every < nchunks ? ci + 1 + a.save_every : -1;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dst[(16 * dt + 4 * lg + i) * DV + j0 + 16 * jt + li] = S_acc[dt][jt][i];
    }
  };

  if constexpr (DB) {
    // one step: chunk ci from `cur` while chunk ci + 1 streams into `nxt`
    auto step = [&](int64_t ci, unsigned char *cur, unsigned char *nxt)
                    __attribute__((always_inline)) {
      if (ci + 1 < c_end) stage(ci + 1, nxt);
      // the previous chunk's xdot sums, stored at the end of the step (a
      // store issued here would hold its data register while the DMA is in
      // flight)
      const float rs = rd_sum();
      const int64_t rs_t0 = rd_t0;
      const int rs_n = rd_n;
      compute(ci, cur, [] {});
      if (rs_t0 >= 0 && tid < rs_n) a.rdot[bh * T + rs_t0 + fresh(tid)] = rs;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // the next chunk has landed; this chunk's buffer is free
    };
    stage(c_begin, buf0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int64_t ci = c_begin; ci < c_end; ci += 2) {
      step(ci, buf0, buf1);
      if (ci + 1 < c_end) step(ci + 1, buf1, buf0);
    }
  } else {
    // One buffer: Q, X and the log decays of the next chunk are copied while
    // the state update runs (it reads none of them), K and V once it is done.
    stage(c_begin, buf0, 1);
    for (int64_t ci = c_begin; ci < c_end; ++ci) {
      lds_barrier();  // the previous chunk's LDS reads (and RD writes) are done
      const float rs = rd_sum();
      const int64_t rs_t0 = rd_t0;
      const int rs_n = rd_n;
      stage(ci, buf0, 2);
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();  // every wave's DMA has landed
      // (stored with nothing in flight)
      if (rs_t0 >= 0 && tid < rs_n) a.rdot[bh * T + rs_t0 + fresh(tid)] = rs;
      compute(ci, buf0, [&] {
        lds_barrier();  // every wave is done with Q and X
        if (ci + 1 < c_end) stage(ci + 1, buf0, 1);
      });
    }
    lds_barrier();
  }
  {
    const float rs = rd_sum();
    if (rd_t0 >= 0 && tid < rd_n) a.rdot[bh * T + rd_t0 + tid] = rs;
  }

  // ---- segment outputs ----
  if (GSUM && do_g) {
    // stored transposed (row j, then d): as the dK/dV pass's G in the dQ pass
    float *dst = a.gloc + ((seg - 1) * a.nh + bh) * DK * DV;
#pragma unroll
    for (int dt = 0; dt < (GSUM ? NDT : 0); ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
        *reinterpret_cast<f32x4 *>(dst + (j0 + 16 * jt + li) * DK + 16 * dt + 4 * lg) =
            G_acc[dt][jt];
    if (tid == 0) a.galoc[(seg - 1) * a.nh + bh] = alpha_total;
  }
  if (XD && a.Send && seg < a.P - 1) {
    // this pass's own state at the segment's end, for the decay gradient's
    // boundary term (row-major, coalesced 64-byte pieces)
    float *dst = a.Send + (seg * a.nh + bh) * DK * DV;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(16 * dt + 4 * lg + i) * DV + j0 + 16 * jt + li] = S_acc[dt][jt][i];
  }
  if (seg == a.P - 1 && a.ST) {
    float *dst = a.ST + bh * DK * DV;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 16 * dt + 4 * lg + i, j = j0 + 16 * jt + li;
          dst[a.st_trans ? j * DK + d : d * DV + j] = S_acc[dt][jt][i];
        }
  }
}
#undef FRESH_LANE

// Segment state pass: the pair (alpha_p, S_p) of segment p = blockIdx.y from
// a zero state (ZTF "Splitting one sequence across devices", phase one).
// S_p is a plain sum over the segment's chunks,
//   S_p = sum_j A_j (diag(gamma_j) K_j)^T V_j,   A_j = prod_{i > j} alpha_i,
// the decay from chunk j's end to the segment's end, so the chunks are taken
// last to first with A carried as a running product (no rescaling of the
// accumulated state).  Once A is exactly 0 in fp32 (strong decays, or a reset
// with l = -inf), every earlier chunk contributes exactly 0: the pass stops
// there without reading them, and alpha_p = 0.  Only K, V and l are read.
// Four waves; wave w owns columns [w DV/4, (w+1) DV/4); two staging buffers.
//
// GRAD: the mirror image, for the backward's dQ pass when its own
// segment-local sums do not fit in its registers.  For every segment p >= 1,
// the local state gradient G_p = sum_t A_t k_t v_t^T (run on k = q, v = dO),
// A_t = the decay from the segment's start through token t; the chunks are
// taken first to last with the product of the chunk decays carried, and the
// pass stops once it is exactly 0 (every later token adds exactly 0).  Slot
// p - 1 receives G_p, aloc[p - 1] its total decay.
template <int DK, int DV, bool GRAD>
__global__ __launch_bounds__(NTHR, 2) void chunk_state_kernel(FwdArgs a) {
  constexpr int NJ = DV / 64, NDT = DK / 16;
  constexpr int NCK = DK / 8, NCV = DV / 8;
  constexpr int B_VS = 64 * DK * 2, B_L = B_VS + 64 * DV * 2, BUF = B_L + 64 * 4;
  constexpr int NBK = DK / 8, NBV = DV / 8, NBLK = NBK + NBV;
  __shared__ __attribute__((aligned(1024))) unsigned char st0[BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int li = lane & 15, lg = lane >> 4;
  const int64_t bh = blockIdx.x;
  const int64_t seg = blockIdx.y + (GRAD ? 1 : 0);
  const int64_t slot = GRAD ? seg - 1 : seg;
  const int64_t T = a.T;
  const int64_t nchunks = (T + TC - 1) / TC;
  const int64_t c_begin = seg * a.seg_chunks;
  const int64_t c_end = min(nchunks, c_begin + a.seg_chunks);
  const int j0 = w * (DV / 4);
  const uint16_t *kh = a.k + bh * T * DK;
  const uint16_t *vh = a.v + bh * T * DV;
  const float *lh = a.l + bh * T;

  f32x4 S_acc[NDT][NJ];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) S_acc[dt][jt] = zero4();
  // decay from the end of the chunk being added to the segment's end (GRAD:
  // from the segment's start to the start of that chunk); every wave forms
  // it from the same data with the same instructions, so it is the same in
  // all waves
  float A = 1.f;

  auto stage = [&](int64_t cj, unsigned char *buf) __attribute__((always_inline)) {
    const int64_t tj = cj * TC;
    const int nj = (int)min<int64_t>(TC, T - tj);
    static_assert(NBK % NWAVE == 0 && NBV % NWAVE == 0, "rounds");
    const uint32_t lb = staging_base(buf);
#pragma unroll
    for (int r0 = 0; r0 < NBLK; r0 += NWAVE) {
      const int b = w + r0;
      // (untracked copies: every staged chunk is waited for explicitly)
      if (r0 < NBK)
        lds_copy16_untracked(bf16_block_src<DK>(kh + tj * DK, nj, b, lane), lb + b * 1024);
      else
        lds_copy16_untracked(bf16_block_src<DV>(vh + tj * DV, nj, b - NBK, lane),
                             lb + B_VS + (b - NBK) * 1024);
    }
    if (w == 0) lds_copy4_untracked(lh + tj + min(lane, nj - 1), lb + B_L);
  };

  auto compute = [&](int64_t ci, const unsigned char *cur) __attribute__((always_inline)) {
    const int64_t t0 = ci * TC;
    const int n = (int)min<int64_t>(TC, T - t0);
    const unsigned char *KS = cur;
    const unsigned char *VS = cur + B_VS;
    const float *LC = reinterpret_cast<const float *>(cur + B_L);
    int l_ = lane;
    asm volatile("" : "+v"(l_));
    li = l_ & 15;
    lg = l_ >> 4;
    const ChunkDecay dc = chunk_decay(l_ < n ? LC[l_] : 0.f, l_);
    // weight of token s: its decay to the chunk end, times A (GRAD: the decay
    // from the chunk start through s, times A)
    const float wt_l = GRAD ? (l_ < n && dc.k == 0 ? A * expf(dc.c) : 0.f)
                            : (l_ < n && dc.k == dc.k_last ? A * expf(dc.c_last - dc.c) : 0.f);
    const float alpha = dc.k_last == 0 ? expf(dc.c_last) : 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float wt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) wt[e] = __shfl(wt_l, 32 * kb + 8 * lg + e, 64);
      bf16x8 vb[NJ];  // (A gamma V) B operands: k = s, column j
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        const bf16x8 x = tr_frag<NCV>(VS, 32 * kb, j0 + 16 * jt, li, lg);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = tof(x[e]) * wt[e];
        vb[jt] = cvt8(y);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8 ka = tr_frag<NCK>(KS, 32 * kb, 16 * dt, li, lg);  // K^T: row d, k = s
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) S_acc[dt][jt] = mfma(ka, vb[jt], S_acc[dt][jt]);
      }
    }
    A *= alpha;
  };

  // Chunk ci from `cur` while the next chunk to take (ci - 1; GRAD: ci + 1)
  // streams into `nxt`; returns false once the chunks not yet taken can add
  // nothing.  Nothing is in flight on return.
  auto step = [&](int64_t ci, const unsigned char *cur, unsigned char *nxt)
                  __attribute__((always_inline)) -> bool {
    if (GRAD ? ci + 1 < c_end : ci > c_begin) stage(GRAD ? ci + 1 : ci - 1, nxt);
    compute(ci, cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // the next chunk has landed; this chunk's buffer is free
    return __builtin_amdgcn_readfirstlane(A != 0.f ? 1 : 0) != 0;
  };

  if constexpr (GRAD) {
    stage(c_begin, st0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int64_t ci = c_begin; ci < c_end; ci += 2) {
      if (!step(ci, st0, st1)) break;
      if (ci + 1 < c_end && !step(ci + 1, st1, st0)) break;
    }
  } else {
    stage(c_end - 1, st0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int64_t ci = c_end - 1; ci >= c_begin; ci -= 2) {
      if (!step(ci, st0, st1)) break;
      if (ci - 1 >= c_begin && !step(ci - 1, st1, st0)) break;
    }
  }

  float *dst = a.Sloc + (slot * a.nh + bh) * DK * DV;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * dt + 4 * lg + i, j = j0 + 16 * jt + li;
        dst[a.slot_trans ? j * DK + d : d * DV + j] = S_acc[dt][jt][i];
      }
  // the product of every chunk decay of the segment (0 after an early stop)
  if (tid == 0) a.aloc[slot * a.nh + bh] = A;
}

// Incoming state of every segment from the segment pairs (alpha_p, S_p):
// S_in(0) = S0, S_in(p+1) = alpha_p S_in(p) + S_p (ZTF "Splitting one
// sequence across devices": an exclusive scan of per-piece pairs).  In place:
// slot p of Sloc becomes the state entering segment p+1.  One thread per
// state element, sequential over segments.
__global__ void segment_scan_kernel(float *Sloc, const float *aloc, const float *S0,
                                    int s0_trans, int reverse, int64_t nh, int64_t P, int DK,
                                    int DV) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)DK * DV;
  if (e >= nh * per) return;
  const int64_t bh = e / per, x = e % per;
  const int d = (int)(x / DV), j = (int)(x % DV);
  float carry = S0 ? S0[bh * per + (s0_trans ? (int64_t)j * DK + d : x)] : 0.f;
  // Only the carry is sequential: the slots and decays of U segments are
  // loaded together, then folded in order.
  constexpr int U = 8;
  for (int64_t i0 = 0; i0 + 1 < P; i0 += U) {
    float sv[U], av[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u;
      if (i + 1 < P) {
        const int64_t p = reverse ? P - 2 - i : i;
        sv[u] = Sloc[(p * nh + bh) * per + x];
        av[u] = aloc[p * nh + bh];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u;
      if (i + 1 < P) {
        const int64_t p = reverse ? P - 2 - i : i;
        carry = av[u] * carry + sv[u];
        Sloc[(p * nh + bh) * per + x] = carry;
      }
    }
  }
}

template <int DK, int DV>
hipError_t fwd_impl(FwdArgs args, hipStream_t stream) {
  const int64_t P = args.P;
  if (P > 1 && !args.sin_given) {
    dim3 g1((unsigned)args.nh, (unsigned)(P - 1));
    CLA_LAUNCH(args.xdot ? "chunk_dq_segments" : "chunk_fwd_segments",
               (chunk_state_kernel<DK, DV, false>), g1, dim3(NTHR), stream, args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // slots and S0 are combined elementwise; S0 is read transposed only when
    // its layout differs from the slots'
    e = launch_segment_scan(args.Sloc, args.aloc, args.S0, args.s0_trans != args.slot_trans, 0,
                            args.nh, P, DK, DV, stream);
    if (e != hipSuccess) return e;
    args.Sin = args.Sloc;
  }
  dim3 g((unsigned)args.nh, (unsigned)P);
  if (args.xdot && args.gloc && P > 1) {
    // (at DK = DV = 128 the segment-local sums come from a separate pass)
    if constexpr (DK * DV < 128 * 128) {
      CLA_LAUNCH("chunk_dq", (chunk_fwd_kernel<DK, DV, true, true>), g, dim3(NTHR), stream,
                 args);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (args.xdot) {
    CLA_LAUNCH("chunk_dq", (chunk_fwd_kernel<DK, DV, false, true>), g, dim3(NTHR), stream,
               args);
  } else {
    CLA_LAUNCH("chunk_fwd", (chunk_fwd_kernel<DK, DV, false, false>), g, dim3(NTHR), stream,
               args);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_segment_scan(float *slots, const float *aloc, const float *init,
                               int init_trans, int reverse, int64_t nh, int64_t P, int DK,
                               int DV, hipStream_t stream) {
  const int64_t n = nh * DK * DV;
  CLA_LAUNCH("chunk_segment_scan", segment_scan_kernel, dim3((unsigned)((n + 255) / 256)),
             dim3(256), stream, slots, aloc, init, init_trans, reverse, nh, P, DK, DV);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t grad_state_impl(const FwdArgs &args, hipStream_t stream) {
  CLA_LAUNCH("chunk_grad_segments", (chunk_state_kernel<DK, DV, true>),
             dim3((unsigned)args.nh, (unsigned)(args.P - 1)), dim3(NTHR), stream, args);
  return hipSuccess;
}

// The segment-local state gradients G_p (segments 1..P-1) by the GRAD state
// pass; args.k = q, args.v = dO, args.Sloc / args.aloc receive them.
hipError_t grad_state_dispatch(const FwdArgs &args, int DK, int DV, hipStream_t stream) {
  if (args.P <= 1) return hipSuccess;
  if (DK == 64 && DV == 64) return grad_state_impl<64, 64>(args, stream);
  if (DK == 64 && DV == 128) return grad_state_impl<64, 128>(args, stream);
  if (DK == 128 && DV == 64) return grad_state_impl<128, 64>(args, stream);
  if (DK == 128 && DV == 128) return grad_state_impl<128, 128>(args, stream);
  return hipErrorInvalidValue;
}

hipError_t fwd_dispatch(FwdArgs args, int DK, int DV, hipStream_t stream) {
  if (DK == 64 && DV == 64) return fwd_impl<64, 64>(args, stream);
  if (DK == 64 && DV == 128) return fwd_impl<64, 128>(args, stream);
  if (DK == 128 && DV == 64) return fwd_impl<128, 64>(args, stream);
  if (DK == 128 && DV == 128) return fwd_impl<128, 128>(args, stream);
  return hipErrorInvalidValue;
}

namespace {

// workspace carve-up for one forward-type pass
struct FwdWs {
  float *Sloc;
  float *aloc;
  size_t bytes;
};

FwdWs fwd_ws(void *base, int64_t nh, int64_t P, int64_t DK, int64_t DV) {
  FwdWs w{};
  if (P <= 1) return w;
  const size_t s_bytes = (size_t)(P - 1) * nh * DK * DV * sizeof(float);
  const size_t a_bytes = ((size_t)(P - 1) * nh * sizeof(float) + 255) & ~(size_t)255;
  w.Sloc = static_cast<float *>(base);
  w.aloc = base ? reinterpret_cast<float *>(static_cast<char *>(base) + s_bytes) : nullptr;
  w.bytes = s_bytes + a_bytes;
  return w;
}

// backward workspace: the segment states of the dQ pass (the states its
// segments start from, and the states it ends them with) and of the reverse
// pass (G at segment ends), q . dq per token and the final state S_T
struct BwdWs {
  FwdWs seg;   // dQ pass: slots p = S^T entering segment p + 1
  FwdWs gseg;  // reverse pass: slots p = G at the end of segment p
  float *Send; // dQ pass: [P-1, nh] S^T at the end of segment p, as that pass held it
  float *r1, *ST;
  size_t bytes;
};

BwdWs bwd_ws(void *base, int64_t nh, int64_t T, int64_t P, int64_t DK, int64_t DV) {
  BwdWs w{};
  w.seg = fwd_ws(base, nh, P, DK, DV);
  size_t off = w.seg.bytes;
  w.gseg = fwd_ws(base ? static_cast<char *>(base) + off : nullptr, nh, P, DK, DV);
  off += w.gseg.bytes;
  auto carve = [&](size_t bytes) -> float * {
    float *p = base ? reinterpret_cast<float *>(static_cast<char *>(base) + off) : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  w.Send = P > 1 ? carve((size_t)(P - 1) * nh * DK * DV * sizeof(float)) : nullptr;
  w.r1 = carve((size_t)nh * T * sizeof(float));
  w.ST = carve((size_t)nh * DK * DV * sizeof(float));
  w.bytes = off;
  return w;
}

}  // namespace
}  // namespace chunk

ChunkPlan plan_chunk(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV) {
  ChunkPlan plan;
  const int64_t nh = B * H;
  const int64_t nchunks = (T + chunk::TC - 1) / chunk::TC;
  plan.seg_chunks = nchunks;
  if (nh <= 0 || nchunks <= 0) return plan;
  const int64_t maxP = (nchunks + chunk::kMinSegChunks - 1) / chunk::kMinSegChunks;
  int64_t P = 1;
  if (2 * nh < chunk::kFwdSlots) {
    P = chunk::kFwdSlots / nh;  // one full round of workgroups
    if (P > maxP) P = maxP;
    if (P < 1) P = 1;
  }
  const int64_t segc = (nchunks + P - 1) / P;
  P = (nchunks + segc - 1) / segc;
  plan.P = P;
  plan.seg_chunks = segc;
  plan.ws_fwd = chunk::fwd_ws(nullptr, nh, P, DK, DV).bytes;
  int64_t Pb = 1;
  if (2 * nh < chunk::kBwdSlots) {
    Pb = chunk::kBwdSlots / nh;
    if (Pb > maxP) Pb = maxP;
    if (Pb < 1) Pb = 1;
  }
  const int64_t minPb = (nchunks + chunk::kMaxBwdSegChunks - 1) / chunk::kMaxBwdSegChunks;
  if (Pb < minPb) Pb = minPb;
  const int64_t segb = (nchunks + Pb - 1) / Pb;
  Pb = (nchunks + segb - 1) / segb;
  plan.P_b = Pb;
  plan.seg_chunks_b = segb;
  plan.ws_bwd = chunk::bwd_ws(nullptr, nh, T, Pb, DK, DV).bytes;
  plan.saved_bytes = (size_t)(Pb - 1) * nh * DK * DV * sizeof(float);
  return plan;
}

hipError_t launch_chunk_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const float *l, const float *S0, uint16_t *o, float *ST,
                            float *saved, int64_t B, int64_t H, int64_t T, int64_t DK,
                            int64_t DV, const ChunkPlan &plan, void *ws, hipStream_t stream) {
  chunk::FwdArgs args{};
  if (plan.P_b > 1) {
    args.saved = saved;
    args.save_every = plan.seg_chunks_b;
  }
  args.q = q;
  args.k = k;
  args.v = v;
  args.l = l;
  args.S0 = S0;
  args.o = o;
  args.ST = ST;
  args.nh = B * H;
  args.T = T;
  args.seg_chunks = plan.seg_chunks;
  args.P = plan.P;
  const chunk::FwdWs w = chunk::fwd_ws(ws, args.nh, plan.P, DK, DV);
  args.Sloc = w.Sloc;
  args.aloc = w.aloc;
  return chunk::fwd_dispatch(args, (int)DK, (int)DV, stream);
}

hipError_t launch_chunk_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const float *l, const float *S0, const uint16_t *dO,
                            const float *dST, const float *saved, uint16_t *dq, uint16_t *dk,
                            uint16_t *dv, float *dl, float *dS0, int64_t B, int64_t H,
                            int64_t T, int64_t DK, int64_t DV, const ChunkPlan &plan, void *ws,
                            hipStream_t stream) {
  if (plan.P_b <= 1) saved = nullptr;
  const int64_t nh = B * H;
  const chunk::BwdWs w = chunk::bwd_ws(ws, nh, T, plan.P_b, DK, DV);
  // dQ pass (forward chunk order): the forward recurrence on the transposed
  // state S^T with keys v and values k, read by dO:
  //   dQ_[j] = (dO V^T (.) D) K + diag(lambda) dO S_[j-1]^T   (LA2 Eq. 15)
  // It also yields q . dq per token and S_T for the decay gradient.
  chunk::FwdArgs fa{};
  fa.q = dO;
  fa.k = v;
  fa.v = k;
  fa.l = l;
  fa.S0 = S0;
  fa.s0_trans = 1;
  // segment states and S_T stay in this pass's own layout (S^T), written
  // and read coalesced; the dK/dV pass reads them against G^T
  fa.slot_trans = 0;
  fa.o = dq;
  fa.ST = dST ? w.ST : nullptr;
  fa.st_trans = 0;
  fa.xdot = q;
  fa.rdot = w.r1;
  fa.Sloc = w.seg.Sloc;
  fa.aloc = w.seg.aloc;
  if (saved) {
    // segments start from the forward's saved states (S, read transposed)
    fa.Sin = saved;
    fa.slot_trans = 1;
    fa.sin_given = 1;
  }
  // The dK/dV pass's segment-local G states: formed by this pass from the dO
  // and q rows it stages anyway, except at DK = DV = 128, where its state,
  // the split state operands and a second set of accumulators do not fit in
  // its registers; a separate pass over q and dO (which stops where the decay
  // from the segment start reaches 0) forms them there.
  const bool gsum_in_dq = DK * DV < 128 * 128;
  if (plan.P_b > 1 && gsum_in_dq) {
    fa.gloc = w.gseg.Sloc;
    fa.galoc = w.gseg.aloc;
  }
  if (plan.P_b > 1) {
    // the state each segment ends with, for the boundary terms of the decay
    // gradient (the states the segments start from were formed apart from
    // this pass, by the segment pass and scan or by the forward)
    fa.Send = w.Send;
  }
  fa.nh = nh;
  fa.T = T;
  fa.seg_chunks = plan.seg_chunks_b;
  fa.P = plan.P_b;
  hipError_t e = chunk::fwd_dispatch(fa, (int)DV, (int)DK, stream);
  if (e != hipSuccess) return e;
  if (plan.P_b > 1 && !gsum_in_dq) {
    chunk::FwdArgs ga{};
    ga.k = q;
    ga.v = dO;
    ga.l = l;
    ga.Sloc = w.gseg.Sloc;
    ga.aloc = w.gseg.aloc;
    ga.nh = nh;
    ga.T = T;
    ga.seg_chunks = plan.seg_chunks_b;
    ga.P = plan.P_b;
    e = chunk::grad_state_dispatch(ga, (int)DK, (int)DV, stream);
    if (e != hipSuccess) return e;
  }
  // dK/dV pass (reverse chunk order)
  chunk::BwdArgs ba{};
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.dO = dO;
  ba.l = l;
  ba.dST = dST;
  ba.dk = dk;
  ba.dv = dv;
  ba.r1 = w.r1;
  ba.dl = dl;
  ba.dS0 = dS0;
  ba.Gloc = w.gseg.Sloc;
  ba.aloc = w.gseg.aloc;
  ba.Sseg = w.Send;
  ba.STb = dST ? w.ST : nullptr;
  ba.nh = nh;
  ba.T = T;
  ba.seg_chunks = plan.seg_chunks_b;
  ba.P = plan.P_b;
  e = chunk::bwd_kv_dispatch(ba, (int)DK, (int)DV, stream);
  if (e != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace cla
