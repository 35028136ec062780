// Chunkwise linear attention with one decay per key dimension, backward pass,
// for gfx950.
//
// Citations (page title, then section):
//   ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
//
// ZTF "The backward pass of linear attention" with the diagonal decay: the
// adjoint obeys Sbar_t = q_t dO_t^T + diag(a_{t+1}) Sbar_{t+1}; a query's
// gradient needs the forward state (a sweep in time order), a key's, value's
// and decay's the adjoint (a sweep in reverse).  Chunkwise, with the in-chunk
// cumulative logs c and the sub-block factors of the forward (gla.hip):
//   dq_r[d] = sum_{s <= r} B[r, s] k_s[d] exp(c_r[d] - c_s[d])
//             + exp(c_r[d]) (S dO_r)[d],                B[r, s] = dO_r . v_s
//   dk_s[d] = sum_{r >= s} B[r, s] q_r[d] exp(c_r[d] - c_s[d])
//             + exp(c_n[d] - c_s[d]) (G v_s)[d]
//   dv_s    = sum_{r >= s} A[r, s] dO_r + sum_d k_s[d] exp(c_n[d] - c_s[d]) G[d, :]
//   G      <- diag(exp(c_n)) G + (q (.) exp(c))^T dO    (state gradient entering the chunk)
// with A the forward's decayed scores and G the gradient of the state after
// the chunk.  The decay gradient is the closed form of ZTF for a vector of
// decays (Yang et al. 2023, Section 4.3), per key dimension:
//   dl_u[d] = sum_{t >= u} (q_t[d] dq_t[d] - k_t[d] dk_t[d]) + paths past the end,
// evaluated in segments of 16 chunks: the suffix sums run inside a segment
// only and start from the exact term <S[d, :], G[d, :]> of the two fp32 states
// at the segment's end (the dQ pass saves S there), so no long sum of
// cancelling terms builds up.  Inside a chunk, most paths do not cross a given
// step and must cancel between the two sums; both passes therefore form the
// in-chunk contributions to q dq and k dk from the same rounded operands: one
// 16-deep MFMA per pair of 16-token blocks (Qh^T B or Kh^T B^T), the block
// factor applied in fp32 after it, and q dq = Qh (.) that, k dk = Kh (.) that.
//
// dQ pass: one wave per 16 key dimensions; wave w owns dq columns d in
// [16 w, 16 w + 16) and the same columns of the state, kept transposed (S^T)
// in MFMA accumulators.
// dK/dV pass: 8 waves holding value columns of G (for dv) and key columns of
// G^T (for dk and the decay gradient): at DK = DV = 128 each wave 16 of both,
// otherwise waves 0-3 the value columns and waves 4-7 the key columns.  Both
// copies are updated every chunk, as in the scalar kernel.  One workgroup per
// sequence-head, one per CU (LDS ~146 KB and ~158 KB at DK = DV = 128).
#include "chunk_common.h"
#include "gla_kernels.h"
#include "internal.h"

namespace cla {
namespace gla {

using namespace cla::chunk;

namespace {

constexpr float kBadLog = 60.f * kLog2e;  // e^-60, as in the forward (base-2 units)
constexpr int BTHR = 512;

// v_mfma_f32_16x16x16_bf16: lane 16 lg + li holds A row li and B column li,
// k-values 4 lg .. 4 lg + 3; C as for the 32-deep instruction.
typedef short __attribute__((ext_vector_type(4))) s16x4;
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Lane exchange within 16-lane rows (DPP, no LDS).  row_shl:n: lane i reads
// lane i + n of its row, 0 past the row's end; row_newbcast:0: every lane
// reads its row's lane 0.
template <int CTRL>
__device__ __forceinline__ float row_dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// One path of the in-chunk score product, write s -> read t through key
// dimension d: both passes form it with this same expression, so that the
// decay gradient's two sums hold the same numbers and the paths that do not
// cross a step cancel in it up to fp32 summation order.
__device__ __forceinline__ float path_term(float b, float q, float k, float ct, float cs) {
  return ((b * q) * k) * exp_c(ct - cs);
}

// DMA of the [64 x D] fp32 log tile in the swizzled layout of csx: 1 KB
// blocks of RPB rows; rows past the chunk re-read row n - 1.
template <int D>
__device__ __forceinline__ const float *dma_f32_rows_src(const float *chunk_src, int n, int block,
                                                         int lane) {
  constexpr int PPR = D / 4;
  constexpr int RPB = 64 / PPR;
  const int row = block * RPB + lane / PPR;
  const int grow = min(row, n - 1);
  // this lane lands at piece lane % PPR of the row: it fetches the piece the
  // row's swizzle puts there
  return chunk_src + (int64_t)grow * D + (((lane % PPR) ^ (row & 15)) * 4);
}

template <int D>
__device__ __forceinline__ void dma_f32_rows(const float *chunk_src, int n, unsigned char *tile,
                                             int block, int lane) {
  __builtin_amdgcn_global_load_lds(dma_f32_rows_src<D>(chunk_src, n, block, lane),
                                   (lds_void *)(tile + block * 1024), 16, 0, 0);
}

// ---------------------------------------------------------------------------
// Register staging of a chunk's inputs.  A workgroup's LDS holds one chunk
// (there is no room for a second), so the next chunk is fetched into
// registers while the current one is worked on and written to LDS between
// the two.  The LDS layout is the 1 KB-block layout of the DMA staging of the
// scalar kernels (lane i holds bytes 16 i .. 16 i + 15 of its block): q, k,
// v, dO as swizzled bf16 tiles, then the [64 x DK] fp32 log rows (swizzled as
// csx describes).
// Wave w holds blocks w, w + NW, ...; each tensor's block count is a multiple
// of NW, so the tensor of every held block is known at compile time.  Rows
// past the chunk's n tokens re-read row n - 1 (finite data, masked later).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ uint4 fetch_bf16_block(const uint16_t *chunk_src, int n, int block,
                                                  int lane) {
  constexpr int NCH = D / 8;
  constexpr int RPB = 64 / NCH;
  const int row = block * RPB + lane / NCH;
  const int c = (lane % NCH) ^ swz_pat(row);
  const int grow = min(row, n - 1);
  return *reinterpret_cast<const uint4 *>(chunk_src + (int64_t)grow * D + c * 8);
}

template <int D>
__device__ __forceinline__ uint4 fetch_f32_block(const float *chunk_src, int n, int block,
                                                 int lane) {
  constexpr int PPR = D / 4;     // 16-byte pieces per row
  constexpr int RPB = 64 / PPR;  // rows per 1 KB block
  const int row = block * RPB + lane / PPR;
  const int grow = min(row, n - 1);
  return *reinterpret_cast<const uint4 *>(chunk_src + (int64_t)grow * D +
                                          (((lane % PPR) ^ (row & 15)) * 4));
}

template <int DK, int DV, int NW>
struct ChunkRegs {
  static constexpr int NBQ = DK / 8, NBV = DV / 8, NBL = DK / 4;
  static_assert(NBQ % NW == 0 && NBV % NW == 0 && NBL % NW == 0, "whole rounds per tensor");
  static constexpr int NPF = (2 * NBQ + 2 * NBV + NBL) / NW;
  uint4 r[NPF];

  // tokens [t0, t0 + n) of one sequence-head (pointers at its first token)
  __device__ __forceinline__ void fetch(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                        const uint16_t *dO, const float *l, int64_t t0, int n,
                                        int w, int lane) {
#pragma unroll
    for (int x = 0; x < NPF; ++x) {
      const int r0 = NW * x;  // first block of this round
      const int b = w + r0;
      if (r0 < NBQ)
        r[x] = fetch_bf16_block<DK>(q + t0 * DK, n, b, lane);
      else if (r0 < 2 * NBQ)
        r[x] = fetch_bf16_block<DK>(k + t0 * DK, n, b - NBQ, lane);
      else if (r0 < 2 * NBQ + NBV)
        r[x] = fetch_bf16_block<DV>(v + t0 * DV, n, b - 2 * NBQ, lane);
      else if (r0 < 2 * NBQ + 2 * NBV)
        r[x] = fetch_bf16_block<DV>(dO + t0 * DV, n, b - 2 * NBQ - NBV, lane);
      else
        r[x] = fetch_f32_block<DK>(l + t0 * DK, n, b - 2 * NBQ - 2 * NBV, lane);
    }
  }

  __device__ __forceinline__ void store(unsigned char *QS, unsigned char *KS, unsigned char *VS,
                                        unsigned char *DOS, unsigned char *CS, int w,
                                        int lane) const {
#pragma unroll
    for (int x = 0; x < NPF; ++x) {
      const int r0 = NW * x;
      const int b = w + r0;
      unsigned char *dst;
      if (r0 < NBQ)
        dst = QS + b * 1024;
      else if (r0 < 2 * NBQ)
        dst = KS + (b - NBQ) * 1024;
      else if (r0 < 2 * NBQ + NBV)
        dst = VS + (b - 2 * NBQ) * 1024;
      else if (r0 < 2 * NBQ + 2 * NBV)
        dst = DOS + (b - 2 * NBQ - NBV) * 1024;
      else
        dst = CS + (b - 2 * NBQ - 2 * NBV) * 1024;
      *reinterpret_cast<uint4 *>(dst + lane * 16) = r[x];
    }
  }
};

// In-chunk cumulative logs, in place, with NTH threads (rows past n: no decay).
template <int DK, int NTH>
__device__ __forceinline__ void cumsum_rows(float *CS, int n, int tid) {
  cumsum_rows_dpp<DK, NTH>(CS, n, tid);
  lds_barrier();
}

// Scaled copies: Qh = q exp(c - cb_R) (if QH), Kh = k exp(ce_S - c), both 0 on
// rows past the chunk (which hold copies of its last row), and the per-block
// factor rows FQ[R] = exp(cb_R), FK[S] =
// exp(c_n - ce_S), AL = exp(c_n).
template <int DK, int NTH>
__device__ __forceinline__ void prep_scaled(const unsigned char *QS, const unsigned char *KS,
                                            unsigned char *QH, unsigned char *KH, const float *CS,
                                            float *FQ, float *FK, float *AL, int n, int tid) {
  constexpr int NCK = DK / 8;
  // each thread takes RPT rows of one 16-row block (one 8-column group), so
  // it reads the block's boundary logs once
  constexpr int RPT = 64 * NCK / NTH, SPB = 16 / RPT;
  static_assert(RPT * NTH == 64 * NCK && SPB * RPT == 16, "whole rounds in one block");
  {
    const int c8 = tid % NCK, q = tid / NCK;
    const int B = q / SPB, i0 = q % SPB;
    const int re = 16 * B + 15, rb = 16 * B - 1;
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
      const bf16x8 kv = *reinterpret_cast<const bf16x8 *>(KS + off);
      float yk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) yk[e] = r < n ? tof(kv[e]) * exp_c(ce8[e] - cr8[e]) : 0.f;
      *reinterpret_cast<bf16x8 *>(KH + off) = cvt8(yk);
      if (QH) {
        const bf16x8 qv = *reinterpret_cast<const bf16x8 *>(QS + off);
        float yq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) yq[e] = r < n ? tof(qv[e]) * exp_c(cr8[e] - cb8[e]) : 0.f;
        *reinterpret_cast<bf16x8 *>(QH + off) = cvt8(yq);
      }
    }
  }
  for (int d = tid; d < DK; d += NTH) {
    float ce[4];
#pragma unroll
    for (int B = 0; B < 4; ++B) ce[B] = CS[csx<DK>(16 * B + 15, d)];
#pragma unroll
    for (int B = 0; B < 4; ++B) {
      FQ[B * DK + d] = B > 0 ? exp_c(ce[B - 1]) : 1.f;
      FK[B * DK + d] = exp_c(ce[3] - ce[B]);
    }
    AL[d] = exp_c(ce[3]);
  }
}

// index of the block pair (R, S), S <= R, in 0..9
__device__ __forceinline__ int pair_index(int R, int S) { return R * (R + 1) / 2 + S; }

// The block factors exp(cb_R - ce_S) of the 10 pairs S <= R for every key
// dimension, FT[pair][d], formed once per chunk for all lanes (a diagonal
// block past the decay limit is skipped by its users, not zeroed here).
template <int DK, int NTH>
__device__ __forceinline__ void block_factors(const float *CS, float *FT, int tid) {
  for (int g = tid; g < 10 * DK; g += NTH) {
    const int p = g / DK, d = g % DK;
    const int R = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
    const int S = p - R * (R + 1) / 2;
    const float cb = R > 0 ? CS[csx<DK>(16 * R - 1, d)] : 0.f;
    FT[g] = exp_c(cb - CS[csx<DK>(16 * S + 15, d)]);
  }
}

// Bit R set: block R of the chunk decays below e^-60 in some dimension
// (wave-uniform; formed once per chunk from the four block-end rows)
template <int DK>
__device__ __forceinline__ uint32_t bad_blocks(const float *CS, int lane) {
  uint32_t mask = 0;
#pragma unroll
  for (int R = 0; R < 4; ++R) {
    bool bad = false;
#pragma unroll
    for (int d0 = 0; d0 < DK; d0 += 64) {
      const int d = d0 + lane;
      const float cb = R > 0 ? CS[csx<DK>(16 * R - 1, d)] : 0.f;
      bad |= cb - CS[csx<DK>(16 * R + 15, d)] > kBadLog;
    }
    if (__ballot(bad) != 0) mask |= 1u << R;
  }
  return mask;
}

// ===========================================================================
// dQ pass
// ===========================================================================

// One wave per 16 key dimensions (DK = 128: 8 waves, two per SIMD, which
// hides the latency of each phase better than one wave per SIMD).
template <int DK>
constexpr int dq_threads() {
  return 4 * DK;
}

template <int DK, int DV>
__global__ __launch_bounds__(dq_threads<DK>(), 1) void gla_dq_kernel(GlaBwdArgs a) {
  constexpr int NCK = DK / 8, NCV = DV / 8;
  constexpr int NT = dq_threads<DK>(), NW = NT / 64;
  constexpr int NDT = DK / (16 * NW);  // 16-column d tiles per wave
  static_assert(NDT == 1, "one d tile per wave");
  constexpr int NJT = DV / 16;  // 16-row j tiles of S^T
  constexpr int B_KS = 64 * DK * 2, B_KH = 2 * B_KS, B_VS = 3 * B_KS;
  constexpr int B_DO = B_VS + 64 * DV * 2, B_CS = B_DO + 64 * DV * 2;
  constexpr int B_BS = B_CS + 64 * DK * 4, B_FQ = B_BS + 64 * 64 * 2;
  constexpr int B_FK = B_FQ + 4 * DK * 4, B_AL = B_FK + 4 * DK * 4;
  constexpr int B_FT = B_AL + DK * 4;
  constexpr int BUF = B_FT + 10 * DK * 4;
  static_assert(BUF <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char buf[BUF];
  unsigned char *QS = buf, *KS = buf + B_KS, *KH = buf + B_KH;
  unsigned char *VS = buf + B_VS;
  unsigned char *DOS = buf + B_DO, *BS = buf + B_BS;
  float *CS = reinterpret_cast<float *>(buf + B_CS);
  float *FQ = reinterpret_cast<float *>(buf + B_FQ);
  float *FK = reinterpret_cast<float *>(buf + B_FK);
  float *AL = reinterpret_cast<float *>(buf + B_AL);
  float *FT = reinterpret_cast<float *>(buf + B_FT);

  const int tid0 = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
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
  const int d0 = w * (DK / NW);
  const uint16_t *qh = a.q + bh * T * DK;
  const uint16_t *kh = a.k + bh * T * DK;
  const uint16_t *vh = a.v + bh * T * DV;
  const uint16_t *doh = a.dO + bh * T * DV;
  const float *lh = a.l + bh * T * DK;

  // ST_acc[jt][dt][i] = S^T[16 jt + 4 lg + i][d0 + 16 dt + li] = S[d][j]
  f32x4 ST_acc[NJT][NDT];
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      ST_acc[jt][dt] = zero4();
      // the state this segment starts from: S0, or the scanned segment state
      const float *src = seg == 0 ? (a.S0 ? a.S0 + bh * DK * DV : nullptr)
                                  : a.Sin + ((seg - 1) * a.nh + bh) * DK * DV;
      if (src) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ST_acc[jt][dt][i] = src[(d0 + 16 * dt + li) * DV + 16 * jt + 4 * lg + i];
      }
    }
  // segments after the first: the local adjoint state sum_t diag(A_t) q_t dO_t^T
  // (A_t the decay from the segment's start through step t), laid out as
  // ST_acc, and the running decay from the segment's start to the chunk
  const bool gsum = a.P > 1 && seg > 0;
  f32x4 G_acc[NJT][NDT];
  float apre[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    apre[dt] = 1.f;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) G_acc[jt][dt] = zero4();
  }

  // the first chunk's inputs; every step then fetches the next one
  ChunkRegs<DK, DV, NW> stage;
  stage.fetch(qh, kh, vh, doh, lh, c_begin * TC, (int)min<int64_t>(TC, T - c_begin * TC), w, lane);
  for (int64_t ci = c_begin; ci < c_end; ++ci) {
    const int64_t t0 = ci * TC;
    const int n = (int)min<int64_t>(TC, T - t0);

    lds_barrier();  // the previous chunk's LDS reads are done
    FRESH_LANE();
    stage.store(QS, KS, VS, DOS, buf + B_CS, w, lane);
    if (ci + 1 < c_end)
      stage.fetch(qh, kh, vh, doh, lh, t0 + TC, (int)min<int64_t>(TC, T - t0 - TC), w, lane);
    lds_barrier();
    FRESH_LANE();
    cumsum_rows<DK, NT>(CS, n, tid);
    const uint32_t bad_mask = bad_blocks<DK>(CS, lane);
    FRESH_LANE();
    // (no Qh copy: this pass needs only this lane's few Qh values, re-formed
    // where they are used)
    prep_scaled<DK, NT>(QS, KS, nullptr, KH, CS, FQ, FK, AL, n, tid);
    block_factors<DK, NT>(CS, FT, tid);

    // ---- B[r][s] = dO_r . v_s (masked), stored [r][s]; the 32-column steps
    // read up to the diagonal also cover tiles (0,1) and (2,3): zeros ----
    FRESH_LANE();
    for (int t = w; t < 12; t += NW) {
      const int R = tile_rt(t), S = tile_st(t);
      f32x4 acc = zero4();
      if (S <= R) {
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk)
          acc = mfma(lds_frag<NCV>(VS, 16 * S + li, 4 * kk + lg),
                     lds_frag<NCV>(DOS, 16 * R + li, 4 * kk + lg), acc);
      }
      bf16x4 pv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * R + li, s = 16 * S + 4 * lg + i;
        pv[i] = tobf(s <= r && s < n && r < n ? acc[i] : 0.f);
      }
      *reinterpret_cast<bf16x4 *>(BS + swz_off<8>(16 * R + li, 2 * S + (lg >> 1)) + (lg & 1) * 8) =
          pv;
    }
    lds_barrier();

    // ---- dq^T[d][r] for this wave's columns d ----
    {
      FRESH_LANE();
      bf16x8 sfrag[DV / 32][NDT];  // S as A operands: row d, k = j (permuted)
#pragma unroll
      for (int kk = 0; kk < DV / 32; ++kk)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) sfrag[kk][dt] = cvt8(ST_acc[2 * kk][dt], ST_acc[2 * kk + 1][dt]);
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const bool good = !((bad_mask >> R) & 1u);
        const int r = 16 * R + li;
        bf16x8 dofrag[DV / 32];  // dO^T B operands: k = j (same permutation), n = r
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk)
          dofrag[kk] = cat8(lds_half<NCV>(DOS, r, 32 * kk + 4 * lg),
                            lds_half<NCV>(DOS, r, 32 * kk + 16 + 4 * lg));
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int dc = d0 + 16 * dt + 4 * lg;  // this lane's 4 output d's
          // in-chunk part: sum over blocks S <= R of F_RS (Kh_S^T B_RS^T), one
          // 16-deep product per block, the factor applied after it
          f32x4 accI = zero4();
#pragma unroll
          for (int S = 0; S <= R; ++S) {
            if (S == R && !good) break;  // done elementwise below
            f32x4 P = zero4();
            P = mfma16(tr_read4<NCK>(KH, 16 * S + 4 * lg, d0 + 16 * dt, li),  // Kh^T: row d, k = s
                       lds_half<8>(BS, r, 16 * S + 4 * lg), P);                // B: k = s, col t
            const f32x4 F = *reinterpret_cast<const f32x4 *>(FT + pair_index(R, S) * DK + dc);
#pragma unroll
            for (int i = 0; i < 4; ++i) accI[i] += F[i] * P[i];
          }
          f32x4 acc2 = zero4();
#pragma unroll
          for (int kk = 0; kk < DV / 32; ++kk) acc2 = mfma(sfrag[kk][dt], dofrag[kk], acc2);
          // accI[i], acc2[i] at d = dc + i, row t = r
          const bf16x4 qv = lds_half<NCK>(QS, min(r, 63), dc);
          // this lane's 4 dimensions are one 16-byte piece of each row (dc is
          // a multiple of 4): read as such, not as 4 separate words
          const f32x4 cbv = R > 0 ? *reinterpret_cast<const f32x4 *>(CS + csx<DK>(16 * R - 1, dc))
                                  : zero4();
          const f32x4 crv = *reinterpret_cast<const f32x4 *>(CS + csx<DK>(r, dc));
          const f32x4 fqv = *reinterpret_cast<const f32x4 *>(FQ + R * DK + dc);
          float out[4], r1v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = dc + i;
            const float u = exp_c(crv[i] - cbv[i]);
            // Q-hat exactly as the scaled copy of the dK/dV pass forms it
            // (same factor, same rounding), so the in-chunk paths cancel
            // against k.dk there
            const float qhd = tof(tobf(tof(qv[i]) * u));
            const float inter = fqv[i] * acc2[i] * u;
            float v = accI[i] * u + inter;
            float rv = qhd * accI[i] + tof(qv[i]) * inter;
            if (!good) {
              // the block's own tokens, elementwise
              const float qd = tof(qv[i]);
              const int sr = min(r, n - 1);
              for (int s2 = 16 * R; s2 <= sr; ++s2) {
                const float bsc = tof(*reinterpret_cast<const __bf16 *>(
                    BS + swz_off<8>(r, s2 >> 3) + (s2 & 7) * 2));
                const float kd = tof(*reinterpret_cast<const __bf16 *>(
                    KS + swz_off<NCK>(s2, d >> 3) + (d & 7) * 2));
                v += (bsc * kd) * exp_c(CS[csx<DK>(r, d)] - CS[csx<DK>(s2, d)]);
                rv += path_term(bsc, qd, kd, CS[csx<DK>(r, d)], CS[csx<DK>(s2, d)]);
              }
            }
            out[i] = v;
            r1v[i] = rv;
          }
          if (r < n) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = tobf(out[i]);
            *reinterpret_cast<bf16x4 *>(a.dq + (bh * T + t0 + r) * DK + dc) = ov;
            f32x4 r1;
#pragma unroll
            for (int i = 0; i < 4; ++i) r1[i] = r1v[i];
            *reinterpret_cast<f32x4 *>(a.r1 + (bh * T + t0 + r) * DK + dc) = r1;
          }
        }
      }
    }

    // ---- state update: S^T <- S^T diag(alpha) + V^T KG, KG = k e^{c_n - c_s}
    // formed in fp32 and applied as two bf16 parts (hi + lo), so that the
    // state at a segment's end holds the chunk's paths to fp32-level accuracy:
    // the decay gradient pairs it with the same paths summed from k.dk ----
    {
      FRESH_LANE();
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const float al = AL[d0 + 16 * dt + li];
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
          for (int i = 0; i < 4; ++i) ST_acc[jt][dt][i] *= al;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 kg[NDT], kl[NDT];  // KG B operands (hi, lo): k = s, column d
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int d = d0 + 16 * dt + li;
          const bf16x8 x = tr_frag<NCK>(KS, 32 * kb, d0 + 16 * dt, li, lg);
          const float cn = CS[csx<DK>(63, d)];
          float y[8], z[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int s = 32 * kb + 8 * lg + e;
            y[e] = s < n ? tof(x[e]) * exp_c(cn - CS[csx<DK>(s, d)]) : 0.f;
          }
          kg[dt] = cvt8(y);
#pragma unroll
          for (int e = 0; e < 8; ++e) z[e] = y[e] - tof(kg[dt][e]);
          kl[dt] = cvt8(z);
        }
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          const bf16x8 va = tr_frag<NCV>(VS, 32 * kb, 16 * jt, li, lg);  // V^T: row j, k = s
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            ST_acc[jt][dt] = mfma(va, kg[dt], ST_acc[jt][dt]);
            ST_acc[jt][dt] = mfma(va, kl[dt], ST_acc[jt][dt]);
          }
        }
      }
    }

    // ---- the segment's local adjoint state: G^T += dO^T (A (.) Q) ----
    if (gsum) {
      FRESH_LANE();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 qa[NDT];  // (A (.) Q) B operands: k = t, column d
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int d = d0 + 16 * dt + li;
          const bf16x8 x = tr_frag<NCK>(QS, 32 * kb, d0 + 16 * dt, li, lg);
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = 32 * kb + 8 * lg + e;
            y[e] = t < n ? tof(x[e]) * (apre[dt] * exp_c(CS[csx<DK>(t, d)])) : 0.f;
          }
          qa[dt] = cvt8(y);
        }
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          const bf16x8 da = tr_frag<NCV>(DOS, 32 * kb, 16 * jt, li, lg);  // dO^T: row j, k = t
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) G_acc[jt][dt] = mfma(da, qa[dt], G_acc[jt][dt]);
        }
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) apre[dt] *= AL[d0 + 16 * dt + li];
    }

    // ---- the state at the end of each 16-chunk block (and of the sequence) ----
    if ((ci + 1) % kSegChunks == 0 || ci + 1 == nchunks) {
      FRESH_LANE();
      float *dst = a.Sseg + ((ci / kSegChunks) * a.nh + bh) * DK * DV;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<f32x4 *>(dst + (d0 + 16 * dt + li) * DV + 16 * jt + 4 * lg) =
              ST_acc[jt][dt];
    }
  }
  if (gsum) {
    FRESH_LANE();
    float *dst = a.Gloc + (seg * a.nh + bh) * DK * DV;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4 *>(dst + (d0 + 16 * dt + li) * DV + 16 * jt + 4 * lg) =
            G_acc[jt][dt];
    if (lg == 0) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) a.Aq[(seg * a.nh + bh) * DK + d0 + 16 * dt + li] = apre[dt];
    }
  }
}
#undef FRESH_LANE

// ===========================================================================
// dK/dV pass
// ===========================================================================

// Score tiles of the dK/dV pass per wave, one byte per job (0xFF: none):
// tile t (tile_rt / tile_st) of the decayed A (t) or of B (16 + t).  An A
// tile scales its K-hat operand by the block factors, about twice a B tile's
// work; waves 0-1 take two A tiles, waves 2-7 one A and two B tiles, and the
// two structurally zero tiles of each kind (t = 10, 11) go to waves 6 and 7.
__constant__ uint32_t kScoreJobs[8] = {0xFFFF0100u, 0xFFFF0302u, 0xFF111004u, 0xFF131205u,
                                       0xFF151406u, 0xFF171607u, 0x1A0A1808u, 0x1B0B1909u};

template <int DK, int DV>
__global__ __launch_bounds__(BTHR, 1) void gla_dkdv_kernel(GlaBwdArgs a) {
  constexpr int NCK = DK / 8, NCV = DV / 8;
  // At DK = DV = 128 every wave takes one 16-column tile of each product:
  // value columns j0 = 16 w of dv and key dimensions d0 = 16 w of dk (the dk
  // side's per-element work, the larger, is then spread over all eight waves).
  // Otherwise waves 0-3 take dv and waves 4-7 dk.
  constexpr bool MIX = DK == 128 && DV == 128;
  constexpr int NJ = MIX ? 1 : DV / 64;  // dv: 16-column j tiles per wave
  constexpr int NI = MIX ? 1 : DK / 64;  // dk: 16-column d tiles per wave
  constexpr int NG0 = DK / 16 * NJ;       // tiles of G held for dv
  constexpr int NG = MIX ? NG0 + DV / 16 * NI : NG0;
  constexpr int NRED = MIX ? 8 : 4;       // partial sums of the boundary term per d
  constexpr int B_KS = 64 * DK * 2, B_QH = 2 * B_KS, B_KH = 3 * B_KS, B_VS = 4 * B_KS;
  constexpr int B_DO = B_VS + 64 * DV * 2, B_CS = B_DO + 64 * DV * 2;
  constexpr int B_AS = B_CS + 64 * DK * 4, B_BS = B_AS + 8192;
  constexpr int B_FQ = B_BS + 8192, B_FK = B_FQ + 4 * DK * 4, B_AL = B_FK + 4 * DK * 4;
  constexpr int B_RED = B_AL + DK * 4;
  constexpr int B_FT = B_RED + NRED * DK * 4;
  constexpr int BUF = B_FT + 10 * DK * 4;
  constexpr int NBQ = DK / 8, NBV = DV / 8, NBL = DK / 4;
  static_assert(BUF <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char buf[BUF];
  unsigned char *QS = buf, *KS = buf + B_KS, *QH = buf + B_QH, *KH = buf + B_KH;
  unsigned char *VS = buf + B_VS, *DOS = buf + B_DO, *AS = buf + B_AS, *BS = buf + B_BS;
  float *CS = reinterpret_cast<float *>(buf + B_CS);
  float *FQ = reinterpret_cast<float *>(buf + B_FQ);
  float *FK = reinterpret_cast<float *>(buf + B_FK);
  float *AL = reinterpret_cast<float *>(buf + B_AL);
  float *RED = reinterpret_cast<float *>(buf + B_RED);
  float *FT = reinterpret_cast<float *>(buf + B_FT);

  const int tid0 = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  const int side = w >> 2, wv = w & 3;
  const bool do_dv = MIX || side == 0, do_dk = MIX || side == 1;
  const int rw = MIX ? w : wv;  // this wave's row of boundary-term partials
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
  const int j0 = MIX ? 16 * w : wv * (DV / 4);  // dv columns
  const int d0 = MIX ? 16 * w : wv * (DK / 4);  // dk dimensions
  const uint16_t *qh = a.q + bh * T * DK;
  const uint16_t *kh = a.k + bh * T * DK;
  const uint16_t *vh = a.v + bh * T * DV;
  const uint16_t *doh = a.dO + bh * T * DV;
  const float *lh = a.l + bh * T * DK;

  // dv: G0(dt, jt)[i] = G[16 dt + 4 lg + i][j0 + 16 jt + li]
  // dk: G1(jt, it)[i] = G^T[16 jt + 4 lg + i][d0 + 16 it + li]
  f32x4 Gs[NG];
#define G0(dt, jt) Gs[(dt) * NJ + (jt)]
#define G1(jt, it) Gs[(MIX ? NG0 : 0) + (jt) * NI + (it)]
#pragma unroll
  for (int x = 0; x < NG; ++x) Gs[x] = zero4();
  // the adjoint state at this segment's end: dS_T, or the reverse scan's
  const float *gsrc = seg == a.P - 1 ? (a.dST ? a.dST + bh * DK * DV : nullptr)
                                     : a.Gloc + ((seg + 1) * a.nh + bh) * DK * DV;
  if (gsrc) {
    const float *src = gsrc;
    if (do_dv) {
#pragma unroll
      for (int dt = 0; dt < DK / 16; ++dt)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            G0(dt, jt)[i] = src[(16 * dt + 4 * lg + i) * DV + j0 + 16 * jt + li];
    }
    if (do_dk) {
#pragma unroll
      for (int jt = 0; jt < DV / 16; ++jt)
#pragma unroll
        for (int it = 0; it < NI; ++it)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            G1(jt, it)[i] = src[(d0 + 16 * it + li) * DV + 16 * jt + 4 * lg + i];
    }
  }
  // dk: the running suffix sum of q.dq - k.dk for its dimensions
  // d0 + 16 it + 4 lg + i (the same in every lane of a 16-lane row)
  float carry[NI][4];
#pragma unroll
  for (int it = 0; it < NI; ++it)
#pragma unroll
    for (int i = 0; i < 4; ++i) carry[it][i] = 0.f;

  // Staging: k, v and the logs of a chunk are copied during the previous
  // chunk's state update (which reads none of them), q and dO (which it
  // reads) at the chunk's start; all by untracked copies, waited for at the
  // chunk's start.
  auto stage_kvl = [&](int64_t cj) __attribute__((always_inline)) {
    const int64_t tj = cj * TC;
    const int nj = (int)min<int64_t>(TC, T - tj);
    for (int b = w; b < NBQ + NBV + NBL; b += BTHR / 64) {
      if (b < NBQ)
        lds_copy16_untracked(bf16_block_src<DK>(kh + tj * DK, nj, b, lane), KS + b * 1024);
      else if (b < NBQ + NBV)
        lds_copy16_untracked(bf16_block_src<DV>(vh + tj * DV, nj, b - NBQ, lane),
                             VS + (b - NBQ) * 1024);
      else
        lds_copy16_untracked(dma_f32_rows_src<DK>(lh + tj * DK, nj, b - NBQ - NBV, lane),
                             buf + B_CS + (b - NBQ - NBV) * 1024);
    }
  };
  if (c_end > c_begin) {
    FRESH_LANE();
    stage_kvl(c_end - 1);
  }
  for (int64_t ci = c_end - 1; ci >= c_begin; --ci) {
    const int64_t t0 = ci * TC;
    const int n = (int)min<int64_t>(TC, T - t0);

    // ---- at a segment's end: carry = <S[d, :], G[d, :]> (dv waves' sums), with
    // G rounded to bf16 as the dK product below takes it: the paths from this
    // chunk past the segment end then cancel against k.dk term by term ----
    if ((ci + 1) % kSegChunks == 0 || ci + 1 == nchunks) {
      FRESH_LANE();
      if (do_dv) {
        const float *Sg = a.Sseg + ((ci / kSegChunks) * a.nh + bh) * DK * DV;
#pragma unroll
        for (int dt = 0; dt < DK / 16; ++dt) {
          f32x4 p;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float s = 0.f;
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
              s += tof(tobf(G0(dt, jt)[i])) * Sg[(16 * dt + 4 * lg + i) * DV + j0 + 16 * jt + li];
            // sum over the 16 lanes of this row group (the columns li)
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
            p[i] = s;
          }
          if (li == 0) *reinterpret_cast<f32x4 *>(RED + rw * DK + 16 * dt + 4 * lg) = p;
        }
      }
      lds_barrier();
      if (do_dk) {
#pragma unroll
        for (int it = 0; it < NI; ++it)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = d0 + 16 * it + 4 * lg + i;
            float c = RED[d];
#pragma unroll
            for (int u = 1; u < NRED; ++u) c += RED[u * DK + d];
            carry[it][i] = c;
          }
      }
    }

    lds_barrier();
    FRESH_LANE();
    for (int b = w; b < NBQ + NBV; b += BTHR / 64) {
      if (b < NBQ)
        lds_copy16_untracked(bf16_block_src<DK>(qh + t0 * DK, n, b, lane), QS + b * 1024);
      else
        lds_copy16_untracked(bf16_block_src<DV>(doh + t0 * DV, n, b - NBQ, lane),
                             DOS + (b - NBQ) * 1024);
    }
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    // this lane's q.dq (rows s = 16 S + li, its 4 dimensions of each d tile),
    // loaded here so that the phases before the dk side hide their latency
    f32x4 r1b[4][NI];
    if (do_dk) {
      FRESH_LANE();
#pragma unroll
      for (int S = 0; S < 4; ++S)
#pragma unroll
        for (int it = 0; it < NI; ++it) {
          const int s = 16 * S + li;
          r1b[S][it] = s < n ? *reinterpret_cast<const f32x4 *>(
                                   a.r1 + (bh * T + t0 + s) * DK + d0 + 16 * it + 4 * lg)
                             : zero4();
        }
    }
    FRESH_LANE();
    cumsum_rows<DK, BTHR>(CS, n, tid);
    const uint32_t bad_mask = bad_blocks<DK>(CS, lane);
    FRESH_LANE();
    prep_scaled<DK, BTHR>(QS, KS, QH, KH, CS, FQ, FK, AL, n, tid);
    block_factors<DK, BTHR>(CS, FT, tid);
    lds_barrier();

    // ---- scores, stored transposed [s][r]: the decayed A and B ----
    {
      FRESH_LANE();
      const uint32_t jobs = kScoreJobs[w];
      for (int slot = 0; slot < 4; ++slot) {
        const uint32_t job = (jobs >> (8 * slot)) & 0xFFu;
        if (job == 0xFFu) break;
        const bool is_a = job < 16;
        const int t = job & 15;
        unsigned char *PT = is_a ? AS : BS;
        // the tiles (rows s in block S, columns r in block R) that the
        // 32-column steps over r >= s read: S <= (R | 1); those with R < S
        // are zero
        const int R = tile_rt(t), S = tile_st(t);
        f32x4 acc = zero4();
        // acc[i] = X[r = 16R + 4lg + i][s = 16S + li]
        if (S <= R) {
          if (is_a) {
            const bool good = R != S || !((bad_mask >> R) & 1u);
            if (good) {
#pragma unroll
              for (int kk = 0; kk < DK / 32; ++kk) {
                const int dd = 32 * kk + 8 * lg;
                const bf16x8 kv = lds_frag<NCK>(KH, 16 * S + li, 4 * kk + lg);
                const float *ft = FT + pair_index(R, S) * DK + dd;
                const f32x4 f0 = *reinterpret_cast<const f32x4 *>(ft);
                const f32x4 f1 = *reinterpret_cast<const f32x4 *>(ft + 4);
                float y[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  y[e] = tof(kv[e]) * f0[e];
                  y[e + 4] = tof(kv[e + 4]) * f1[e];
                }
                acc = mfma(lds_frag<NCK>(QH, 16 * R + li, 4 * kk + lg), cvt8(y), acc);
              }
            } else {
              const int s = 16 * S + li;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int r = 16 * R + 4 * lg + i;
                float sum = 0.f;
                if (s <= r) {
                  for (int dd = 0; dd < DK; dd += 8) {
                    const bf16x8 qv = lds_frag<NCK>(QS, r, dd >> 3);
                    const bf16x8 kv = lds_frag<NCK>(KS, s, dd >> 3);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                      sum += tof(qv[e]) * tof(kv[e]) *
                             exp_c(CS[csx<DK>(r, dd + e)] - CS[csx<DK>(s, dd + e)]);
                  }
                }
                acc[i] = sum;
              }
            }
          } else {
#pragma unroll
            for (int kk = 0; kk < DV / 32; ++kk)
              acc = mfma(lds_frag<NCV>(DOS, 16 * R + li, 4 * kk + lg),
                         lds_frag<NCV>(VS, 16 * S + li, 4 * kk + lg), acc);
          }
        }
        bf16x4 pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * R + 4 * lg + i, s = 16 * S + li;
          pv[i] = tobf(s <= r && s < n && r < n ? acc[i] : 0.f);
        }
        *reinterpret_cast<bf16x4 *>(PT + swz_off<8>(16 * S + li, 2 * R + (lg >> 1)) + (lg & 1) * 8) =
            pv;
      }
    }
    lds_barrier();
    // KH -> KG = KH (.) FK[S] in place, the dv product's operand, and QL =
    // Qh (.) FQ[R] over the raw q tile, the state update's: every wave reads
    // them in full, so they are formed once here instead of by each wave.
    // The dk side re-forms the K-hat values it needs from k and the factor
    // it computes, and its exact path reads raw q from global memory.
    FRESH_LANE();
    scale_rows_by_block<DK, BTHR>(KH, KH, FK, tid);
    scale_rows_by_block<DK, BTHR>(QH, QS, FQ, tid);
    lds_barrier();

    if (do_dv) {
      // ---- dV^T[j][s] = (dO^T A^T)[j][s] + (G^T KG^T)[j][s] ----
      FRESH_LANE();
      bf16x8 gfrag[DK / 32][NJ];  // G^T A operands: row j, k = d (permuted)
#pragma unroll
      for (int kk = 0; kk < DK / 32; ++kk)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) gfrag[kk][jt] = cvt8(G0(2 * kk, jt), G0(2 * kk + 1, jt));
      for (int S = 0; S < 4; ++S) {
        const int s = 16 * S + li;
        bf16x8 kgf[DK / 32];  // KG^T B operands: k = d (same permutation), n = s
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
          const int da = 32 * kk + 4 * lg, db = da + 16;
          kgf[kk] = cat8(lds_half<NCK>(KH, s, da), lds_half<NCK>(KH, s, db));
        }
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < DK / 32; ++kk) acc = mfma(gfrag[kk][jt], kgf[kk], acc);
          for (int kb = S >> 1; kb < 2; ++kb)
            acc = mfma(tr_frag<NCV>(DOS, 32 * kb, j0 + 16 * jt, li, lg),
                       lds_frag<8>(AS, s, 4 * kb + lg), acc);
          // acc[i] = dV[s][j0 + 16 jt + 4 lg + i]
          if (s < n) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = tobf(acc[i]);
            *reinterpret_cast<bf16x4 *>(a.dv + (bh * T + t0 + s) * DV + j0 + 16 * jt + 4 * lg) =
                ov;
          }
        }
      }
    }
    if (do_dk) {
      // ---- dK^T[d][s], r2 = k dk, and the decay gradient ----
      FRESH_LANE();
      bf16x8 gfrag[DV / 32][NI];  // G A operands: row d, k = j (permuted)
#pragma unroll
      for (int kk = 0; kk < DV / 32; ++kk)
#pragma unroll
        for (int it = 0; it < NI; ++it) gfrag[kk][it] = cvt8(G1(2 * kk, it), G1(2 * kk + 1, it));
      // blocks last to first: the suffix sums of x = q.dq - k.dk over s run
      // through `carry` (later rows of this segment plus its boundary term)
      for (int S = 3; S >= 0; --S) {
        const int s = 16 * S + li;
        const bool good = !((bad_mask >> S) & 1u);
        bf16x8 vfr[DV / 32];  // V^T B operands: k = j (same permutation), n = s
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk)
          vfr[kk] = cat8(lds_half<NCV>(VS, s, 32 * kk + 4 * lg),
                         lds_half<NCV>(VS, s, 32 * kk + 16 + 4 * lg));
#pragma unroll
        for (int it = 0; it < NI; ++it) {
          const int dc = d0 + 16 * it + 4 * lg;  // this lane's 4 output d's
          // in-chunk part: sum over blocks R >= S of F_RS (Qh_R^T B_RS), one
          // 16-deep product per block, the factor applied after it
          f32x4 accI = zero4();
#pragma unroll
          for (int R = S; R < 4; ++R) {
            if (R == S && !good) continue;  // done elementwise below
            f32x4 P = zero4();
            P = mfma16(tr_read4<NCK>(QH, 16 * R + 4 * lg, d0 + 16 * it, li),  // Qh^T: row d, k = t
                       lds_half<8>(BS, s, 16 * R + 4 * lg), P);                // B^T: k = t, col s
            const f32x4 F = *reinterpret_cast<const f32x4 *>(FT + pair_index(R, S) * DK + dc);
#pragma unroll
            for (int i = 0; i < 4; ++i) accI[i] += F[i] * P[i];
          }
          f32x4 acc2 = zero4();
#pragma unroll
          for (int kk = 0; kk < DV / 32; ++kk) acc2 = mfma(gfrag[kk][it], vfr[kk], acc2);
          const bf16x4 kv = lds_half<NCK>(KS, s, dc);
          // this lane's 4 dimensions are one 16-byte piece of each row (dc is
          // a multiple of 4): read as such, not as 4 separate words
          const f32x4 csv = *reinterpret_cast<const f32x4 *>(CS + csx<DK>(s, dc));
          const f32x4 cev = *reinterpret_cast<const f32x4 *>(CS + csx<DK>(16 * S + 15, dc));
          const f32x4 fkv = *reinterpret_cast<const f32x4 *>(FK + S * DK + dc);
          float out[4], r2v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = dc + i;
            const float csd = csv[i];
            const float ue = exp_c(cev[i] - csd);
            // K-hat exactly as the scaled copy formed it (same factor, same
            // rounding), so the in-chunk paths still cancel against q.dq
            const float khd = tof(tobf(tof(kv[i]) * ue));
            const float inter = fkv[i] * acc2[i] * ue;
            float v = accI[i] * ue + inter;
            float rv = khd * accI[i] + tof(kv[i]) * inter;
            if (!good) {
              const float kd = tof(kv[i]);
              for (int r = s; r < min(16 * S + 16, n); ++r) {
                const float bsc = tof(*reinterpret_cast<const __bf16 *>(
                    BS + swz_off<8>(s, r >> 3) + (r & 7) * 2));
                // (raw q from global memory: its LDS tile holds QL by now)
                const float qd = tof(*reinterpret_cast<const __bf16 *>(qh + (t0 + r) * DK + d));
                v += (bsc * qd) * exp_c(CS[csx<DK>(r, d)] - csd);
                rv += path_term(bsc, qd, kd, CS[csx<DK>(r, d)], csd);
              }
            }
            out[i] = v;
            r2v[i] = rv;
          }
          const f32x4 r1 = r1b[S][it];
          // (the decay gradient first: its q.dq loads are then waited for
          // before this block's stores are issued, not after them)
          f32x4 dl4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // inclusive suffix sum over the 16 rows li of block S
            float x = s < n ? r1[i] - r2v[i] : 0.f;
            x += row_dpp<0x101>(x);  // row_shl:1
            x += row_dpp<0x102>(x);  // row_shl:2
            x += row_dpp<0x104>(x);  // row_shl:4
            x += row_dpp<0x108>(x);  // row_shl:8
            const float tot = row_dpp<0x150>(x);  // row_newbcast:0 -- the block's total
            dl4[i] = x + carry[it][i];
            carry[it][i] += tot;
          }
          if (s < n) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = tobf(out[i]);
            *reinterpret_cast<bf16x4 *>(a.dk + (bh * T + t0 + s) * DK + dc) = ov;
            *reinterpret_cast<f32x4 *>(a.dl + (bh * T + t0 + s) * DK + dc) = dl4;
          }
        }
      }
    }

    // ---- G <- diag(alpha) G + QL^T dO (both copies) ----
    // the next chunk's k, v and logs start streaming in (every read of them
    // in this chunk is done)
    lds_barrier();
    FRESH_LANE();
    if (ci > c_begin) stage_kvl(ci - 1);
    {
      FRESH_LANE();
      if (do_dv) {
#pragma unroll
        for (int dt = 0; dt < DK / 16; ++dt) {
          const f32x4 av = *reinterpret_cast<const f32x4 *>(AL + 16 * dt + 4 * lg);
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) G0(dt, jt)[i] *= av[i];
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 db[NJ];  // dO B operands: k = r, column j
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) db[jt] = tr_frag<NCV>(DOS, 32 * kb, j0 + 16 * jt, li, lg);
#pragma unroll
          for (int dt = 0; dt < DK / 16; ++dt) {
            const bf16x8 qa = tr_frag<NCK>(QS, 32 * kb, 16 * dt, li, lg);  // QL^T: row d, k = r
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) G0(dt, jt) = mfma(qa, db[jt], G0(dt, jt));
          }
        }
      }
      if (do_dk) {
#pragma unroll
        for (int it = 0; it < NI; ++it) {
          const float al = AL[d0 + 16 * it + li];
#pragma unroll
          for (int jt = 0; jt < DV / 16; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) G1(jt, it)[i] *= al;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 qb[NI];  // QL B operands: k = r, column d
#pragma unroll
          for (int it = 0; it < NI; ++it) qb[it] = tr_frag<NCK>(QS, 32 * kb, d0 + 16 * it, li, lg);
#pragma unroll
          for (int jt = 0; jt < DV / 16; ++jt) {
            const bf16x8 da = tr_frag<NCV>(DOS, 32 * kb, 16 * jt, li, lg);  // dO^T: row j, k = r
#pragma unroll
            for (int it = 0; it < NI; ++it) G1(jt, it) = mfma(da, qb[it], G1(jt, it));
          }
        }
      }
    }
  }

  FRESH_LANE();
  if (a.dS0 && do_dv && seg == 0) {
    float *dst = a.dS0 + bh * DK * DV;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(16 * dt + 4 * lg + i) * DV + j0 + 16 * jt + li] = G0(dt, jt)[i];
  }
}
#undef G0
#undef G1
#undef FRESH_LANE

// The adjoint state at each segment's end, right to left (the backward's
// mirror of the forward's scan): G_end(P-1) = dS_T and
// G_end(p - 1) = diag(A(p)) G_end(p) + G_loc(p), one thread per entry,
// written over G_loc(p) once read.
__global__ __launch_bounds__(256) void gla_grad_scan_kernel(const float *dST, float *Gloc,
                                                            const float *Aq, int64_t nh,
                                                            int64_t DK, int64_t DV, int64_t P) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= nh * DK * DV) return;
  const int64_t bh = e / (DK * DV), d = (e / DV) % DK;
  float g = dST ? dST[e] : 0.f;
  for (int64_t p = P - 1; p >= 1; --p) {
    float *slot = Gloc + p * nh * DK * DV + e;
    g = Aq[(p * nh + bh) * DK + d] * g + *slot;
    *slot = g;
  }
}

template <int DK, int DV>
hipError_t gla_bwd_impl(const GlaBwdArgs &args, hipStream_t stream) {
  const dim3 grid((unsigned)args.nh, (unsigned)args.P);
  CLA_LAUNCH("gla_dq", (gla_dq_kernel<DK, DV>), grid, dim3(dq_threads<DK>()), stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (args.P > 1) {
    const int64_t n = args.nh * DK * DV;
    CLA_LAUNCH("gla_grad_scan", gla_grad_scan_kernel, dim3((unsigned)((n + 255) / 256)),
               dim3(256), stream, args.dST, args.Gloc, args.Aq, args.nh, (int64_t)DK, (int64_t)DV,
               args.P);
  }
  CLA_LAUNCH("gla_dkdv", (gla_dkdv_kernel<DK, DV>), grid, dim3(BTHR), stream, args);
  return hipGetLastError();
}

}  // namespace

size_t gla_bwd_ws_bytes(int64_t nh, int64_t T, int64_t DK, int64_t DV) {
  auto r256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t nchunks = (T + TC - 1) / TC;
  const int64_t nblk = (nchunks + kSegChunks - 1) / kSegChunks;
  size_t b = r256((size_t)nh * T * DK * sizeof(float)) +
             r256((size_t)nblk * nh * DK * DV * sizeof(float));
  const GlaPlan p = plan_gla(nh, T);
  if (p.P > 1)
    b += gla_fwd_ws_bytes(nh, T, DK, DV) + r256((size_t)(p.P * nh * DK * DV) * sizeof(float)) +
         r256((size_t)(p.P * nh * DK) * sizeof(float));
  return b;
}

hipError_t gla_bwd_dispatch(const GlaBwdArgs &args, int DK, int DV, hipStream_t stream) {
  if (DK == 64 && DV == 64) return gla_bwd_impl<64, 64>(args, stream);
  if (DK == 64 && DV == 128) return gla_bwd_impl<64, 128>(args, stream);
  if (DK == 128 && DV == 64) return gla_bwd_impl<128, 64>(args, stream);
  if (DK == 128 && DV == 128) return gla_bwd_impl<128, 128>(args, stream);
  return hipErrorInvalidValue;
}

}  // namespace gla
}  // namespace cla
