// Selective scan with N state entries per channel (Mamba-1's recurrence),
// forward and backward, for gfx950.
//
// Citations (page title, then section):
//   ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
//
//   h_t[d, n] = exp(delta_t[d] A[d, n]) h_{t-1}[d, n] + delta_t[d] B_t[n] x_t[d]
//   y_t[d]    = sum_n C_t[n] h_t[d, n]
//
// One diagonal recurrence per (channel, entry) (ZTF "Scans over vector and
// matrix states"), with the decay and the input formed from the per-token
// step size inside the kernel and the state contracted with C there, so that
// no [B, T, D, N] tensor reaches HBM (ZTF "What limits a recurrent layer", on
// Mamba's fused kernel).  B*D*N recurrences are independent; each lane runs
// N/4 of them in time order -- the same section's count: with that many
// independent recurrences the GPU is full without a scan over time.
//
// Layout: x, delta, y, dy, dx, ddelta [B, T, D]; A [D, N]; B, C [B, T, N];
// h0, hT, dhT, dh0 [B, D, N]; checkpoints [B, ceil(T/16), D, N]; all fp32.
// A workgroup is 4 waves = 64 channels of one sequence; lane 4c + q of a wave
// (c = its channel among the wave's 16) holds entries q NPT .. q NPT + NPT - 1,
// so y's sum over entries is two quad DPP adds.  Time runs in tiles of 32
// steps, each staged HBM -> LDS by DMA (x, delta, dy rows of 64 channels, B
// and C rows of N entries).
//
// Backward (ZTF "The backward pass is a scan in reverse", per entry): the
// forward writes the state before every 16th step; the backward walks
// 16-step tiles last to first, recomputes a tile's 16 states into registers
// from its checkpoint (Mamba recomputes its states rather than storing them, the same
// section says), then runs hbar_t = C_t dy_t + a_{t+1} hbar_{t+1} in reverse
// with the chain rule through exp(delta A) and delta B x.  The sums over
// channels that dB and dC need are taken over each 16-lane row's 4 channels
// with DPP, then through LDS in blocks of 8 steps to one partial per
// workgroup; a small last kernel adds the partials, and dA over
// the batch, in a fixed order, so every result is deterministic.
#include "chunk_common.h"
#include "internal.h"
#include "sscan_kernels.h"

namespace cla {
namespace sscan {
namespace {

using chunk::lds_barrier;
using chunk::lds_void;

constexpr int NTH = 256;
constexpr int TT = kTile;
constexpr int CH = kChannels;
constexpr float kLog2e = 1.4426950408889634f;

// decay exp(delta A) as 2^(delta * A log2 e): one v_exp_f32
__device__ __forceinline__ float decay(float dv, float A2) {
  return __builtin_amdgcn_exp2f(dv * A2);
}

// sum over the 4 lanes of a quad (all four get the same value)
__device__ __forceinline__ float quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1,
                                                             0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E,
                                                             0xF, 0xF, true));
  return v;
}

// sum over the 4 lanes of a 16-lane row that are 4 apart (lane 4c + q: the
// row's 4 channels at one q); every lane gets the sum of its residue class
__device__ __forceinline__ float row_channel_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124,
                                                             0xF, 0xF, true));  // row_ror:4
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128,
                                                             0xF, 0xF, true));  // row_ror:8
  return v;
}

// Stage ROWS rows of a fp32 array (row r at src + r * ld; rows past nrows
// re-read row nrows - 1; 16-byte pieces past column maxcol4 re-read that
// piece) into a row-major [ROWS][W] LDS tile, W a multiple of 4.  Lane i of a
// wave's DMA writes bytes 16 i .. 16 i + 15 of the wave's 1 KB destination.
template <int ROWS, int W>
__device__ __forceinline__ void dma_rows(const float *src, int64_t ld, int nrows, int col0,
                                         int maxcol4, float *tile, int tid) {
  constexpr int PPR = W / 4;
  constexpr int NP = ROWS * PPR;
  const int lane = tid & 63, w = tid >> 6;
  for (int base = w * 64; base < NP; base += NTH) {
    const int p = base + lane;
    if (p < NP) {
      const int r = min(p / PPR, nrows - 1);
      const int k = min(col0 + 4 * (p % PPR), maxcol4);
      __builtin_amdgcn_global_load_lds(src + (int64_t)r * ld + k, (lds_void *)(tile + 4 * base),
                                       16, 0, 0);
    }
  }
}

// Store rows r < nt, channels d0 + k < D of a [ROWS][CH] LDS tile (16 bytes a lane).
template <int ROWS>
__device__ __forceinline__ void store_rows(float *dst, int64_t ld, int nt, int d0, int64_t D,
                                           const float *tile, int tid) {
  for (int p = tid; p < ROWS * CH / 4; p += NTH) {
    const int r = p / (CH / 4), k = 4 * (p % (CH / 4));
    if (r < nt && d0 + k < D)
      *reinterpret_cast<float4 *>(dst + (int64_t)r * ld + d0 + k) =
          *reinterpret_cast<const float4 *>(tile + r * CH + k);
  }
}

// AGG = false: the forward over time segment blockIdx.z (from h0 or the
// scanned state of the segments before it).  AGG = true: segment blockIdx.z
// of the first P - 1 from a zero state, writing its local state and its
// product of decays for the scan across segments.
// The channel group of this workgroup.  Workgroups are dispatched to the 8
// XCDs round-robin by linear id (x fastest); with a multiple of 8 groups this
// gives each XCD a contiguous range of channel groups, so that the rows an
// XCD streams at a time step are one contiguous span (results are the same
// for any order).
__device__ __forceinline__ int xcd_group() {
  const unsigned G = gridDim.x;
  return G % 8 == 0 ? (int)((blockIdx.x % 8) * (G / 8) + blockIdx.x / 8) : (int)blockIdx.x;
}

template <int NPT, bool AGG>
__global__ __launch_bounds__(NTH) void sscan_fwd_kernel(FwdArgs a) {
  constexpr int N = 4 * NPT;
  __shared__ __attribute__((aligned(16))) float XS[TT * CH];
  __shared__ __attribute__((aligned(16))) float DS[TT * CH];
  __shared__ __attribute__((aligned(16))) float YS[TT * CH];
  __shared__ __attribute__((aligned(16))) float BS[TT * N];
  __shared__ __attribute__((aligned(16))) float CS[TT * N];
  const int tid = threadIdx.x;
  const int c = tid >> 2, q = tid & 3;
  const int64_t b = blockIdx.y, seg = blockIdx.z;
  const int64_t T = a.T, D = a.D;
  const int gx = xcd_group();
  const int d0 = gx * CH;
  const int d = d0 + c;
  const bool valid = d < D;
  const int dc = min(d, (int)D - 1);
  const int e0 = q * NPT;  // this lane's first entry
  const int64_t bdn = a.B * D * N;
  // the state this segment starts from
  const float *hsrc = AGG ? nullptr
                          : seg == 0 ? (a.h0 ? a.h0 + (b * D + dc) * N + e0 : nullptr)
                                     : a.Hloc + (seg - 1) * bdn + (b * D + dc) * N + e0;
  float A2[NPT], h[NPT], ap[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    A2[j] = a.A[(int64_t)dc * N + e0 + j] * kLog2e;
    h[j] = hsrc ? hsrc[j] : 0.f;
    ap[j] = 1.f;
  }
  const int64_t ntiles = num_tiles(T), nck = num_ckpts(T);
  const int64_t s_begin = seg * a.seg_tiles, s_end = min(ntiles, s_begin + a.seg_tiles);
  const bool save = !AGG && a.ckpt && valid;
  for (int64_t s = s_begin; s < s_end; ++s) {
    const int64_t t0 = s * TT;
    const int nt = (int)min<int64_t>(TT, T - t0);
    dma_rows<TT, CH>(a.x + (b * T + t0) * D, D, nt, d0, (int)D - 4, XS, tid);
    dma_rows<TT, CH>(a.delta + (b * T + t0) * D, D, nt, d0, (int)D - 4, DS, tid);
    dma_rows<TT, N>(a.Bm + (b * T + t0) * N, N, nt, 0, N - 4, BS, tid);
    if (!AGG) dma_rows<TT, N>(a.Cm + (b * T + t0) * N, N, nt, 0, N - 4, CS, tid);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (AGG) {
      for (int t = 0; t < nt; ++t) {
        const float dv = DS[t * CH + c];
        const float dx = dv * XS[t * CH + c];
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
          const float av = decay(dv, A2[j]);
          h[j] = fmaf(av, h[j], dx * BS[t * N + e0 + j]);
          ap[j] *= av;
        }
      }
      lds_barrier();
      continue;
    }
    for (int th = 0; th < nt; th += kCkpt) {
      if (save) {
        // the state before step t0 + th, for the backward
        float *dst = a.ckpt + ((b * nck + (t0 + th) / kCkpt) * D + d) * N + e0;
#pragma unroll
        for (int j = 0; j < NPT; ++j) dst[j] = h[j];
      }
      const int te = min(th + kCkpt, nt);
      for (int t = th; t < te; ++t) {
        const float xv = XS[t * CH + c], dv = DS[t * CH + c];
        const float dx = dv * xv;
        float yp = 0.f;
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
          h[j] = fmaf(decay(dv, A2[j]), h[j], dx * BS[t * N + e0 + j]);
          yp = fmaf(CS[t * N + e0 + j], h[j], yp);
        }
        const float yv = quad_sum(yp);
        if (q == 0) YS[t * CH + c] = yv;
      }
    }
    lds_barrier();
    if (a.y) store_rows<TT>(a.y + (b * T + t0) * D, D, nt, d0, D, YS, tid);
  }
  if (AGG) {
    if (valid) {
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        a.Hloc[seg * bdn + (b * D + d) * N + e0 + j] = h[j];
        a.Aprod[seg * bdn + (b * D + d) * N + e0 + j] = ap[j];
      }
    }
  } else if (a.hT && valid && seg == a.P - 1) {
#pragma unroll
    for (int j = 0; j < NPT; ++j) a.hT[(b * D + d) * N + e0 + j] = h[j];
  }
}

// The state each time segment starts from (ZTF "Splitting one sequence
// across devices", per (channel, entry)): H_in(0) = h0,
// H_in(p) = Aprod(p-1) H_in(p-1) + Hloc(p-1), written over Hloc(p-1).
__global__ __launch_bounds__(256) void sscan_fwd_scan_kernel(FwdArgs a) {
  const int64_t bdn = a.B * a.D * a.N;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= bdn) return;
  float h = a.h0 ? a.h0[e] : 0.f;
  for (int64_t p = 1; p < a.P; ++p) {
    const int64_t slot = (p - 1) * bdn + e;
    h = a.Aprod[slot] * h + a.Hloc[slot];
    a.Hloc[slot] = h;
  }
}

// The adjoint each time segment starts from on its right, from its end back
// over the later segments: X(P-1) = dhT, X(q-1) = Aprod(q) X(q) + Gloc(q),
// written over Gloc(q).
__global__ __launch_bounds__(256) void sscan_bwd_scan_kernel(BwdArgs a) {
  const int64_t bdn = a.B * a.D * a.N;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= bdn) return;
  float x = a.dhT ? a.dhT[e] : 0.f;
  for (int64_t p = a.P - 1; p >= 1; --p) {
    const int64_t slot = p * bdn + e;
    x = a.Aprod[slot] * x + a.Gloc[slot];
    a.Gloc[slot] = x;
  }
}

// Time segment q = 1 + blockIdx.z, last step to first, from a zero adjoint:
// the segment's own contribution to the adjoint at its first step, times that
// step's decay (what it hands to the segment before it), and its product of
// decays.  Only the decays, C and dy are needed, not the states.
template <int NPT>
__global__ __launch_bounds__(NTH) void sscan_bwd_agg_kernel(BwdArgs a) {
  constexpr int N = 4 * NPT;
  __shared__ __attribute__((aligned(16))) float DS[TT * CH];
  __shared__ __attribute__((aligned(16))) float GS[TT * CH];
  __shared__ __attribute__((aligned(16))) float CS[TT * N];
  const int tid = threadIdx.x;
  const int c = tid >> 2, q = tid & 3;
  const int64_t b = blockIdx.y, seg = 1 + blockIdx.z;
  const int64_t T = a.T, D = a.D;
  const int gx = xcd_group();
  const int d0 = gx * CH;
  const int d = d0 + c;
  const int dc = min(d, (int)D - 1);
  const int e0 = q * NPT;
  const int64_t bdn = a.B * D * N;
  float A2[NPT], hb[NPT], an[NPT], ap[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    A2[j] = a.A[(int64_t)dc * N + e0 + j] * kLog2e;
    hb[j] = 0.f;
    an[j] = 1.f;
    ap[j] = 1.f;
  }
  const int64_t ntiles = num_tiles(T);
  const int64_t s_begin = seg * a.seg_tiles, s_end = min(ntiles, s_begin + a.seg_tiles);
  for (int64_t s = s_end - 1; s >= s_begin; --s) {
    const int64_t t0 = s * TT;
    const int nt = (int)min<int64_t>(TT, T - t0);
    dma_rows<TT, CH>(a.delta + (b * T + t0) * D, D, nt, d0, (int)D - 4, DS, tid);
    dma_rows<TT, CH>(a.dy + (b * T + t0) * D, D, nt, d0, (int)D - 4, GS, tid);
    dma_rows<TT, N>(a.Cm + (b * T + t0) * N, N, nt, 0, N - 4, CS, tid);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    for (int t = nt - 1; t >= 0; --t) {
      const float dv = DS[t * CH + c], gv = GS[t * CH + c];
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        const float av = decay(dv, A2[j]);
        hb[j] = fmaf(hb[j], an[j], CS[t * N + e0 + j] * gv);
        an[j] = av;
        ap[j] *= av;
      }
    }
    lds_barrier();
  }
  if (d < D) {
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      a.Gloc[seg * bdn + (b * D + d) * N + e0 + j] = an[j] * hb[j];
      a.Aprod[seg * bdn + (b * D + d) * N + e0 + j] = ap[j];
    }
  }
}

template <int NPT>
__global__ __launch_bounds__(NTH, 3) void sscan_bwd_kernel(BwdArgs a) {
  constexpr int N = 4 * NPT;
  constexpr int TB = kCkpt;   // steps per tile: one checkpoint each
  constexpr int RS = 8;       // steps per block of the channel sums
  constexpr int NG = CH / 4;  // channel groups: the 4 channels of a 16-lane row
  constexpr int PC = NG + 4;  // padded row of the channel-sum area (no bank conflicts)
  __shared__ __attribute__((aligned(16))) float XS[TB * CH];
  __shared__ __attribute__((aligned(16))) float DS[TB * CH];
  __shared__ __attribute__((aligned(16))) float GS[TB * CH];  // dy
  __shared__ __attribute__((aligned(16))) float OX[TB * CH];  // dx out
  __shared__ __attribute__((aligned(16))) float OD[TB * CH];  // ddelta out
  __shared__ __attribute__((aligned(16))) float BS[TB * N];
  __shared__ __attribute__((aligned(16))) float CS[TB * N];
  __shared__ __attribute__((aligned(16))) float PR[RS * 2 * N * PC];
  const int tid = threadIdx.x;
  const int c = tid >> 2, q = tid & 3;
  const int64_t b = blockIdx.y, seg = blockIdx.z;
  const int64_t T = a.T, D = a.D;
  const int64_t G = num_groups(D);
  const int gx = xcd_group();
  const int d0 = gx * CH;
  const int d = d0 + c;
  const bool valid = d < D;
  const int dc = min(d, (int)D - 1);
  const int e0 = q * NPT;
  float Av[NPT], A2[NPT], hbar[NPT], an[NPT], dAacc[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    Av[j] = a.A[(int64_t)dc * N + e0 + j];
    A2[j] = Av[j] * kLog2e;
    // the adjoint from the steps after this segment: dhT, or the scan's
    const float *gsrc = seg == a.P - 1 ? (a.dhT ? a.dhT + (b * D + dc) * N : nullptr)
                                       : a.Gloc + (seg + 1) * a.B * D * N + (b * D + dc) * N;
    hbar[j] = gsrc ? gsrc[e0 + j] : 0.f;
    an[j] = 1.f;  // a_{t+1}; none after the last step
    dAacc[j] = 0.f;
  }
  const int64_t nck = num_ckpts(T);
  // this segment's 16-step tiles (its 32-step tiles, two each)
  const int64_t s_begin = seg * a.seg_tiles * (TT / TB);
  const int64_t s_end = min(nck, s_begin + a.seg_tiles * (TT / TB));
  for (int64_t s = s_end - 1; s >= s_begin; --s) {
    const int64_t t0 = s * TB;
    const int nt = (int)min<int64_t>(TB, T - t0);
    float hs[TB][NPT];  // hs[t] = the state before step t of the tile
    float he[NPT];
    {
      const float *src = a.ckpt + ((b * nck + s) * D + dc) * N + e0;
#pragma unroll
      for (int j = 0; j < NPT; ++j) he[j] = src[j];
    }
    dma_rows<TB, CH>(a.x + (b * T + t0) * D, D, nt, d0, (int)D - 4, XS, tid);
    dma_rows<TB, CH>(a.delta + (b * T + t0) * D, D, nt, d0, (int)D - 4, DS, tid);
    dma_rows<TB, CH>(a.dy + (b * T + t0) * D, D, nt, d0, (int)D - 4, GS, tid);
    dma_rows<TB, N>(a.Bm + (b * T + t0) * N, N, nt, 0, N - 4, BS, tid);
    dma_rows<TB, N>(a.Cm + (b * T + t0) * N, N, nt, 0, N - 4, CS, tid);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    // the tile's states, recomputed from its checkpoint
#pragma unroll
    for (int t = 0; t < TB; ++t) {
#pragma unroll
      for (int j = 0; j < NPT; ++j) hs[t][j] = he[j];
      if (t < nt) {
        const float dv = DS[t * CH + c];
        const float dx = dv * XS[t * CH + c];
#pragma unroll
        for (int j = 0; j < NPT; ++j)
          he[j] = fmaf(decay(dv, A2[j]), he[j], dx * BS[t * N + e0 + j]);
      }
    }
    // he = the state after the tile's last step
#pragma unroll
    for (int t = TB - 1; t >= 0; --t) {
      const int tl = t & (RS - 1);
      float pb[NPT], pc[NPT];
#pragma unroll
      for (int j = 0; j < NPT; ++j) pb[j] = pc[j] = 0.f;
      if (t < nt) {
        const float xv = XS[t * CH + c], dv = DS[t * CH + c], gv = GS[t * CH + c];
        const float dx = dv * xv;
        float sbp = 0.f, ddp = 0.f;
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
          const float av = decay(dv, A2[j]);
          hbar[j] = fmaf(hbar[j], an[j], CS[t * N + e0 + j] * gv);
          const float ht = t + 1 < nt ? hs[t + 1 < TB ? t + 1 : TB - 1][j] : he[j];
          const float daa = hbar[j] * hs[t][j] * av;  // dL/da_t times a_t
          ddp = fmaf(daa, Av[j], ddp);
          dAacc[j] = fmaf(daa, dv, dAacc[j]);
          sbp = fmaf(hbar[j], BS[t * N + e0 + j], sbp);
          pb[j] = valid ? hbar[j] * dx : 0.f;
          pc[j] = valid ? gv * ht : 0.f;
          an[j] = av;
        }
        const float sb = quad_sum(sbp), dd = quad_sum(ddp);
        if (q == 0) {
          OX[t * CH + c] = dv * sb;
          OD[t * CH + c] = fmaf(sb, xv, dd);
        }
      }
      // dB, dC terms summed over the row's 4 channels in registers; the
      // row's first quad stores them for the workgroup's sum below
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        pb[j] = row_channel_sum(pb[j]);
        pc[j] = row_channel_sum(pc[j]);
      }
      if ((tid & 12) == 0) {
        const int gi = (tid >> 4);  // the row: 4 channels
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
          PR[(tl * 2 * N + e0 + j) * PC + gi] = pb[j];
          PR[(tl * 2 * N + N + e0 + j) * PC + gi] = pc[j];
        }
      }
      if (tl == 0) {
        // sums over the workgroup's 16 rows: one thread per (step, entry row)
        lds_barrier();
        for (int o = tid; o < RS * 2 * N; o += NTH) {
          const int tt = o / (2 * N), row = o % (2 * N);
          if (t + tt < nt) {
            const float *pr = PR + (tt * 2 * N + row) * PC;
            const float4 v0 = *reinterpret_cast<const float4 *>(pr);
            const float4 v1 = *reinterpret_cast<const float4 *>(pr + 4);
            const float4 v2 = *reinterpret_cast<const float4 *>(pr + 8);
            const float4 v3 = *reinterpret_cast<const float4 *>(pr + 12);
            const float sum = (((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w))) +
                              (((v2.x + v2.y) + (v2.z + v2.w)) + ((v3.x + v3.y) + (v3.z + v3.w)));
            a.part[((b * G + gx) * T + t0 + t + tt) * 2 * N + row] = sum;
          }
        }
        lds_barrier();
      }
    }
    store_rows<TB>(a.dx + (b * T + t0) * D, D, nt, d0, D, OX, tid);
    store_rows<TB>(a.ddelta + (b * T + t0) * D, D, nt, d0, D, OD, tid);
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      a.dAp[seg * a.B * D * N + (b * D + d) * N + e0 + j] = dAacc[j];
      if (a.dh0 && seg == 0) a.dh0[(b * D + d) * N + e0 + j] = an[j] * hbar[j];
    }
  }
}

// dB, dC: the per-workgroup partials summed over workgroups in order; dA: the
// per-sequence sums added over the batch in order.
__global__ __launch_bounds__(256) void sscan_reduce_kernel(BwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t N = a.N, T = a.T, D = a.D, B = a.B, G = num_groups(D);
  const int64_t nbt = B * T * N;
  if (i < nbt) {
    const int64_t b = i / (T * N), r = i % (T * N);
    const int64_t t = r / N, n = r % N;
    float sb = 0.f, sc = 0.f;
    for (int64_t g = 0; g < G; ++g) {
      const float *p = a.part + ((b * G + g) * T + t) * 2 * N;
      sb += p[n];
      sc += p[N + n];
    }
    a.dB[i] = sb;
    a.dC[i] = sc;
  } else if (i < nbt + D * N) {
    const int64_t k = i - nbt;
    float s = 0.f;
    for (int64_t pb = 0; pb < a.P * B; ++pb) s += a.dAp[pb * D * N + k];
    a.dA[k] = s;
  }
}

template <int NPT>
hipError_t fwd_impl(const FwdArgs &a, hipStream_t stream) {
  const unsigned G = (unsigned)num_groups(a.D), Bu = (unsigned)a.B;
  if (a.P > 1) {
    CLA_LAUNCH("sscan_fwd_segments", (sscan_fwd_kernel<NPT, true>), dim3(G, Bu, (unsigned)(a.P - 1)),
               dim3(NTH), stream, a);
    const int64_t n = a.B * a.D * a.N;
    CLA_LAUNCH("sscan_segment_scan", sscan_fwd_scan_kernel, dim3((unsigned)((n + 255) / 256)),
               dim3(256), stream, a);
  }
  CLA_LAUNCH("sscan_fwd", (sscan_fwd_kernel<NPT, false>), dim3(G, Bu, (unsigned)a.P), dim3(NTH),
             stream, a);
  return hipGetLastError();
}

template <int NPT>
hipError_t bwd_impl(const BwdArgs &a, hipStream_t stream) {
  const unsigned G = (unsigned)num_groups(a.D), Bu = (unsigned)a.B;
  if (a.P > 1) {
    CLA_LAUNCH("sscan_bwd_segments", sscan_bwd_agg_kernel<NPT>, dim3(G, Bu, (unsigned)(a.P - 1)),
               dim3(NTH), stream, a);
    const int64_t n = a.B * a.D * a.N;
    CLA_LAUNCH("sscan_grad_scan", sscan_bwd_scan_kernel, dim3((unsigned)((n + 255) / 256)),
               dim3(256), stream, a);
  }
  const dim3 grid(G, Bu, (unsigned)a.P);
  CLA_LAUNCH("sscan_bwd", sscan_bwd_kernel<NPT>, grid, dim3(NTH), stream, a);
  const int64_t n = a.B * a.T * a.N + a.D * a.N;
  CLA_LAUNCH("sscan_reduce", sscan_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256),
             stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t fwd_dispatch(const FwdArgs &a, hipStream_t stream) {
  switch (a.N) {
    case 4: return fwd_impl<1>(a, stream);
    case 8: return fwd_impl<2>(a, stream);
    case 16: return fwd_impl<4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t bwd_dispatch(const BwdArgs &a, hipStream_t stream) {
  switch (a.N) {
    case 4: return bwd_impl<1>(a, stream);
    case 8: return bwd_impl<2>(a, stream);
    case 16: return bwd_impl<4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sscan
}  // namespace cla
