// Diagonal (per-channel) linear-recurrence scan, forward and backward, for
// gfx950.
//
// Citations (page title, then section):
//   ZTF  = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
//   WIKI = "Parallel Scan" (aiwiki.thehackersbrain.dev)
//
// The recurrence h_t = a_t h_{t-1} + b_t is a scan of affine pairs under
// (a1, b1) . (a2, b2) = (a1 a2, a2 b1 + b2), the earlier step on the left
// (ZTF "The scan for one number of state").  The backward is the same scan
// run in reverse time over the pairs (a_{t+1}, dh_t) (ZTF "The backward pass
// is a scan in reverse").  Both directions share one kernel template.
//
// Layout: [B, T, D] fp32, channels contiguous.  A workgroup owns 16 * VEC
// channels of one batch row and sweeps its time range in blocks of
// 4 * NW * K steps (NW waves, K steps per lane):
//   lane  = 16 channel lanes (VEC channels each, float4 when VEC = 4)
//         x 4 time slots;   wave w holds slots 4w .. 4w+3;
//   slot j of a block owns the kK consecutive steps j*kK .. j*kK + kK - 1.
// Per block: coalesced loads (each wave instruction covers 4 rows of 64
// channels) -> a serial compose of kK steps in registers -> a Hillis-Steele
// scan over the 4 slots of a wave with lane shuffles (WIKI code listing; ZTF
// "The scan for one number of state") -> wave aggregates through LDS, folded
// onto the pair carried from the previous block (one composed pair goes from
// tile to tile and no intermediate state goes to HBM: WIKI, the closing
// section on tiled, IO-aware kernels) -> each lane recomputes its kK states
// from its incoming state and stores them.
//
// When B * D alone gives too few workgroups, the time axis is cut into P
// segments: a first pass (AGG) writes each segment's composed pair, and the
// main pass starts each segment from the fold of the earlier segments' pairs
// (ZTF "Splitting one sequence across devices", done across workgroups).
#include <mutex>

#include "internal.h"

namespace cla {
namespace {

// Tile shapes (compile-time; overridable for tuning builds).  Measured on
// MI355X at B=8, T=16384, D=4096: the forward is fastest with 4 waves x 2
// steps per lane, the backward (3 reads, 2 writes per element) with 2 waves
// x 2 steps per lane.
#ifndef CLA_SCAN_FWD_NW
#define CLA_SCAN_FWD_NW 4
#endif
#ifndef CLA_SCAN_FWD_K
#define CLA_SCAN_FWD_K 2
#endif
#ifndef CLA_SCAN_BWD_NW
#define CLA_SCAN_BWD_NW 2
#endif
#ifndef CLA_SCAN_BWD_K
#define CLA_SCAN_BWD_K 2
#endif
#ifndef CLA_SCAN_PREFETCH
#define CLA_SCAN_PREFETCH 1
#endif
#ifndef CLA_SCAN_NT
#define CLA_SCAN_NT 1
#endif
#ifndef CLA_SCAN_NT_LD
#define CLA_SCAN_NT_LD CLA_SCAN_NT
#endif
#ifndef CLA_SCAN_NT_ST
#define CLA_SCAN_NT_ST CLA_SCAN_NT
#endif
#ifndef CLA_SCAN_TARGET_GROUPS
#define CLA_SCAN_TARGET_GROUPS 512
#endif
// Segment lengths are multiples of kPlanBlock, a multiple of both block
// lengths 4 * NW * K.
constexpr int kPlanBlock = 128;
static_assert(kPlanBlock % (4 * CLA_SCAN_FWD_NW * CLA_SCAN_FWD_K) == 0, "block");
static_assert(kPlanBlock % (4 * CLA_SCAN_BWD_NW * CLA_SCAN_BWD_K) == 0, "block");
constexpr int64_t kTargetGroups = CLA_SCAN_TARGET_GROUPS;  // to fill 256 CUs

template <int VEC>
struct Pair {
  float A[VEC];
  float S[VEC];
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming loads/stores: every element is touched once, so they are marked
// non-temporal to keep them from displacing reusable lines in the caches.
template <int VEC>
__device__ __forceinline__ void ldv(const float *p, float (&x)[VEC]) {
  if constexpr (VEC == 4) {
#if CLA_SCAN_NT_LD
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
#else
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#endif
    x[0] = v.x;
    x[1] = v.y;
    x[2] = v.z;
    x[3] = v.w;
  } else {
#if CLA_SCAN_NT_LD
    x[0] = __builtin_nontemporal_load(p);
#else
    x[0] = *p;
#endif
  }
}

template <int VEC>
__device__ __forceinline__ void stv(float *p, const float (&x)[VEC]) {
  if constexpr (VEC == 4) {
    const f32x4 v = {x[0], x[1], x[2], x[3]};
#if CLA_SCAN_NT_ST
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
#else
    *reinterpret_cast<f32x4 *>(p) = v;
#endif
  } else {
#if CLA_SCAN_NT_ST
    __builtin_nontemporal_store(x[0], p);
#else
    *p = x[0];
#endif
  }
}

template <int VEC>
__device__ __forceinline__ void fillv(float (&x)[VEC], float v) {
#pragma unroll
  for (int e = 0; e < VEC; ++e) x[e] = v;
}

struct ScanArgs {
  const float *a;      // [B, T, D] decays
  const float *x;      // forward: b; backward: dh
  const float *hprev;  // backward: forward output h (h_{t-1}); forward: unused
  const float *init;   // forward: h0; backward: dhT (NULL = zeros)
  const float *h0;     // backward: forward h0 for da at t = 0 (NULL = zeros)
  float *y;            // forward: h; backward: db
  float *y2;           // backward: da
  float *fin;          // forward: hT; backward: dh0 (NULL = skip)
  float2 *agg;         // [P - 1][B * D] composed pair of each segment
  int64_t B, T, D;
  int64_t seg_len;
  int64_t P;
  int64_t groups_per_batch;
};

// DIR = 0: scan position u is time t = u, pair (a_t, b_t), state h.
// DIR = 1: scan position u is time t = T - 1 - u, pair (a_{t+1}, dh_t) with
//          a_{T+1} = 1, state hbar; outputs db_t = hbar_t, da_t = hbar_t h_{t-1}.
// AGG    : only compose each segment's pair (segments 0 .. P-2) into agg.
// kNW waves per workgroup, kK steps per lane per block.
template <int VEC, int DIR, bool AGG, int kNW, int kK>
__global__ __launch_bounds__(kNW * 64) void scan_kernel(ScanArgs p) {
  constexpr int CG = 16 * VEC;
  constexpr int kBlock = 4 * kNW * kK;
  __shared__ Pair<VEC> wagg[2][kNW][16];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int cq = lane & 15;
  const int s = lane >> 4;
  const int slot = w * 4 + s;

  // Workgroups are dispatched to the 8 XCDs round-robin by their linear id.
  // Give each XCD a contiguous range of channel groups (at 8 batch rows of 64
  // groups: one batch row per XCD), so that the rows an XCD streams at a time
  // step are one contiguous span (scan_large: forward 1.27 -> 1.19 ms,
  // backward 2.05 -> 2.01 ms against the plain order).
  const int64_t ng = gridDim.x;
  const int64_t g = ng % 8 == 0 ? (int64_t)(blockIdx.x % 8) * (ng / 8) + blockIdx.x / 8
                                : (int64_t)blockIdx.x;
  const int64_t seg = blockIdx.y;
  const int64_t bb = g / p.groups_per_batch;
  const int64_t c = (g % p.groups_per_batch) * CG + cq * VEC;
  const bool cvalid = c < p.D;  // VEC = 4 implies D % 4 == 0
  const int64_t T = p.T, D = p.D;
  const int64_t u_begin = seg * p.seg_len;
  const int64_t u_end = min(T, u_begin + p.seg_len);
  const int64_t base = bb * T * D + c;

  // carry: the state entering this segment (main pass) or the composed pair
  // of the steps seen so far (AGG pass)
  float cA[VEC], cS[VEC];
  fillv<VEC>(cA, 1.0f);
  fillv<VEC>(cS, 0.0f);
  if constexpr (!AGG) {
    if (cvalid && p.init) ldv<VEC>(p.init + bb * D + c, cS);
    for (int64_t q = 0; q < seg; ++q) {
      if (cvalid) {
        const float2 *ap = p.agg + q * p.B * D + bb * D + c;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float2 pr = ap[e];
          cS[e] = pr.x * cS[e] + pr.y;
        }
      }
    }
  }

  // Loads of one block of kK steps for this lane; steps outside the segment
  // (or channels past D) load the identity pair (1, 0).
  auto load_block = [&](int64_t ub, float (&av)[kK][VEC], float (&xv)[kK][VEC],
                        float (&hv)[kK][VEC]) {
#pragma unroll
    for (int i = 0; i < kK; ++i) {
      const int64_t u = ub + slot * kK + i;
      const bool ok = cvalid && u < u_end;
      fillv<VEC>(av[i], 1.0f);
      fillv<VEC>(xv[i], 0.0f);
      fillv<VEC>(hv[i], 0.0f);
      if (ok) {
        if constexpr (DIR == 0) {
          ldv<VEC>(p.a + base + u * D, av[i]);
          ldv<VEC>(p.x + base + u * D, xv[i]);
        } else {
          const int64_t t = T - 1 - u;
          if (t + 1 < T) ldv<VEC>(p.a + base + (t + 1) * D, av[i]);
          ldv<VEC>(p.x + base + t * D, xv[i]);
          if constexpr (!AGG) {
            if (t >= 1) {
              ldv<VEC>(p.hprev + base + (t - 1) * D, hv[i]);
            } else if (p.h0) {
              ldv<VEC>(p.h0 + bb * D + c, hv[i]);
            }
          }
        }
      }
    }
  };

  float av[kK][VEC], xv[kK][VEC], hv[kK][VEC];
#if CLA_SCAN_PREFETCH
  float nav[kK][VEC], nxv[kK][VEC], nhv[kK][VEC];
  load_block(u_begin, av, xv, hv);
#endif
  int it = 0;
  for (int64_t ub = u_begin; ub < u_end; ub += kBlock, ++it) {
#if CLA_SCAN_PREFETCH
    // issue the next block's loads before working on this one; the LDS-only
    // barrier below does not wait for them
    if (ub + kBlock < u_end) load_block(ub + kBlock, nav, nxv, nhv);
#else
    load_block(ub, av, xv, hv);
#endif

    // serial compose of this lane's kK steps (earlier step on the left)
    float A[VEC], S[VEC];
    fillv<VEC>(A, 1.0f);
    fillv<VEC>(S, 0.0f);
#pragma unroll
    for (int i = 0; i < kK; ++i) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        S[e] = av[i][e] * S[e] + xv[i][e];
        A[e] = A[e] * av[i][e];
      }
    }

    // Hillis-Steele over the 4 slots of the wave: shifts of 1 and 2 slots
#pragma unroll
    for (int sh = 16; sh < 64; sh <<= 1) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float pA = __shfl_up(A[e], sh, 64);
        const float pS = __shfl_up(S[e], sh, 64);
        if (lane >= sh) {
          S[e] = A[e] * pS + S[e];
          A[e] = A[e] * pA;
        }
      }
    }
    // exclusive prefix inside the wave
    float eA[VEC], eS[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      eA[e] = __shfl_up(A[e], 16, 64);
      eS[e] = __shfl_up(S[e], 16, 64);
      if (lane < 16) {
        eA[e] = 1.0f;
        eS[e] = 0.0f;
      }
    }
    const int buf = it & 1;
    if (s == 3) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        wagg[buf][w][cq].A[e] = A[e];
        wagg[buf][w][cq].S[e] = S[e];
      }
    }
    __syncthreads();

    // fold the wave aggregates onto the carry; remember the state entering
    // this wave
    float hs[VEC];
    fillv<VEC>(hs, 0.0f);
#pragma unroll
    for (int u = 0; u < kNW; ++u) {
      if (u == w) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) hs[e] = cS[e];
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float wa = wagg[buf][u][cq].A[e];
        const float ws = wagg[buf][u][cq].S[e];
        cS[e] = wa * cS[e] + ws;
        if constexpr (AGG) cA[e] = cA[e] * wa;
      }
    }

    if constexpr (!AGG) {
      float st[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) st[e] = eA[e] * hs[e] + eS[e];
#pragma unroll
      for (int i = 0; i < kK; ++i) {
        const int64_t u = ub + slot * kK + i;
#pragma unroll
        for (int e = 0; e < VEC; ++e) st[e] = av[i][e] * st[e] + xv[i][e];
        if (cvalid && u < u_end) {
          const int64_t t = DIR == 0 ? u : T - 1 - u;
          stv<VEC>(p.y + base + t * D, st);
          if constexpr (DIR == 1) {
            float dav[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) dav[e] = st[e] * hv[i][e];
            stv<VEC>(p.y2 + base + t * D, dav);
          }
        }
      }
    }
#if CLA_SCAN_PREFETCH
#pragma unroll
    for (int i = 0; i < kK; ++i) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        av[i][e] = nav[i][e];
        xv[i][e] = nxv[i][e];
        hv[i][e] = nhv[i][e];
      }
    }
#endif
  }

  if (w == 0 && s == 0 && cvalid) {
    if constexpr (AGG) {
      float2 *ap = p.agg + seg * p.B * D + bb * D + c;
#pragma unroll
      for (int e = 0; e < VEC; ++e) ap[e] = make_float2(cA[e], cS[e]);
    } else {
      if (seg == p.P - 1 && p.fin) {
        if constexpr (DIR == 0) {
          stv<VEC>(p.fin + bb * D + c, cS);
        } else {
          float a0[VEC];
          ldv<VEC>(p.a + base, a0);  // a_1, the decay of the first step
          float d0[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) d0[e] = a0[e] * cS[e];
          stv<VEC>(p.fin + bb * D + c, d0);
        }
      }
    }
  }
}

__global__ void copy_or_zero_kernel(float *dst, const float *src, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

bool aligned16(const void *ptr) {
  return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

template <int VEC, int DIR>
hipError_t run(ScanArgs args, const ScanPlan &plan, hipStream_t stream) {
  constexpr int CG = 16 * VEC;
  constexpr int kNW = DIR == 0 ? CLA_SCAN_FWD_NW : CLA_SCAN_BWD_NW;
  constexpr int kK = DIR == 0 ? CLA_SCAN_FWD_K : CLA_SCAN_BWD_K;
  args.groups_per_batch = (args.D + CG - 1) / CG;
  const int64_t groups = args.B * args.groups_per_batch;
  if (plan.P > 1) {
    dim3 grid((unsigned)groups, (unsigned)(plan.P - 1));
    CLA_LAUNCH(DIR == 0 ? "scan_fwd_segments" : "scan_bwd_segments",
               (scan_kernel<VEC, DIR, true, kNW, kK>), grid, dim3(kNW * 64), stream, args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)groups, (unsigned)plan.P);
  CLA_LAUNCH(DIR == 0 ? "scan_fwd" : "scan_bwd", (scan_kernel<VEC, DIR, false, kNW, kK>),
             grid, dim3(kNW * 64), stream, args);
  return hipGetLastError();
}

}  // namespace

ScanPlan plan_scan(int64_t B, int64_t T, int64_t D) {
  ScanPlan plan;
  plan.seg_len = T;
  if (B <= 0 || T <= 0 || D <= 0) return plan;
  const int64_t groups = B * ((D + 63) / 64);
  const int64_t nblk = (T + kPlanBlock - 1) / kPlanBlock;
  int64_t P = 1;
  if (groups < kTargetGroups) {
    P = (kTargetGroups + groups - 1) / groups;
    if (P > nblk) P = nblk;
  }
  const int64_t seg_blocks = (nblk + P - 1) / P;
  P = (nblk + seg_blocks - 1) / seg_blocks;
  plan.P = P;
  plan.seg_len = seg_blocks * kPlanBlock;
  plan.ws_bytes = (size_t)(P - 1) * (size_t)B * (size_t)D * sizeof(float2);
  return plan;
}

hipError_t launch_scan_fwd(const float *a, const float *b, const float *h0,
                           float *h, float *hT, int64_t B, int64_t T,
                           int64_t D, const ScanPlan &plan, void *ws,
                           hipStream_t stream) {
  ScanArgs args{};
  args.a = a;
  args.x = b;
  args.init = h0;
  args.y = h;
  args.fin = hT;
  args.agg = static_cast<float2 *>(ws);
  args.B = B;
  args.T = T;
  args.D = D;
  args.seg_len = plan.seg_len;
  args.P = plan.P;
  const bool v4 = (D % 4 == 0) && aligned16(a) && aligned16(b) && aligned16(h) &&
                  (!h0 || aligned16(h0)) && (!hT || aligned16(hT));
  return v4 ? run<4, 0>(args, plan, stream) : run<1, 0>(args, plan, stream);
}

hipError_t launch_scan_bwd(const float *a, const float *h, const float *h0,
                           const float *dh, const float *dhT, float *da,
                           float *db, float *dh0, int64_t B, int64_t T,
                           int64_t D, const ScanPlan &plan, void *ws,
                           hipStream_t stream) {
  ScanArgs args{};
  args.a = a;
  args.x = dh;
  args.hprev = h;
  args.init = dhT;
  args.h0 = h0;
  args.y = db;
  args.y2 = da;
  args.fin = dh0;
  args.agg = static_cast<float2 *>(ws);
  args.B = B;
  args.T = T;
  args.D = D;
  args.seg_len = plan.seg_len;
  args.P = plan.P;
  const bool v4 = (D % 4 == 0) && aligned16(a) && aligned16(h) && aligned16(dh) &&
                  aligned16(da) && aligned16(db) && (!h0 || aligned16(h0)) &&
                  (!dhT || aligned16(dhT)) && (!dh0 || aligned16(dh0));
  return v4 ? run<4, 1>(args, plan, stream) : run<1, 1>(args, plan, stream);
}

// ---------------------------------------------------------------------------
// Forward scan without a caller workspace
// ---------------------------------------------------------------------------
// The segment pairs go to `scratch`, a fixed array that every GPU the library
// runs on holds once, until the process ends.  The planner never needs more:
// the time axis is split only when groups = B * ceil(D / 64) < kTargetGroups,
// into P <= ceil(kTargetGroups / groups) segments, so (P - 1) * B * D <=
// (kTargetGroups - 1) / groups * 64 * groups < 64 * kTargetGroups pairs.
// Every pair the main pass reads is written by the segment pass of the same
// call, so the array is never cleared; calls that overlap on one GPU share it
// and race.
namespace {

constexpr int64_t kScratchPairs = (int64_t)(kScanNoAllocScratchBytes / sizeof(float2));
static_assert(64 * kTargetGroups <= kScratchPairs, "scratch smaller than the largest plan");
static __device__ __align__(256) float2 scratch[kScratchPairs];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float2 *scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

}  // namespace

hipError_t launch_scan_fwd_noalloc(const float *a, const float *b, const float *h0,
                                   float *h, float *hT, int64_t B, int64_t T,
                                   int64_t D, const ScanPlan &plan,
                                   hipStream_t stream) {
  if (plan.ws_bytes > kScanNoAllocScratchBytes) return hipErrorInvalidValue;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float2 *ptr = nullptr;
  {
    std::lock_guard<std::mutex> g(scratch_mu);
    if (!scratch_ptr[dev]) {
      // once per device, with that device current: the host-side name of the
      // array is not a device address, so kernels get this address instead
      void *addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!addr) return hipErrorInvalidSymbol;
      scratch_ptr[dev] = static_cast<float2 *>(addr);
    }
    ptr = scratch_ptr[dev];
  }
  return launch_scan_fwd(a, b, h0, h, hT, B, T, D, plan, ptr, stream);
}

hipError_t launch_copy_or_zero(float *dst, const float *src, int64_t n,
                               hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  CLA_LAUNCH("copy_or_zero", copy_or_zero_kernel, dim3((unsigned)blocks), dim3(threads),
             stream, dst, src, n);
  return hipGetLastError();
}

}  // namespace cla
