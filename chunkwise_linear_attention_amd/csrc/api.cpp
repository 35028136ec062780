// The C ABI of libcla (declared in include/cla.h): host-side argument
// validation, workspace sizing and kernel launches.  Every check runs before
// the first HIP call, so a rejected call touches no device state.
#include <stdint.h>
#include <string.h>

#include <initializer_list>

#include "../../include/cla.h"
#include "gla_kernels.h"
#include "internal.h"
#include "sscan_kernels.h"

namespace {

struct Range {
  const void *p;
  size_t bytes;
};

bool overlap(const Range &x, const Range &y) {
  if (!x.p || !y.p || x.bytes == 0 || y.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), a1 = a0 + x.bytes;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(y.p), b1 = b0 + y.bytes;
  return a0 < b1 && b0 < a1;
}

// Every output must be disjoint from every input and from every other output.
bool any_alias(std::initializer_list<Range> inputs,
               std::initializer_list<Range> outputs) {
  for (const Range &o : outputs) {
    for (const Range &i : inputs)
      if (overlap(o, i)) return true;
    for (const Range &o2 : outputs)
      if (&o2 != &o && overlap(o, o2)) return true;
  }
  return false;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CLA_OK : CLA_ERR_HIP; }

bool supported_head_dim(int64_t d) { return d == 64 || d == 128; }

// bf16 tiles are moved in 16-byte pieces
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

const char *cla_status_string(int status) {
  switch (status) {
    case CLA_OK: return "CLA_OK";
    case CLA_ERR_NULL_ARG: return "CLA_ERR_NULL_ARG: a required pointer is NULL";
    case CLA_ERR_BAD_SHAPE: return "CLA_ERR_BAD_SHAPE: a size is negative";
    case CLA_ERR_UNSUPPORTED: return "CLA_ERR_UNSUPPORTED: a size, alignment or option is not supported";
    case CLA_ERR_WORKSPACE: return "CLA_ERR_WORKSPACE: workspace missing or too small";
    case CLA_ERR_ALIAS: return "CLA_ERR_ALIAS: an output overlaps an input or another output";
    case CLA_ERR_HIP: return "CLA_ERR_HIP: a HIP launch failed";
    default: return "CLA_ERR_UNKNOWN";
  }
}

const char *cla_version(void) { return "cla 0.1 gfx950"; }

int cla_check_log_decay(const float *log_decay, int64_t n, uint32_t *counts,
                        cla_stream_t stream) {
  if (n < 0) return CLA_ERR_BAD_SHAPE;
  if (!counts || (n > 0 && !log_decay)) return CLA_ERR_NULL_ARG;
  if ((reinterpret_cast<uintptr_t>(counts) & 3) != 0) return CLA_ERR_UNSUPPORTED;
  if (any_alias({{log_decay, (size_t)n * sizeof(float)}}, {{counts, 4 * sizeof(uint32_t)}}))
    return CLA_ERR_ALIAS;
  return hip_status(
      cla::launch_check_log_decay(log_decay, n, counts, reinterpret_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// diagonal scan
// ---------------------------------------------------------------------------

size_t cla_scan_workspace_bytes(int64_t B, int64_t T, int64_t D) {
  if (B < 0 || T < 0 || D < 0) return 0;
  return cla::plan_scan(B, T, D).ws_bytes;
}

int cla_scan_fwd(const float *a, const float *b, const float *h0, float *h,
                 float *hT, int64_t B, int64_t T, int64_t D, void *workspace,
                 size_t workspace_bytes, cla_stream_t stream) {
  if (B < 0 || T < 0 || D < 0) return CLA_ERR_BAD_SHAPE;
  if (B == 0 || D == 0) return CLA_OK;
  const size_t full = (size_t)B * (size_t)T * (size_t)D * sizeof(float);
  const size_t row = (size_t)B * (size_t)D * sizeof(float);
  if (T > 0 && (!a || !b || !h)) return CLA_ERR_NULL_ARG;
  const cla::ScanPlan plan = cla::plan_scan(B, T, D);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return CLA_ERR_WORKSPACE;
  const Range ws{plan.ws_bytes ? workspace : nullptr, plan.ws_bytes};
  if (any_alias({{a, full}, {b, full}, {h0, row}}, {{h, full}, {hT, row}, ws}))
    return CLA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0) return hT ? hip_status(cla::launch_copy_or_zero(hT, h0, B * D, s)) : CLA_OK;
  return hip_status(cla::launch_scan_fwd(a, b, h0, h, hT, B, T, D, plan, workspace, s));
}

int cla_scan_fwd_noalloc(const float *a, const float *b, const float *h0, float *h,
                         float *hT, int64_t B, int64_t T, int64_t D, cla_stream_t stream) {
  static_assert(cla::kScanNoAllocScratchBytes == CLA_SCAN_NOALLOC_SCRATCH_BYTES, "header");
  if (B < 0 || T < 0 || D < 0) return CLA_ERR_BAD_SHAPE;
  if (B == 0 || D == 0) return CLA_OK;
  const size_t full = (size_t)B * (size_t)T * (size_t)D * sizeof(float);
  const size_t row = (size_t)B * (size_t)D * sizeof(float);
  if (T > 0 && (!a || !b || !h)) return CLA_ERR_NULL_ARG;
  const cla::ScanPlan plan = cla::plan_scan(B, T, D);
  if (plan.ws_bytes > cla::kScanNoAllocScratchBytes) return CLA_ERR_WORKSPACE;
  if (any_alias({{a, full}, {b, full}, {h0, row}}, {{h, full}, {hT, row}}))
    return CLA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0) return hT ? hip_status(cla::launch_copy_or_zero(hT, h0, B * D, s)) : CLA_OK;
  // the fixed array is looked up on the current device, so the stream must
  // belong to it
  if (s) {
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(s, &sdev) != hipSuccess)
      return CLA_ERR_HIP;
    if (cur != sdev) return CLA_ERR_UNSUPPORTED;
  }
  return hip_status(cla::launch_scan_fwd_noalloc(a, b, h0, h, hT, B, T, D, plan, s));
}

int cla_scan_bwd(const float *a, const float *h, const float *h0,
                 const float *dh, const float *dhT, float *da, float *db,
                 float *dh0, int64_t B, int64_t T, int64_t D, void *workspace,
                 size_t workspace_bytes, cla_stream_t stream) {
  if (B < 0 || T < 0 || D < 0) return CLA_ERR_BAD_SHAPE;
  if (B == 0 || D == 0) return CLA_OK;
  const size_t full = (size_t)B * (size_t)T * (size_t)D * sizeof(float);
  const size_t row = (size_t)B * (size_t)D * sizeof(float);
  if (T > 0 && (!a || !h || !dh || !da || !db)) return CLA_ERR_NULL_ARG;
  const cla::ScanPlan plan = cla::plan_scan(B, T, D);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return CLA_ERR_WORKSPACE;
  const Range ws{plan.ws_bytes ? workspace : nullptr, plan.ws_bytes};
  if (any_alias({{a, full}, {h, full}, {h0, row}, {dh, full}, {dhT, row}},
                {{da, full}, {db, full}, {dh0, row}, ws}))
    return CLA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0) return dh0 ? hip_status(cla::launch_copy_or_zero(dh0, dhT, B * D, s)) : CLA_OK;
  return hip_status(
      cla::launch_scan_bwd(a, h, h0, dh, dhT, da, db, dh0, B, T, D, plan, workspace, s));
}

// ---------------------------------------------------------------------------
// chunkwise linear attention
// ---------------------------------------------------------------------------

size_t cla_chunk_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t DK,
                                 int64_t DV, int64_t chunk, int backward) {
  if (B < 0 || H < 0 || T < 0) return 0;
  if (!supported_head_dim(DK) || !supported_head_dim(DV) || chunk != 64) return 0;
  const cla::ChunkPlan plan = cla::plan_chunk(B, H, T, DK, DV);
  return backward ? plan.ws_bwd : plan.ws_fwd;
}

}  // extern "C"

namespace {

// The forward with an optional saved-state output (`saved_bytes` is ignored
// when `with_saved` is false).
int chunk_fwd_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const float *log_decay, const float *S0, uint16_t *o, float *ST,
                   bool with_saved, float *saved, size_t saved_bytes, int64_t B, int64_t H,
                   int64_t T, int64_t DK, int64_t DV, int64_t chunk, void *workspace,
                   size_t workspace_bytes, cla_stream_t stream) {
  if (B < 0 || H < 0 || T < 0 || DK < 0 || DV < 0 || chunk < 0) return CLA_ERR_BAD_SHAPE;
  if (!supported_head_dim(DK) || !supported_head_dim(DV) || chunk != 64)
    return CLA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return CLA_OK;
  const size_t nh = (size_t)B * (size_t)H;
  const size_t qk = nh * (size_t)T * (size_t)DK * 2, vv = nh * (size_t)T * (size_t)DV * 2;
  const size_t ll = nh * (size_t)T * 4, ss = nh * (size_t)DK * (size_t)DV * 4;
  if (T > 0 && (!q || !k || !v || !log_decay || !o)) return CLA_ERR_NULL_ARG;
  if (T > 0 && !(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o)))
    return CLA_ERR_UNSUPPORTED;
  const cla::ChunkPlan plan = cla::plan_chunk(B, H, T, DK, DV);
  if (!cla::chunk_plan_launchable(plan, B * H)) return CLA_ERR_UNSUPPORTED;
  if (plan.ws_fwd > 0 && (!workspace || workspace_bytes < plan.ws_fwd))
    return CLA_ERR_WORKSPACE;
  const size_t sv = with_saved ? plan.saved_bytes : 0;
  if (sv > 0 && (!saved || saved_bytes < sv)) return CLA_ERR_WORKSPACE;
  const Range ws{plan.ws_fwd ? workspace : nullptr, plan.ws_fwd};
  if (any_alias({{q, qk}, {k, qk}, {v, vv}, {log_decay, ll}, {S0, ss}},
                {{o, vv}, {ST, ss}, ws, {sv ? saved : nullptr, sv}}))
    return CLA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0)
    return ST ? hip_status(cla::launch_copy_or_zero(ST, S0, (int64_t)(nh * DK * DV), s))
              : CLA_OK;
  return hip_status(cla::launch_chunk_fwd(q, k, v, log_decay, S0, o, ST, sv ? saved : nullptr,
                                          B, H, T, DK, DV, plan, workspace, s));
}

int chunk_bwd_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const float *log_decay, const float *S0, const uint16_t *dO,
                   const float *dST, bool with_saved, const float *saved, size_t saved_bytes,
                   uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dlog_decay, float *dS0,
                   int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV, int64_t chunk,
                   void *workspace, size_t workspace_bytes, cla_stream_t stream) {
  if (B < 0 || H < 0 || T < 0 || DK < 0 || DV < 0 || chunk < 0) return CLA_ERR_BAD_SHAPE;
  if (!supported_head_dim(DK) || !supported_head_dim(DV) || chunk != 64)
    return CLA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return CLA_OK;
  const size_t nh = (size_t)B * (size_t)H;
  const size_t qk = nh * (size_t)T * (size_t)DK * 2, vv = nh * (size_t)T * (size_t)DV * 2;
  const size_t ll = nh * (size_t)T * 4, ss = nh * (size_t)DK * (size_t)DV * 4;
  if (T > 0 && (!q || !k || !v || !log_decay || !dO || !dq || !dk || !dv || !dlog_decay))
    return CLA_ERR_NULL_ARG;
  if (T > 0 && !(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(dO) &&
                 aligned16(dq) && aligned16(dk) && aligned16(dv)))
    return CLA_ERR_UNSUPPORTED;
  const cla::ChunkPlan plan = cla::plan_chunk(B, H, T, DK, DV);
  if (!cla::chunk_plan_launchable(plan, B * H)) return CLA_ERR_UNSUPPORTED;
  if (plan.ws_bwd > 0 && (!workspace || workspace_bytes < plan.ws_bwd))
    return CLA_ERR_WORKSPACE;
  const size_t sv = with_saved ? plan.saved_bytes : 0;
  if (sv > 0 && (!saved || saved_bytes < sv)) return CLA_ERR_WORKSPACE;
  const Range ws{plan.ws_bwd ? workspace : nullptr, plan.ws_bwd};
  if (any_alias({{q, qk}, {k, qk}, {v, vv}, {log_decay, ll}, {S0, ss}, {dO, vv}, {dST, ss},
                 {sv ? saved : nullptr, sv}},
                {{dq, qk}, {dk, qk}, {dv, vv}, {dlog_decay, ll}, {dS0, ss}, ws}))
    return CLA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0)
    return dS0 ? hip_status(cla::launch_copy_or_zero(dS0, dST, (int64_t)(nh * DK * DV), s))
               : CLA_OK;
  return hip_status(cla::launch_chunk_bwd(q, k, v, log_decay, S0, dO, dST,
                                          sv ? saved : nullptr, dq, dk, dv, dlog_decay, dS0,
                                          B, H, T, DK, DV, plan, workspace, s));
}

}  // namespace

extern "C" {

int cla_chunk_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const float *log_decay, const float *S0, uint16_t *o,
                  float *ST, int64_t B, int64_t H, int64_t T, int64_t DK,
                  int64_t DV, int64_t chunk, void *workspace,
                  size_t workspace_bytes, cla_stream_t stream) {
  return chunk_fwd_impl(q, k, v, log_decay, S0, o, ST, false, nullptr, 0, B, H, T, DK, DV,
                        chunk, workspace, workspace_bytes, stream);
}

int cla_chunk_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const float *log_decay, const float *S0, const uint16_t *dO,
                  const float *dST, uint16_t *dq, uint16_t *dk, uint16_t *dv,
                  float *dlog_decay, float *dS0, int64_t B, int64_t H,
                  int64_t T, int64_t DK, int64_t DV, int64_t chunk,
                  void *workspace, size_t workspace_bytes,
                  cla_stream_t stream) {
  return chunk_bwd_impl(q, k, v, log_decay, S0, dO, dST, false, nullptr, 0, dq, dk, dv,
                        dlog_decay, dS0, B, H, T, DK, DV, chunk, workspace, workspace_bytes,
                        stream);
}

size_t cla_chunk_saved_bytes(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV,
                             int64_t chunk) {
  if (B < 0 || H < 0 || T < 0) return 0;
  if (!supported_head_dim(DK) || !supported_head_dim(DV) || chunk != 64) return 0;
  return cla::plan_chunk(B, H, T, DK, DV).saved_bytes;
}

int cla_chunk_fwd_saved(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const float *log_decay, const float *S0, uint16_t *o, float *ST,
                        float *saved, size_t saved_bytes, int64_t B, int64_t H, int64_t T,
                        int64_t DK, int64_t DV, int64_t chunk, void *workspace,
                        size_t workspace_bytes, cla_stream_t stream) {
  return chunk_fwd_impl(q, k, v, log_decay, S0, o, ST, true, saved, saved_bytes, B, H, T, DK,
                        DV, chunk, workspace, workspace_bytes, stream);
}

int cla_chunk_bwd_saved(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const float *log_decay, const float *S0, const uint16_t *dO,
                        const float *dST, const float *saved, size_t saved_bytes, uint16_t *dq,
                        uint16_t *dk, uint16_t *dv, float *dlog_decay, float *dS0, int64_t B,
                        int64_t H, int64_t T, int64_t DK, int64_t DV, int64_t chunk,
                        void *workspace, size_t workspace_bytes, cla_stream_t stream) {
  return chunk_bwd_impl(q, k, v, log_decay, S0, dO, dST, true, saved, saved_bytes, dq, dk, dv,
                        dlog_decay, dS0, B, H, T, DK, DV, chunk, workspace, workspace_bytes,
                        stream);
}


// ---- one decay per key dimension ----

size_t cla_gla_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV,
                               int64_t chunk, int backward) {
  if (B < 0 || H < 0 || T < 0) return 0;
  if (!supported_head_dim(DK) || !supported_head_dim(DV) || chunk != 64) return 0;
  if (B == 0 || H == 0 || T == 0) return 0;
  return backward ? cla::gla::gla_bwd_ws_bytes(B * H, T, DK, DV)
                  : cla::gla::gla_fwd_ws_bytes(B * H, T, DK, DV);
}

size_t cla_gla_saved_bytes(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV,
                           int64_t chunk) {
  if (B < 0 || H < 0 || T < 0) return 0;
  if (!supported_head_dim(DK) || !supported_head_dim(DV) || chunk != 64) return 0;
  if (B == 0 || H == 0 || T == 0) return 0;
  const cla::gla::GlaPlan plan = cla::gla::plan_gla(B * H, T);
  return plan.P > 1 ? (size_t)(plan.P - 1) * (size_t)(B * H) * DK * DV * sizeof(float) : 0;
}

namespace {

// saved != NULL or use_saved: the forward's segment start states go to
// `saved` (cla_gla_fwd_saved) instead of the workspace.
int gla_fwd_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                 const float *log_decay, const float *S0, uint16_t *o, float *ST, bool use_saved,
                 float *saved, size_t saved_bytes, int64_t B, int64_t H, int64_t T, int64_t DK,
                 int64_t DV, int64_t chunk, void *workspace, size_t workspace_bytes,
                 cla_stream_t stream) {
  if (B < 0 || H < 0 || T < 0 || DK < 0 || DV < 0 || chunk < 0) return CLA_ERR_BAD_SHAPE;
  if (!supported_head_dim(DK) || !supported_head_dim(DV) || chunk != 64)
    return CLA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return CLA_OK;
  const size_t nh = (size_t)B * (size_t)H;
  if (nh > 0x7fffffffu) return CLA_ERR_UNSUPPORTED;
  const size_t qk = nh * (size_t)T * (size_t)DK * 2, vv = nh * (size_t)T * (size_t)DV * 2;
  const size_t ll = nh * (size_t)T * (size_t)DK * 4, ss = nh * (size_t)DK * (size_t)DV * 4;
  if (T > 0 && (!q || !k || !v || !log_decay || !o)) return CLA_ERR_NULL_ARG;
  if (T > 0 && !(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) &&
                 aligned16(log_decay)))
    return CLA_ERR_UNSUPPORTED;
  const cla::gla::GlaPlan plan = cla::gla::plan_gla((int64_t)nh, T);
  if (plan.P > 65535) return CLA_ERR_UNSUPPORTED;
  const size_t need = T > 0 ? cla::gla::gla_fwd_ws_bytes((int64_t)nh, T, DK, DV) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return CLA_ERR_WORKSPACE;
  const size_t sneed = use_saved && T > 0 ? cla_gla_saved_bytes(B, H, T, DK, DV, chunk) : 0;
  if (sneed > 0 && (!saved || saved_bytes < sneed || !aligned16(saved)))
    return CLA_ERR_WORKSPACE;
  const Range ws{need ? workspace : nullptr, need};
  const Range sv{sneed ? saved : nullptr, sneed};
  if (any_alias({{q, qk}, {k, qk}, {v, vv}, {log_decay, ll}, {S0, ss}},
                {{o, vv}, {ST, ss}, ws, sv}))
    return CLA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0)
    return ST ? hip_status(cla::launch_copy_or_zero(ST, S0, (int64_t)(nh * DK * DV), s))
              : CLA_OK;
  cla::gla::GlaFwdArgs a{};
  a.P = plan.P;
  a.seg_chunks = plan.seg_chunks;
  if (plan.P > 1) {
    const size_t sl = (((size_t)(plan.P - 1) * nh * DK * DV * sizeof(float)) + 255) & ~(size_t)255;
    a.Sloc = sneed ? saved : static_cast<float *>(workspace);
    a.Aseg = reinterpret_cast<float *>(static_cast<char *>(workspace) + sl);
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.l = log_decay;
  a.S0 = S0;
  a.o = o;
  a.ST = ST;
  a.nh = (int64_t)nh;
  a.T = T;
  return hip_status(cla::gla::gla_fwd_dispatch(a, (int)DK, (int)DV, s));
}


// use_saved: the segments start from the forward's saved states (no state pass).
int gla_bwd_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                 const float *log_decay, const float *S0, const uint16_t *dO, const float *dST,
                 bool use_saved, const float *saved, size_t saved_bytes, uint16_t *dq,
                 uint16_t *dk, uint16_t *dv, float *dlog_decay, float *dS0, int64_t B, int64_t H,
                 int64_t T, int64_t DK, int64_t DV, int64_t chunk, void *workspace,
                 size_t workspace_bytes, cla_stream_t stream) {
  if (B < 0 || H < 0 || T < 0 || DK < 0 || DV < 0 || chunk < 0) return CLA_ERR_BAD_SHAPE;
  if (!supported_head_dim(DK) || !supported_head_dim(DV) || chunk != 64)
    return CLA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return CLA_OK;
  const size_t nh = (size_t)B * (size_t)H;
  if (nh > 0x7fffffffu) return CLA_ERR_UNSUPPORTED;
  const size_t qk = nh * (size_t)T * (size_t)DK * 2, vv = nh * (size_t)T * (size_t)DV * 2;
  const size_t ll = nh * (size_t)T * (size_t)DK * 4, ss = nh * (size_t)DK * (size_t)DV * 4;
  if (T > 0 && (!q || !k || !v || !log_decay || !dO || !dq || !dk || !dv || !dlog_decay))
    return CLA_ERR_NULL_ARG;
  if (T > 0 && !(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(dO) &&
                 aligned16(dq) && aligned16(dk) && aligned16(dv) && aligned16(log_decay) &&
                 aligned16(dlog_decay)))
    return CLA_ERR_UNSUPPORTED;
  if (cla::gla::plan_gla((int64_t)nh, T).P > 65535) return CLA_ERR_UNSUPPORTED;
  const size_t need = T > 0 ? cla::gla::gla_bwd_ws_bytes((int64_t)nh, T, DK, DV) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return CLA_ERR_WORKSPACE;
  const size_t sneed = use_saved && T > 0 ? cla_gla_saved_bytes(B, H, T, DK, DV, chunk) : 0;
  if (sneed > 0 && (!saved || saved_bytes < sneed || !aligned16(saved)))
    return CLA_ERR_WORKSPACE;
  const Range ws{need ? workspace : nullptr, need};
  if (any_alias({{q, qk}, {k, qk}, {v, vv}, {log_decay, ll}, {S0, ss}, {dO, vv}, {dST, ss},
                 {saved, sneed}},
                {{dq, qk}, {dk, qk}, {dv, vv}, {dlog_decay, ll}, {dS0, ss}, ws}))
    return CLA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0)
    return dS0 ? hip_status(cla::launch_copy_or_zero(dS0, dST, (int64_t)(nh * DK * DV), s))
               : CLA_OK;
  const cla::gla::GlaPlan plan = cla::gla::plan_gla((int64_t)nh, T);
  auto r256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t r1_bytes = r256((size_t)nh * T * DK * sizeof(float));
  const int64_t nblk = ((T + 63) / 64 + cla::gla::kSegChunks - 1) / cla::gla::kSegChunks;
  char *wp = static_cast<char *>(workspace) + r1_bytes + r256((size_t)nblk * nh * DK * DV * 4);
  cla::gla::GlaBwdArgs a{};
  a.P = plan.P;
  a.seg_chunks = plan.seg_chunks;
  if (plan.P > 1 && sneed) {
    // the state each segment starts from, saved by the forward
    a.Sin = saved;
    wp += cla::gla::gla_fwd_ws_bytes((int64_t)nh, T, DK, DV);
    a.Gloc = reinterpret_cast<float *>(wp);
    a.Aq = reinterpret_cast<float *>(wp + r256((size_t)plan.P * nh * DK * DV * 4));
  } else if (plan.P > 1) {
    // the state each segment starts from: the forward's state pass and scan
    cla::gla::GlaFwdArgs f{};
    f.q = q;
    f.k = k;
    f.v = v;
    f.l = log_decay;
    f.S0 = S0;
    f.nh = (int64_t)nh;
    f.T = T;
    f.P = plan.P;
    f.seg_chunks = plan.seg_chunks;
    f.Sloc = reinterpret_cast<float *>(wp);
    f.Aseg = reinterpret_cast<float *>(wp + r256((size_t)(plan.P - 1) * nh * DK * DV * 4));
    const hipError_t e = cla::gla::gla_states_dispatch(f, (int)DK, (int)DV, s);
    if (e != hipSuccess) return hip_status(e);
    a.Sin = f.Sloc;
    wp += cla::gla::gla_fwd_ws_bytes((int64_t)nh, T, DK, DV);
    a.Gloc = reinterpret_cast<float *>(wp);
    a.Aq = reinterpret_cast<float *>(wp + r256((size_t)plan.P * nh * DK * DV * 4));
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.l = log_decay;
  a.S0 = S0;
  a.dST = dST;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dl = dlog_decay;
  a.dS0 = dS0;
  a.r1 = static_cast<float *>(workspace);
  a.Sseg = reinterpret_cast<float *>(static_cast<char *>(workspace) + r1_bytes);
  a.nh = (int64_t)nh;
  a.T = T;
  return hip_status(cla::gla::gla_bwd_dispatch(a, (int)DK, (int)DV, s));
}

}  // namespace

int cla_gla_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                const float *log_decay, const float *S0, uint16_t *o, float *ST, int64_t B,
                int64_t H, int64_t T, int64_t DK, int64_t DV, int64_t chunk, void *workspace,
                size_t workspace_bytes, cla_stream_t stream) {
  return gla_fwd_impl(q, k, v, log_decay, S0, o, ST, false, nullptr, 0, B, H, T, DK, DV, chunk,
                      workspace, workspace_bytes, stream);
}

int cla_gla_fwd_saved(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const float *log_decay, const float *S0, uint16_t *o, float *ST,
                      float *saved, size_t saved_bytes, int64_t B, int64_t H, int64_t T,
                      int64_t DK, int64_t DV, int64_t chunk, void *workspace,
                      size_t workspace_bytes, cla_stream_t stream) {
  return gla_fwd_impl(q, k, v, log_decay, S0, o, ST, true, saved, saved_bytes, B, H, T, DK, DV,
                      chunk, workspace, workspace_bytes, stream);
}

int cla_gla_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                const float *log_decay, const float *S0, const uint16_t *dO, const float *dST,
                uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dlog_decay, float *dS0,
                int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV, int64_t chunk,
                void *workspace, size_t workspace_bytes, cla_stream_t stream) {
  return gla_bwd_impl(q, k, v, log_decay, S0, dO, dST, false, nullptr, 0, dq, dk, dv,
                      dlog_decay, dS0, B, H, T, DK, DV, chunk, workspace, workspace_bytes, stream);
}

int cla_gla_bwd_saved(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const float *log_decay, const float *S0, const uint16_t *dO,
                      const float *dST, const float *saved, size_t saved_bytes, uint16_t *dq,
                      uint16_t *dk, uint16_t *dv, float *dlog_decay, float *dS0, int64_t B,
                      int64_t H, int64_t T, int64_t DK, int64_t DV, int64_t chunk,
                      void *workspace, size_t workspace_bytes, cla_stream_t stream) {
  return gla_bwd_impl(q, k, v, log_decay, S0, dO, dST, true, saved, saved_bytes, dq, dk, dv,
                      dlog_decay, dS0, B, H, T, DK, DV, chunk, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// selective scan (N state entries per channel)
// ---------------------------------------------------------------------------

static bool sscan_shape_ok(int64_t B, int64_t T, int64_t D, int64_t N) {
  return B >= 0 && T >= 0 && D >= 0 && N >= 0;
}

static bool sscan_supported(int64_t B, int64_t D, int64_t N) {
  return (N == 4 || N == 8 || N == 16) && D % 4 == 0 && D <= 0x7fffffc0 && B <= 65535;
}

size_t cla_sscan_ckpt_bytes(int64_t B, int64_t T, int64_t D, int64_t N) {
  if (!sscan_shape_ok(B, T, D, N) || !sscan_supported(B, D, N)) return 0;
  return cla::sscan::ckpt_bytes(B, T, D, N);
}

size_t cla_sscan_workspace_bytes(int64_t B, int64_t T, int64_t D, int64_t N, int backward,
                                 int have_ckpt) {
  if (!sscan_shape_ok(B, T, D, N) || !sscan_supported(B, D, N)) return 0;
  if (B == 0 || T == 0 || D == 0) return 0;
  return backward ? cla::sscan::bwd_ws_bytes(B, T, D, N, !have_ckpt)
                  : cla::sscan::fwd_ws_bytes(B, T, D, N);
}

int cla_sscan_fwd(const float *x, const float *delta, const float *A, const float *Bm,
                  const float *Cm, const float *h0, float *y, float *hT, float *ckpt, int64_t B,
                  int64_t T, int64_t D, int64_t N, void *workspace, size_t workspace_bytes,
                  cla_stream_t stream) {
  if (!sscan_shape_ok(B, T, D, N)) return CLA_ERR_BAD_SHAPE;
  if (!sscan_supported(B, D, N)) return CLA_ERR_UNSUPPORTED;
  if (B == 0 || D == 0) return CLA_OK;
  const size_t full = (size_t)(B * T * D) * 4, bn = (size_t)(B * T * N) * 4;
  const size_t st = (size_t)(B * D * N) * 4, an = (size_t)(D * N) * 4;
  const size_t ck = cla::sscan::ckpt_bytes(B, T, D, N);
  if (!A || (T > 0 && (!x || !delta || !Bm || !Cm || !y))) return CLA_ERR_NULL_ARG;
  if (!(aligned16(x) && aligned16(delta) && aligned16(Bm) && aligned16(Cm) && aligned16(y) &&
        aligned16(ckpt)))
    return CLA_ERR_UNSUPPORTED;
  const cla::sscan::Plan plan = cla::sscan::plan(B, T, D);
  if (plan.P > 65535) return CLA_ERR_UNSUPPORTED;
  const size_t need = T > 0 ? cla::sscan::fwd_ws_bytes(B, T, D, N) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return CLA_ERR_WORKSPACE;
  const Range ws{need ? workspace : nullptr, need};
  if (any_alias({{x, full}, {delta, full}, {A, an}, {Bm, bn}, {Cm, bn}, {h0, st}},
                {{y, full}, {hT, st}, {ckpt, ck}, ws}))
    return CLA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0)
    return hT ? hip_status(cla::launch_copy_or_zero(hT, h0, B * D * N, s)) : CLA_OK;
  cla::sscan::FwdArgs a{x, delta, A, Bm, Cm, h0, y, hT, ckpt, B, T, D, N, plan.P,
                        plan.seg_tiles, nullptr, nullptr};
  if (plan.P > 1) {
    a.Hloc = static_cast<float *>(workspace);
    a.Aprod = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                        cla::sscan::fwd_ws_bytes(B, T, D, N) / 2);
  }
  return hip_status(cla::sscan::fwd_dispatch(a, s));
}

int cla_sscan_bwd(const float *x, const float *delta, const float *A, const float *Bm,
                  const float *Cm, const float *h0, const float *ckpt, const float *dy,
                  const float *dhT, float *dx, float *ddelta, float *dA, float *dB, float *dC,
                  float *dh0, int64_t B, int64_t T, int64_t D, int64_t N, void *workspace,
                  size_t workspace_bytes, cla_stream_t stream) {
  if (!sscan_shape_ok(B, T, D, N)) return CLA_ERR_BAD_SHAPE;
  if (!sscan_supported(B, D, N)) return CLA_ERR_UNSUPPORTED;
  if (D == 0) return CLA_OK;
  const size_t full = (size_t)(B * T * D) * 4, bn = (size_t)(B * T * N) * 4;
  const size_t st = (size_t)(B * D * N) * 4, an = (size_t)(D * N) * 4;
  const size_t ck = cla::sscan::ckpt_bytes(B, T, D, N);
  if (!A || !dA || (B > 0 && T > 0 && (!x || !delta || !Bm || !Cm || !dy || !dx || !ddelta ||
                                       !dB || !dC)))
    return CLA_ERR_NULL_ARG;
  if (!(aligned16(x) && aligned16(delta) && aligned16(Bm) && aligned16(Cm) && aligned16(dy) &&
        aligned16(dx) && aligned16(ddelta) && aligned16(dB) && aligned16(dC) &&
        aligned16(ckpt)))
    return CLA_ERR_UNSUPPORTED;
  const cla::sscan::Plan plan = cla::sscan::plan(B, T, D);
  if (plan.P > 65535) return CLA_ERR_UNSUPPORTED;
  const size_t need = (B > 0 && T > 0) ? cla::sscan::bwd_ws_bytes(B, T, D, N, !ckpt) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return CLA_ERR_WORKSPACE;
  const Range ws{need ? workspace : nullptr, need};
  if (any_alias({{x, full}, {delta, full}, {A, an}, {Bm, bn}, {Cm, bn}, {h0, st}, {ckpt, ck},
                 {dy, full}, {dhT, st}},
                {{dx, full}, {ddelta, full}, {dA, an}, {dB, bn}, {dC, bn}, {dh0, st}, ws}))
    return CLA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (B == 0 || T == 0) {
    hipError_t e = cla::launch_copy_or_zero(dA, nullptr, D * N, s);
    if (e == hipSuccess && dh0 && B > 0) e = cla::launch_copy_or_zero(dh0, dhT, B * D * N, s);
    return hip_status(e);
  }
  const size_t bdn = (size_t)(B * D * N) * sizeof(float);
  char *w = static_cast<char *>(workspace);
  float *part = reinterpret_cast<float *>(w);
  w += cla::sscan::round256(cla::sscan::part_bytes(B, T, D, N));
  float *dAp = reinterpret_cast<float *>(w);
  w += cla::sscan::round256(plan.P * bdn);
  float *Gloc = nullptr, *Aprod = nullptr;
  if (plan.P > 1) {
    Gloc = reinterpret_cast<float *>(w);
    w += cla::sscan::round256(plan.P * bdn);
    Aprod = reinterpret_cast<float *>(w);
    w += cla::sscan::round256(plan.P * bdn);
  }
  if (!ckpt) {
    // no checkpoints from the forward: write them here first
    float *ck_ws = reinterpret_cast<float *>(w);
    w += cla::sscan::round256(cla::sscan::ckpt_bytes(B, T, D, N));
    cla::sscan::FwdArgs f{x, delta, A, Bm, Cm, h0, nullptr, nullptr, ck_ws, B, T, D, N, plan.P,
                          plan.seg_tiles, nullptr, nullptr};
    if (plan.P > 1) {
      f.Hloc = reinterpret_cast<float *>(w);
      f.Aprod = reinterpret_cast<float *>(w + cla::sscan::fwd_ws_bytes(B, T, D, N) / 2);
    }
    const hipError_t e = cla::sscan::fwd_dispatch(f, s);
    if (e != hipSuccess) return hip_status(e);
    ckpt = ck_ws;
  }
  cla::sscan::BwdArgs a{x, delta, A, Bm, Cm, ckpt, dy, dhT, dx, ddelta, dA, dB, dC, dh0,
                        part, dAp, B, T, D, N, plan.P, plan.seg_tiles, Gloc, Aprod};
  return hip_status(cla::sscan::bwd_dispatch(a, s));
}

}  // extern "C"
