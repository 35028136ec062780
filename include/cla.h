/*
 * cla.h -- C ABI of libcla, gated linear-recurrence scans for AMD MI355X
 * (gfx950).
 *
 * Two regimes of the recurrence h_t = a_t h_{t-1} + b_t:
 *
 *   diagonal state   h_t = a_t * h_{t-1} + b_t, elementwise per channel
 *                    ("Parallel scan", zerotofrontier.app ssm/parallel-scan,
 *                    sections "The scan for one number of state" and "A
 *                    vectorized scan for diagonal states"; "Parallel Scan",
 *                    aiwiki.thehackersbrain.dev, section "Composition").
 *
 *   matrix state     S_t = a_t S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t,
 *                    a_t = exp(l_t), computed chunkwise ("Parallel scan",
 *                    section "The chunkwise algorithm"; "Lightning
 *                    Attention-2: A Free Lunch for Handling Unlimited Sequence
 *                    Lengths in Large Language Models", Eq. 4-10 and Alg. 1).
 *
 * Conventions for every entry point:
 *   - Pointers named as inputs/outputs are DEVICE pointers owned by the
 *     caller; tensors are dense, row-major, contiguous.  The library never
 *     allocates, frees or synchronizes: it validates the arguments on the
 *     host, enqueues its kernels on `stream` (NULL = the default stream) and
 *     returns.  Results are ready when the stream reaches that point.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Arguments are checked on the host before any launch, in this order:
 *     shapes (negative -> CLA_ERR_BAD_SHAPE), unsupported sizes
 *     (CLA_ERR_UNSUPPORTED), required pointers (NULL -> CLA_ERR_NULL_ARG),
 *     workspace (too small -> CLA_ERR_WORKSPACE), outputs overlapping inputs
 *     or each other (CLA_ERR_ALIAS).  A failed check launches nothing.
 *     CLA_ERR_HIP reports a failed launch.
 *   - A zero-sized problem (B, D, H = 0) is a no-op.  T = 0 is an empty
 *     sequence: the final state equals the initial state (zeros if NULL) and
 *     the initial-state gradient equals the final-state gradient.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no atomics in any reduction).
 *   - Calls that share a workspace must be ordered (one stream, or events).
 */
#ifndef CLA_H
#define CLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream (hipStream_t); NULL selects the default stream. */
typedef struct ihipStream_t *cla_stream_t;

enum {
  CLA_OK = 0,
  CLA_ERR_NULL_ARG = 1,    /* a required pointer is NULL                      */
  CLA_ERR_BAD_SHAPE = 2,   /* a size is negative                              */
  CLA_ERR_UNSUPPORTED = 3, /* DK/DV not in {64, 128}, chunk != 64, misaligned,
                              chunkwise T > 67,107,840 or B*H >= 2^31 */
  CLA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required         */
  CLA_ERR_ALIAS = 5,       /* an output overlaps an input or another output   */
  CLA_ERR_HIP = 6          /* a HIP launch failed                             */
};

/* Human-readable name of a status code (static storage, never NULL). */
const char *cla_status_string(int status);

/* Library version string, e.g. "cla 0.1 gfx950". */
const char *cla_version(void);

/*
 * Counts, on the device, the log-decay values that the chunkwise entry points
 * do not accept; those calls do not check their decays (a check would cost a
 * pass over the tensor and a synchronization in every call), and such values
 * give wrong results without an error.  In the chunkwise forms the in-chunk
 * decay products are exponentials of differences of cumulative log decays
 * ("Parallel scan", section "The chunkwise algorithm"; "Lightning
 * Attention-2", Eq. 10): one NaN or +inf spoils every later token of its
 * chunk and state.
 *   log_decay : n fp32 values (device), any layout.
 *   counts    : 4 uint32 (device, 4-byte aligned), overwritten with the
 *               numbers of NaN, +inf, finite > 0, and -inf values, in that
 *               order (each wraps past 2^32 - 1).
 * Scalar decays (cla_chunk_*) need counts[0] = counts[1] = 0 (-inf is an
 * exact reset, finite l > 0 a growth factor, both computed exactly).  One
 * decay per key dimension (cla_gla_*) needs all four 0: finite l <= 0, since
 * its 16-token block factors exp(c) and exp(-c) stay bounded only for decays
 * at most 1, and it has no reset.  Asynchronous like every call: counts are
 * valid once the stream reaches this point.  Errors: n < 0 ->
 * CLA_ERR_BAD_SHAPE; counts NULL, or log_decay NULL with n > 0 ->
 * CLA_ERR_NULL_ARG; counts misaligned -> CLA_ERR_UNSUPPORTED; counts inside
 * log_decay -> CLA_ERR_ALIAS.
 */
int cla_check_log_decay(const float *log_decay, int64_t n, uint32_t *counts,
                        cla_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Diagonal state                                                            */
/* ------------------------------------------------------------------------ */

/*
 * Workspace bytes that cla_scan_fwd / cla_scan_bwd need for this shape (may
 * be 0).  When the batch and channel count alone cannot fill the GPU, the
 * time axis is split into segments whose composed pairs (A, beta) are kept
 * in the workspace ("Parallel scan", section "Splitting one sequence across
 * devices": an exclusive scan of per-piece pairs, then each piece resumes
 * from its incoming state).  Returns 0 for invalid shapes.
 */
size_t cla_scan_workspace_bytes(int64_t B, int64_t T, int64_t D);

/*
 * Forward scan.  "Parallel scan", sections "The scan for one number of
 * state" (recurrence, h_0 = 0 unless given) and "Scans over vector and matrix
 * states" (a nonzero h_0 is folded into the first step).
 *   a, b : [B, T, D] fp32 inputs (decays and inputs; a may be 0 or 1).
 *   h0   : [B, D] fp32 initial state, or NULL for zeros.
 *   h    : [B, T, D] fp32 output, h[b, t, d] = state after step t.
 *   hT   : [B, D] fp32 final state, or NULL to skip.
 */
int cla_scan_fwd(const float *a, const float *b, const float *h0, float *h,
                 float *hT, int64_t B, int64_t T, int64_t D, void *workspace,
                 size_t workspace_bytes, cla_stream_t stream);

/*
 * cla_scan_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument, and no allocation of any kind.  When the time axis
 * is split into segments, their composed pairs go to a fixed device array of
 * CLA_SCAN_NOALLOC_SCRATCH_BYTES that the library holds once per GPU until
 * the process ends; every shape cla_scan_workspace_bytes accepts needs at
 * most that much (a larger need returns CLA_ERR_WORKSPACE).  Arguments,
 * results and every other check are those of cla_scan_fwd.
 *   - The array is looked up (hipGetSymbolAddress) on the first call on each
 *     device, with that device current; `stream` must belong to the current
 *     device (CLA_ERR_UNSUPPORTED otherwise).
 *   - Each call writes every entry it reads before reading it, so nothing is
 *     cleared between calls.  All calls on one GPU share the array: calls
 *     that may run at the same time on one GPU (different streams, or
 *     threads) race and must be ordered by the caller.
 */
#define CLA_SCAN_NOALLOC_SCRATCH_BYTES 262144
int cla_scan_fwd_noalloc(const float *a, const float *b, const float *h0, float *h,
                         float *hT, int64_t B, int64_t T, int64_t D, cla_stream_t stream);

/*
 * Backward of cla_scan_fwd.  "Parallel scan", section "The backward pass is a
 * scan in reverse": the adjoint hbar_t = dL/dh_t satisfies
 *   hbar_T = dh_T + dhT,  hbar_t = dh_t + a_{t+1} hbar_{t+1},
 * and db_t = hbar_t, da_t = hbar_t h_{t-1} (h_0 at t = 1), dh0 = a_1 hbar_1.
 *   a    : [B, T, D] fp32, the forward decays.
 *   h    : [B, T, D] fp32, the forward output (supplies h_{t-1}).
 *   h0   : [B, D] fp32 forward initial state, or NULL for zeros.
 *   dh   : [B, T, D] fp32 gradient arriving at h.
 *   dhT  : [B, D] fp32 gradient arriving at the final state, or NULL.
 *   da, db : [B, T, D] fp32 outputs.
 *   dh0  : [B, D] fp32 output, or NULL to skip.
 */
int cla_scan_bwd(const float *a, const float *h, const float *h0,
                 const float *dh, const float *dhT, float *da, float *db,
                 float *dh0, int64_t B, int64_t T, int64_t D, void *workspace,
                 size_t workspace_bytes, cla_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Matrix state, chunkwise (declared here, defined in the chunk kernels)     */
/* ------------------------------------------------------------------------ */

/*
 * Workspace bytes for cla_chunk_fwd (backward = 0) or cla_chunk_bwd
 * (backward = 1) at this shape.  Returns 0 for an invalid shape.
 */
size_t cla_chunk_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t DK,
                                 int64_t DV, int64_t chunk, int backward);

/*
 * Chunkwise forward.  "Parallel scan", section "The chunkwise algorithm":
 * chunks of `chunk` tokens (the last may be shorter); inside a chunk the
 * decay-masked product (Q K^T (.) L) V, between chunks the carried state,
 *   O_[j] = (Q_[j] K_[j]^T (.) L) V_[j] + diag(lambda) Q_[j] S_[j-1],
 *   S_[j] = a_{chunk total} S_[j-1] + K_[j]^T diag(gamma) V_[j],
 * with the decays built from in-chunk cumulative log sums (section "Long
 * products without underflow").  Lightning Attention-2 Alg. 1 is the case of
 * a constant decay.
 *   q, k      : [B, H, T, DK] bf16.     v : [B, H, T, DV] bf16.
 *   log_decay : [B, H, T] fp32, l_t = log a_t: finite, or -inf for a_t = 0,
 *               an exact reset (the state is cleared before step t's write;
 *               the in-chunk decays are formed from finite partial sums and
 *               a count of resets, the additions-only segment sums of
 *               "Parallel scan", section "Long products without underflow").
 *               NaN and +inf are not allowed (not checked here;
 *               cla_check_log_decay counts them).
 *   S0        : [B, H, DK, DV] fp32 initial state, or NULL for zeros.
 *   o         : [B, H, T, DV] bf16 output.
 *   ST        : [B, H, DK, DV] fp32 final state, or NULL to skip.
 *   DK, DV in {64, 128}; chunk must be 64; the bf16 tensors must be
 *   16-byte aligned; T at most 67,107,840 (65535 segments of 16 chunks) and
 *   B*H below 2^31 (CLA_ERR_UNSUPPORTED otherwise).
 */
int cla_chunk_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const float *log_decay, const float *S0, uint16_t *o,
                  float *ST, int64_t B, int64_t H, int64_t T, int64_t DK,
                  int64_t DV, int64_t chunk, void *workspace,
                  size_t workspace_bytes, cla_stream_t stream);

/*
 * Chunkwise backward.  "Parallel scan", section "The backward pass of linear
 * attention" (adjoint state, the four gradients, the closed-form decay
 * gradient that needs no stored states) and Lightning Attention-2 Eq. 11-20,
 * Alg. 2 (dQ in forward chunk order, dK and dV in reverse chunk order).
 *   q, k, v, log_decay, S0 : as in cla_chunk_fwd.
 *   dO        : [B, H, T, DV] bf16 gradient arriving at o.
 *   dST       : [B, H, DK, DV] fp32 gradient arriving at S_T, or NULL.
 *   dq, dk    : [B, H, T, DK] bf16 outputs.   dv : [B, H, T, DV] bf16 output.
 *   dlog_decay: [B, H, T] fp32 output, dL/dl_t.
 *   dS0       : [B, H, DK, DV] fp32 output, or NULL to skip.
 */
int cla_chunk_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const float *log_decay, const float *S0, const uint16_t *dO,
                  const float *dST, uint16_t *dq, uint16_t *dk, uint16_t *dv,
                  float *dlog_decay, float *dS0, int64_t B, int64_t H,
                  int64_t T, int64_t DK, int64_t DV, int64_t chunk,
                  void *workspace, size_t workspace_bytes,
                  cla_stream_t stream);

/*
 * Training variant: the forward also saves the fp32 states the backward's
 * segments start from, and the backward starts from them instead of
 * recomputing them with an extra pass over K and V.  The state at a chunk
 * boundary is the carried S_[j] of "Parallel scan", section "The chunkwise
 * algorithm" (the forward already holds it); the backward's use of it follows
 * Lightning Attention-2 Alg. 2, whose dQ traversal runs forward from S_[j-1].
 * The outputs equal those of cla_chunk_fwd / cla_chunk_bwd up to rounding
 * order.
 *
 * cla_chunk_saved_bytes: bytes of the saved states at this shape (0 when the
 * backward does not split sequences, or for an invalid shape).  The buffer
 * holds, for each of the backward's segment boundaries p = 1 .. P-1 and each
 * (b, h), S [DK, DV] fp32 after chunk p * (segment length) - 1; its layout is
 * private to the library (pass it from cla_chunk_fwd_saved to
 * cla_chunk_bwd_saved unchanged, same shape).
 * saved: device buffer of at least cla_chunk_saved_bytes bytes (may be NULL
 * when that is 0), owned by the caller; written by cla_chunk_fwd_saved, read
 * by cla_chunk_bwd_saved.  Too small or NULL when needed -> CLA_ERR_WORKSPACE;
 * overlapping another argument -> CLA_ERR_ALIAS.  Every other argument and
 * check is that of cla_chunk_fwd / cla_chunk_bwd.
 */
size_t cla_chunk_saved_bytes(int64_t B, int64_t H, int64_t T, int64_t DK,
                             int64_t DV, int64_t chunk);

int cla_chunk_fwd_saved(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const float *log_decay, const float *S0, uint16_t *o,
                        float *ST, float *saved, size_t saved_bytes, int64_t B,
                        int64_t H, int64_t T, int64_t DK, int64_t DV,
                        int64_t chunk, void *workspace, size_t workspace_bytes,
                        cla_stream_t stream);

int cla_chunk_bwd_saved(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const float *log_decay, const float *S0,
                        const uint16_t *dO, const float *dST,
                        const float *saved, size_t saved_bytes, uint16_t *dq,
                        uint16_t *dk, uint16_t *dv, float *dlog_decay,
                        float *dS0, int64_t B, int64_t H, int64_t T,
                        int64_t DK, int64_t DV, int64_t chunk, void *workspace,
                        size_t workspace_bytes, cla_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing (benchmark instrumentation)                                 */
/* ------------------------------------------------------------------------ */

/*
 * enable != 0: from now on every kernel the library launches is bracketed by
 * two HIP events on its stream (a few microseconds of overhead per launch).
 * enable == 0: stop recording.  Returns CLA_OK.
 */
int cla_timing_enable(int enable);

/*
 * Waits for every recorded launch, then reports per kernel name the total
 * milliseconds and the number of launches since the last read, and clears the
 * records.  names[k] point to static strings.  Fills at most `max` entries
 * (any array may be NULL) and returns the number of distinct kernels, or
 * -CLA_ERR_HIP if an event query failed.
 */
int cla_timing_read(const char **names, double *total_ms, int64_t *counts, int max);

/*
 * One decay per key dimension (gated linear attention).  "Parallel scan",
 * sections "Scans over vector and matrix states" (the diagonal transition,
 * one decay per state entry) and "The chunkwise algorithm" (the GLA form
 * S_t = G_t (.) S_{t-1} + k_t^T v_t): row d of the state decays by
 * a_t[d] = exp(l_t[d]),
 *   S_t = diag(a_t) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t.
 *   q, k      : [B, H, T, DK] bf16;  v, o : [B, H, T, DV] bf16.
 *   log_decay : [B, H, T, DK] fp32, finite and <= 0 (decays in (0, 1]; not
 *               checked here: cla_check_log_decay counts the values outside
 *               that range), 16-byte aligned.
 *   S0, ST    : [B, H, DK, DV] fp32 (S0 NULL = zeros; ST NULL = not written).
 *   DK, DV in {64, 128}; chunk must be 64; the bf16 tensors and log_decay
 *   must be 16-byte aligned (CLA_ERR_UNSUPPORTED otherwise).
 * Inside a chunk the cumulative logs are summed over the chunk's own steps
 * ("Long products without underflow"); the in-chunk products are formed
 * from factors that never exceed 1, with an exact elementwise path for any
 * 16-step block whose decay falls below exp(-60) in some dimension.
 * When B*H alone gives fewer than 512 workgroups, each sequence is cut into
 * segments of whole 16-chunk blocks that run on separate workgroups: a state
 * pass gives each segment's local state and total decay, a scan over the
 * segments the state each one starts from ("Splitting one sequence across
 * devices", applied inside one GPU).  The forward's workspace
 * (cla_gla_workspace_bytes(..., backward = 0), 16-byte aligned) holds those
 * states; it is 0 bytes, and workspace may be NULL, when the sequence is not
 * split.
 */
size_t cla_gla_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t DK,
                               int64_t DV, int64_t chunk, int backward);

int cla_gla_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                const float *log_decay, const float *S0, uint16_t *o, float *ST,
                int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV,
                int64_t chunk, void *workspace, size_t workspace_bytes,
                cla_stream_t stream);

/*
 * Backward of cla_gla_fwd.  "Parallel scan", section "The backward pass of
 * linear attention", with the diagonal decay: the adjoint state decays by row,
 * and the decay gradient is the closed form for a vector of decays per step
 * (Yang et al. 2023, Section 4.3, as the page cites it), per key dimension:
 *   dl_u[d] = sum_{t >= u} q_t[d] dq_t[d] - sum_{s >= u} k_s[d] dk_s[d]
 *             (+ <S_T[d, :], dS_T[d, :]> when dS_T is given).
 * It is evaluated in segments of 16 chunks, each started from the boundary
 * term <S[d, :], G[d, :]> of the states at the segment's end (S in fp32, G as
 * the dk product rounds it), and both sums take their in-chunk terms from the
 * same rounded block products, so paths that do not cross step u cancel to
 * fp32 accuracy.
 *   q, k, v, log_decay, S0 : as in cla_gla_fwd.
 *   dO        : [B, H, T, DV] bf16 gradient at o.
 *   dST       : [B, H, DK, DV] fp32 gradient at S_T, or NULL.
 *   dq, dk    : [B, H, T, DK] bf16;  dv : [B, H, T, DV] bf16.
 *   dlog_decay: [B, H, T, DK] fp32, 16-byte aligned.
 *   dS0       : [B, H, DK, DV] fp32, or NULL (not written).
 *   workspace : cla_gla_workspace_bytes(..., backward = 1) bytes, 16-byte
 *               aligned (B*H*T*DK fp32 products q dq, one fp32 state per
 *               block of 16 chunks per sequence-head, and, when the sequence
 *               is split into segments as in the forward, each segment's
 *               starting state, local adjoint state and total decay).
 * With the sequence split, the backward runs the forward's state pass and
 * scan, its dQ pass per segment (also summing each segment's local adjoint
 * state), a reverse scan of the adjoint state over the segments, and its
 * dK/dV pass per segment.
 */
int cla_gla_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                const float *log_decay, const float *S0, const uint16_t *dO,
                const float *dST, uint16_t *dq, uint16_t *dk, uint16_t *dv,
                float *dlog_decay, float *dS0, int64_t B, int64_t H, int64_t T,
                int64_t DK, int64_t DV, int64_t chunk, void *workspace,
                size_t workspace_bytes, cla_stream_t stream);

/*
 * Training path that keeps the forward's segment start states for the
 * backward (the same decomposition as above: "Parallel scan", section
 * "Splitting one sequence across devices", with a decay per key dimension).
 * When a sequence is split into P > 1 segments, cla_gla_fwd_saved writes the
 * state each segment p = 1 .. P-1 starts from (the state pass and scan the
 * forward runs anyway) into `saved`, and cla_gla_bwd_saved starts the dQ
 * pass's segments from them instead of running that state pass again.
 * Results are bit-identical to cla_gla_fwd / cla_gla_bwd.
 * cla_gla_saved_bytes: bytes of the saved states at this shape (0 when the
 * sequence is not split, or for an invalid shape); layout [P-1, B*H, DK, DV]
 * fp32, private to the library (pass it from cla_gla_fwd_saved to
 * cla_gla_bwd_saved unchanged, same shape and inputs).
 * saved: device buffer of at least cla_gla_saved_bytes bytes (may be NULL when
 * that is 0), 16-byte aligned, owned by the caller.  Too small, misaligned or
 * NULL when needed -> CLA_ERR_WORKSPACE; overlapping another argument ->
 * CLA_ERR_ALIAS.  Every other argument and check is that of cla_gla_fwd /
 * cla_gla_bwd.
 */
size_t cla_gla_saved_bytes(int64_t B, int64_t H, int64_t T, int64_t DK,
                           int64_t DV, int64_t chunk);

int cla_gla_fwd_saved(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const float *log_decay, const float *S0, uint16_t *o,
                      float *ST, float *saved, size_t saved_bytes, int64_t B,
                      int64_t H, int64_t T, int64_t DK, int64_t DV,
                      int64_t chunk, void *workspace, size_t workspace_bytes,
                      cla_stream_t stream);

int cla_gla_bwd_saved(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const float *log_decay, const float *S0,
                      const uint16_t *dO, const float *dST, const float *saved,
                      size_t saved_bytes, uint16_t *dq, uint16_t *dk,
                      uint16_t *dv, float *dlog_decay, float *dS0, int64_t B,
                      int64_t H, int64_t T, int64_t DK, int64_t DV,
                      int64_t chunk, void *workspace, size_t workspace_bytes,
                      cla_stream_t stream);

/* ------------------------------------------------------------------------
 * Selective scan with N state entries per channel (Mamba-1's recurrence).
 * "Parallel scan", sections "Scans over vector and matrix states" (each
 * channel keeps N state numbers with their own decays; the input is written
 * into the state) and "What limits a recurrent layer" (the decay
 * exp(delta_{t,d} A_{d,n}) and the fused kernel that keeps the state on chip
 * and contracts it with C):
 *   h_t[d,n] = exp(delta_t[d] A[d,n]) h_{t-1}[d,n] + delta_t[d] B_t[n] x_t[d]
 *   y_t[d]   = sum_n C_t[n] h_t[d,n],   t = 1..T, h_0 = h0 (zeros if NULL).
 * All tensors fp32; x, delta, y, Bm, Cm, ckpt 16-byte aligned
 * (CLA_ERR_UNSUPPORTED otherwise):
 *   x, delta, y : [B, T, D]  (delta is the step size, used as given)
 *   A           : [D, N]
 *   Bm, Cm      : [B, T, N]  (one B_t and C_t per token, shared by channels)
 *   h0, hT      : [B, D, N]; h0 NULL means zeros, hT NULL is not written
 *   ckpt        : [B, ceil(T/16), D, N] (cla_sscan_ckpt_bytes bytes) or NULL:
 *                 the state before every 16th step, kept for the
 *                 backward, which recomputes the 16 states after each from
 *                 it (the page: Mamba recomputes its states in the backward).
 * Supported: N in {4, 8, 16}; D a multiple of 4 (at most 2^31 - 64);
 * B <= 65535 (CLA_ERR_UNSUPPORTED otherwise).  The [B, T, D, N] state tensor
 * is never written.
 * When B * ceil(D / 64) alone gives fewer than 512 workgroups, time is cut
 * into segments of whole 32-step tiles that run on separate workgroups: a
 * first pass gives each segment's local state and product of decays, a scan
 * over the segments the state each one starts from ("Splitting one sequence
 * across devices", per channel and entry).  The workspace
 * (cla_sscan_workspace_bytes(..., backward = 0, 0) bytes, 16-byte aligned)
 * holds those states; it is 0 bytes, and workspace may be NULL, when time is
 * not split.
 */
size_t cla_sscan_ckpt_bytes(int64_t B, int64_t T, int64_t D, int64_t N);

int cla_sscan_fwd(const float *x, const float *delta, const float *A, const float *Bm,
                  const float *Cm, const float *h0, float *y, float *hT, float *ckpt,
                  int64_t B, int64_t T, int64_t D, int64_t N, void *workspace,
                  size_t workspace_bytes, cla_stream_t stream);

/*
 * Backward of cla_sscan_fwd ("Parallel scan", section "The backward pass is
 * a scan in reverse", per (channel, entry), then the chain rule through
 * exp(delta A) and delta B x):  hbar_t = C_t dy_t + a_{t+1} hbar_{t+1}, with
 * dhT added at the last step.
 *   ckpt      : the forward's checkpoints, or NULL (this call then runs the
 *               forward's checkpoint pass itself, into the workspace).
 *   dy        : [B, T, D] gradient at y;  dhT : [B, D, N] or NULL.
 *   dx, ddelta: [B, T, D];  dA : [D, N] (summed over the batch);
 *   dB, dC    : [B, T, N] (summed over channels);  dh0 : [B, D, N] or NULL.
 *   workspace : cla_sscan_workspace_bytes(B, T, D, N, 1, ckpt != NULL) bytes,
 *               16-byte aligned (per-workgroup partial sums for dB and dC,
 *               dA per segment and sequence, when time is split each
 *               segment's own adjoint and product of decays, and the
 *               checkpoints and the forward's workspace when not given).
 * With time split as in the forward, a first pass runs each later segment
 * backwards from a zero adjoint (decays, C and dy only), a reverse scan gives
 * the adjoint each segment receives from the steps after it, and the main
 * pass runs per segment.  Sums run in a fixed order, so results are
 * bit-identical from run to run.
 */
size_t cla_sscan_workspace_bytes(int64_t B, int64_t T, int64_t D, int64_t N, int backward,
                                 int have_ckpt);

int cla_sscan_bwd(const float *x, const float *delta, const float *A, const float *Bm,
                  const float *Cm, const float *h0, const float *ckpt, const float *dy,
                  const float *dhT, float *dx, float *ddelta, float *dA, float *dB, float *dC,
                  float *dh0, int64_t B, int64_t T, int64_t D, int64_t N, void *workspace,
                  size_t workspace_bytes, cla_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CLA_H */
