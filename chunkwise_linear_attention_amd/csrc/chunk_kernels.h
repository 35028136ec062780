// Argument blocks and launchers of the chunkwise kernels, shared by the
// forward (chunk.hip) and backward (chunk_bwd.hip) translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cla {
namespace chunk {

struct FwdArgs {
  const uint16_t *q;       // [nh, T, DK]
  const uint16_t *k;       // [nh, T, DK]
  const uint16_t *v;       // [nh, T, DV]
  const float *l;          // [nh, T]
  const float *S0;         // [nh, DK, DV] (or [nh, DV, DK] if s0_trans); NULL = 0
  const float *Sin;        // [P-1, nh, DK, DV] state entering segments 1..P-1
  uint16_t *o;             // [nh, T, DV]
  float *ST;               // [nh, DK, DV] (or transposed if st_trans); NULL = skip
  float *Sloc;             // state-only pass: [P-1, nh, DK, DV]
  float *aloc;             // state-only pass: [P-1, nh] total decay of the segment
  const uint16_t *xdot;    // optional [nh, T, DV]: rdot[t] = sum_j xdot[t, j] o[t, j]
  float *rdot;             // [nh, T]
  float *saved;            // optional [nT/save_every - 1, nh, DK, DV]: the state after
                           // every save_every chunks (MODE 0)
  float *gloc;             // optional [P-1, nh, DV, DK] (segment p in slot p-1): the
                           // segment-local sum  sum_t A_t v_t x_t^T  over the
                           // segment's tokens, A_t = the decay from the segment
                           // start through t (needs xdot); in the dQ pass this is
                           // the dK/dV pass's local G state, stored as G
  float *galoc;            // with gloc: [P-1, nh] total decay of the segment
  float *Send;             // optional (dQ pass): [P-1, nh, DK, DV] this pass's own state
                           // at the end of segments 0..P-2, row-major in its orientation
  int64_t nh, T, seg_chunks, P, save_every;
  int s0_trans, st_trans;
  int slot_trans;          // segment slots (Sloc, Sin) hold this kernel's state transposed
  int sin_given;           // Sin is supplied: no segment-state pass, no segment scan
};

struct BwdArgs {
  const uint16_t *q, *k, *v, *dO;   // [nh, T, DK|DV]
  const float *l;                   // [nh, T]
  const float *dST;                 // [nh, DK, DV] or NULL
  const float *Gin;                 // [P-1, nh, DK, DV]: G at the end of segments 0..P-2
  uint16_t *dk, *dv;                // [nh, T, DK|DV]
  const float *r1;                  // [nh, T]  q . dq (from the dQ pass)
  float *dl;                        // [nh, T]  the decay gradient
  float *dS0;                       // [nh, DK, DV] or NULL
  float *Gloc;                      // [P-1, nh, DK, DV]: segment p's local G state in slot
                                    // p-1 (written by the dQ pass); the reverse segment
                                    // scan turns it into Gin
  float *aloc;                      // [P-1, nh]: total decay of segment p in slot p-1
  const float *Sseg;                // [P-1, nh, DV, DK]: S^T at the end of segments 0..P-2
                                    // as the dQ pass held it
  const float *STb;                 // [nh, DV, DK]: S_T^T (NULL when there is no dS_T)
  int64_t nh, T, seg_chunks, P;
};

// Forward-type pass (segment state pass, segment scan, main pass).
hipError_t fwd_dispatch(FwdArgs args, int DK, int DV, hipStream_t stream);

// Segment-local state gradients of segments 1..P-1 (args.k = q, args.v = dO)
// into args.Sloc / args.aloc slots 0..P-2, as the dQ pass's gloc / galoc.
hipError_t grad_state_dispatch(const FwdArgs &args, int DK, int DV, hipStream_t stream);

// Reverse dK/dV pass (reverse segment scan of Gloc, main pass).
hipError_t bwd_kv_dispatch(const BwdArgs &args, int DK, int DV, hipStream_t stream);

// Exclusive scan of per-segment pairs (alpha_p, S_p) held in slots, in place.
// Forward (reverse = 0): slot p becomes the state entering segment p + 1,
// starting from init.  Reverse (reverse = 1): slot p (holding segment p + 1's
// pair) becomes the state gradient at the end of segment p, starting from
// init at the end of the sequence.
hipError_t launch_segment_scan(float *slots, const float *aloc, const float *init,
                               int init_trans, int reverse, int64_t nh, int64_t P,
                               int DK, int DV, hipStream_t stream);

}  // namespace chunk
}  // namespace cla
