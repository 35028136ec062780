"""Float64 CPU oracle for the gated linear recurrence -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct statement of what the GPU
library computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``chunkwise_linear_attention_amd``) never imports, links or calls anything
here, and nothing here imports the product path: the two share no code.

Sources (the pages the method is stated on):

* ZTF  -- "Parallel scan" section of Zero to Frontier
  (zerotofrontier.app/ssm/parallel-scan).
* LA2  -- summary page of "Lightning Attention-2: A Free Lunch for Handling
  Unlimited Sequence Lengths in Large Language Models" (paper-graph-ui).
* WIKI -- "Parallel Scan" entry of aiwiki.thehackersbrain.dev.

Modules:

* ``oracle.scan``  -- diagonal (per-channel) recurrence h_t = a_t h_{t-1} + b_t:
  pair algebra, sequential loop, Hillis-Steele and Blelloch scans with
  combine counters, and the reverse-time backward.
* ``oracle.attn``  -- matrix-state recurrence S_t = a_t S_{t-1} + k_t v_t^T,
  o_t = S_t^T q_t: per-token loop, the T x T matrix mode, the chunkwise
  algorithm in the pages' order, and the backward by the adjoint recurrence.
* ``oracle.gla``   -- the same with one decay per key dimension (gated linear
  attention), S_t = diag(a_t) S_{t-1} + k_t v_t^T: loop, matrix mode,
  chunkwise form, adjoint backward and the closed-form vector decay gradient.
* ``oracle.sscan`` -- the selective scan with N state entries per channel
  (Mamba-1's recurrence): decay exp(delta A), input delta B x, output C.h;
  loop, path-sum form, and the reverse-time backward with the chain rule.
* ``oracle.cref``  -- ctypes wrapper over ``oracle/ref.c``, the same loops in
  C (float64, OpenMP over independent channels / heads) for full-size samples
  and for the CPU baseline timing.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values printed on the pages, closed forms, brute force on tiny inputs
or finite differences; none is "parity unpinned".
"""

from . import scan, attn, gla, sscan  # noqa: F401

__all__ = ["scan", "attn", "gla", "sscan"]
