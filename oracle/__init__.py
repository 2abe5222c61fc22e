"""fp64 CPU oracle for one zero-bubble pipeline stage.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only the test suite, the smoke check and
the benchmark's CPU-baseline leg use it.  It shares no code with the HIP path;
the only common module is ``synthetic_inputs``, which draws the seeded inputs
and holds none of the method's arithmetic.

* ``oracle.stage``     -- forward (F), input gradient (B), weight gradient (W)
                          and the fused (unsplit) backward of a stage, in fp64.
* ``oracle.optim``     -- staged reduce of the gradient state, optimistic AdamW
                          step, post-update validation and exact rollback.
* ``oracle.heuristic`` -- the automatic (ZB-1p / ZB-2p) scheduler.
* ``oracle.vshape``    -- the V placement and its list-scheduled order (ZB-V).
* ``oracle.schedules`` -- per-stage pass orders (GPipe, 1F1B, ZB-H1, ZB-H2,
                          interleaved), the list-scheduling simulator, bubble
                          and memory accounting, the order validator and the
                          timed-event inspector.

Every function cites the page passage it follows.  Pages:
  [ZB]  "Zero Bubble Pipeline Parallelism" (structured summary of arXiv 2401.10241)
  [AUD] "Zero-Bubble Pipeline Parallelism, Proven" (practitioner's audit)
  [TUT] "Pipeline Schedules: GPipe, 1F1B and Zero Bubble" (tutorial)

Parity status: every function here is pinned by a CPU test against values
the pages print, closed forms, brute force or invariants, except where a
docstring says "parity unpinned".
"""
