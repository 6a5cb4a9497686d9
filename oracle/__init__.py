"""CPU oracle for CQS-streamed exact attention (test infrastructure, not product code).

Only the test suite under ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The HIP library never calls it and shares no code with it: the two meet only
through the seeded inputs of ``memory_bounded_streaming_amd.inputs`` (which holds
none of the method's arithmetic) and through the results the tests compare.

Sources (the pages that define the method):

* "Stream-CQSA: Exact Out-of-Memory Recovery for Attention", arXiv 2604.20819,
  abstract -- exact recovery of full attention by recomposing local statistics
  of independent subsequence tasks; comparison against a dense float64
  reference.
* "Stream-CQSA: Breaking the Billion-Token Barrier on a Single GPU" (wispaper
  explainer), sections "The 'CQS Divide': Attention as a Steiner System",
  "The Recursive Benefit" and "Implementation: From High-Level Logic to GPU
  Kernels" -- c = l(l-1)+1 chunks, c subsequences of l chunks, every chunk
  pair exactly once (S(2,l,c)), recursion, the CQS Mask, per-task softmax sums.
* Lattice summary page of arXiv:2604.20819 -- the recomposed output equals that of
  undivided attention.

Modules
-------
``attention``  plain two-pass softmax attention in float64 (the definition).
``plan``       reference CQS planner: difference set, subsequences, recursion,
               ownership mask, coverage table, canonical serialisation.
``recompose``  per-task float64 partials and their merge (the method's steps).
``backward``   gradients of attention (the definition) and their per-task sums.
``stream_bytes`` the bytes the streamed forward moves, counted task by task.
``tolerance``  the error metrics the parity tests apply.

Every function states which of the above it follows.  Readings taken where the
pages are silent are listed in the module that applies them.  Parity pins: all
functions here are pinned by ``tests/test_oracle_*.py`` (closed forms, special
cases, brute force, library routines); none is "parity unpinned".
"""
