"""CPU oracle for block-sparse / top-k attention — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct fp64 (numpy) and pure-Python implementations of
what the GPU path computes.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the library and its
Python binding never do.  It shares no code with the HIP/C++ path.

Sources (web pages; cited by title and section):

* "db-SP: load balancing of sparse-attention head parallelism and sequence
  parallelism" (Zhihu repost on yjmstr.github.io) — scenario 2 defines a
  Q-block's work as its block-mask row sum and a KV-block's as its column sum;
  the LPT paragraph and its two bullets give the greedy, the [8,7,6,5,4]
  counter-example and the (4m-1)/(3m) bound.
* "Attention kernels and communication overlap under 6D parallelism" study
  notes (walkerchi.com) — section 2.1 (ring-attention pseudocode: the
  online-softmax state, the per-step partial and the merge), section 2.3
  (causal ring skipping, striped attention), section 7.1 (DSA: low-rank
  indexer, top-k, gather, softmax over the selected keys).

Modules:

* ``oracle.attention`` — masked dense attention, per-chunk partials, merge.
* ``oracle.plan``      — block popcounts, LPT / naive assignment, brute force,
  ring step table.
* ``oracle.topk``      — indexer scores, top-k selection, attention over a
  selected key set.

Every function here is pinned by ``tests/test_oracle_*.py`` against facts the
pages print or mathematics fixes; see those tests for the pin of each one.
"""
from . import attention, plan, topk  # noqa: F401
