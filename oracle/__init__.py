"""Reference oracle for paged split-KV decode attention (TEST INFRASTRUCTURE ONLY).

This package is a plain, slow, float64 CPU statement of what the decode path
computes.  It exists so that tests, the smoke check and the benchmark's
``cpu_baseline`` leg have something independent to compare the HIP kernels
with.  Nothing on the product path may import it: the library in
``paged_split_kv_pa_amd`` never routes through here and fails loudly when its
HIP extension is missing.

Sources (the pages are cited by title and section; no line numbers):

* project_6 commit 96f4baf ("Dockerfile" commit page), V2 plan, "Phase 1:
  Per-partition attention" and "Phase 2: Cross-partition reduction
  (log-sum-exp)" -- the algorithm: per (sequence, head, partition) attention
  producing a partial output, an exp-sum and a max logit, then a log-sum-exp
  merge over partitions.  The same page names the partition size (512) and
  the 100K-context partition count.
* project_6 optimizations/prefix_prefill_patch.py (commit fee8f1b), docstring
  section "_PARTITION_SIZE inconsistency" -- 512 vs 256 must agree between the
  two phases.
* project_6 commit a2a5dd8 ("computility-run.yaml" commit page), decode-path
  summary -- the V1/V2 context-length thresholds.
* project_6_baseline5 GROUND_TRUTH_STATUS_v2.md, section "路径 3" -- the
  prefix-caching cache copy kernel (``cache_ops``).
* project_6 optimizations/prefix_prefill_patch.py (commit fee8f1b) docstring and
  the "Dockerfile" commit page, "What CAN be optimized" -- the prefix-prefill
  attention kernel (``prefill``).

Modules:

* ``storage``   -- exact upcast of stored fp32 / fp16 / bf16 values to float64.
* ``attention`` -- the unpartitioned definition (``decode_attention``), the
  literal two-phase statement (``partitioned_decode``), the partial-statistics
  merge (``merge_partials``) and the partition arithmetic.
* ``cache_ops`` -- the KV block copy of prefix caching (``copy_blocks``).
* ``prefill`` -- paged prefix-prefill attention (``prefill_attention``) and its
  FLOP count.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, brute force and invariants (see each function's docstring).
"""

from .storage import upcast, STORAGE_DTYPES  # noqa: F401
from .attention import (  # noqa: F401
    decode_attention,
    partition_partials,
    combine_partitions,
    partitioned_decode,
    merge_partials,
    num_partitions,
    gather_sequence,
)
from .cache_ops import copy_blocks  # noqa: F401
from .prefill import prefill_attention, prefill_rows, prefill_flops  # noqa: F401
