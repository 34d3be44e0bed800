"""KV-cache block copy for prefix caching (TEST INFRASTRUCTURE ONLY).

Source: project_6_baseline5 GROUND_TRUTH_STATUS_v2.md, section "路径 3" (vllm
Python-layer configuration): prefix caching is enabled and its cache copy kernel
is named as not optimised.  The page names the kernel only; what it computes is
read here as the plain copy-on-write step of a paged cache: for every (src, dst)
pair of block ids, the dst block of the K pool and of the V pool becomes a copy
of the src block, in every head and slot.

Readings (the page is silent on them):
* the copy is bitwise (no dtype conversion);
* all sources are read before any destination is written (a call whose
  destinations are distinct and are not among its sources behaves the same
  under any order; other calls are outside the contract);
* a pair with an id outside [0, num_blocks) is skipped: nothing is written
  for it.
"""
import numpy as np


def copy_blocks(k_cache, v_cache, pairs):
    """Return copies of the K and V pools after the block copies of ``pairs``.

    ``k_cache`` / ``v_cache``: arrays [num_blocks, ...] (any trailing layout, any
    dtype; the copy is of whole blocks).  ``pairs``: int array [n, 2] of
    (src, dst) block ids.
    """
    k_cache = np.asarray(k_cache)
    v_cache = np.asarray(v_cache)
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    nb = k_cache.shape[0]
    ok = (pairs[:, 0] >= 0) & (pairs[:, 0] < nb) & (pairs[:, 1] >= 0) & (pairs[:, 1] < nb)
    src, dst = pairs[ok, 0], pairs[ok, 1]
    k_out, v_out = k_cache.copy(), v_cache.copy()
    k_out[dst] = k_cache[src]  # right-hand side gathered first: every read precedes the writes
    v_out[dst] = v_cache[src]
    return k_out, v_out
