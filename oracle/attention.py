"""Float64 oracle for paged decode attention (test infrastructure only).

What is computed (project_6 commit 96f4baf, "Dockerfile" commit page, V2 plan):
for every (sequence, query head) the decode step attends the single query
vector to all cached tokens of that sequence -- QK^T, a softmax over the
tokens, and the softmax-weighted sum of the V rows.  V2 ("Phase 1") does this
per partition of PARTITION_SIZE tokens and keeps, per partition, the
normalised partial output, the sum of exponentials and the maximum logit;
"Phase 2" merges the partitions with log-sum-exp rescaling.

Readings where the pages are silent (each one is also listed in the design
notes of the repository):

* KV cache layout is ``[num_blocks, num_kv_heads, block_size, head_dim]`` for
  both K and V; token ``t`` of sequence ``b`` lives in physical block
  ``block_tables[b, t // block_size]`` at slot ``t % block_size``.
* Query head ``h`` reads KV head ``h // G`` with ``G = Hq / Hkv`` (grouped-query
  attention: consecutive query heads share one KV head).
* ``scale`` multiplies q.k before the max and the exponential; the stored max
  logit is the scaled logit.
* The partial output of a partition is normalised by that partition's
  exp-sum; ``total_sum`` in Phase 2 is the sum of the rescaled exp-sums.
* A partition is the token range ``[p*P, min((p+1)*P, n))``; the number of
  partitions of a sequence is ``ceil(n / P)`` (196 at n = 100000, P = 512:
  195 full partitions and one of 160 tokens).
* A sequence with no cached tokens has output 0.
* No mask beyond the context length: every one of the ``n`` tokens attends.

Everything is float64.  Inputs arrive in storage form (see ``storage``) and
are upcast exactly; ``scale`` is taken as the binary32 value a C caller
passes.
"""

import math

import numpy as np

from .storage import upcast


def num_partitions(n, partition_size):
    """Number of partitions covering ``n`` tokens: ceil(n / P) (0 for n = 0).

    Source: project_6 commit 96f4baf page, V2 plan -- the context is split into
    PARTITION_SIZE-token chunks processed in parallel.
    """
    if partition_size <= 0:
        raise ValueError("partition_size must be positive")
    if n < 0:
        raise ValueError("context length must be non-negative")
    return (int(n) + int(partition_size) - 1) // int(partition_size)


def gather_sequence(cache, block_tables, b, n):
    """Return the first ``n`` cached rows of sequence ``b``: shape [n, Hkv, D].

    Token ``t`` is read from physical block ``block_tables[b, t // bs]`` at slot
    ``t % bs`` of a ``[NB, Hkv, bs, D]`` cache.  The result keeps the storage
    dtype (no arithmetic happens here).
    """
    bs = cache.shape[2]
    t = np.arange(n)
    phys = np.asarray(block_tables)[b, t // bs].astype(np.int64)
    if n and (phys.min() < 0 or phys.max() >= cache.shape[0]):
        raise IndexError("block table entry outside the KV pool")
    slot = t % bs
    return cache[phys, :, slot, :]


def _check_shapes(q, k_cache, v_cache, block_tables, context_lens):
    S, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if Dk != D:
        raise ValueError("head_dim of q and the cache differ")
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    if np.any(np.asarray(context_lens) > block_tables.shape[1] * bs):
        raise ValueError("context length exceeds the block-table capacity")
    return S, Hq, D, Hkv, bs, Hq // Hkv


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale, dtype):
    """Plain, unpartitioned decode attention in float64.

    out[b, h, :] = sum_t softmax_t(scale * <q[b,h], K_t>) * V_t over the
    ``context_lens[b]`` tokens of sequence ``b``, with K_t / V_t gathered
    through the block table from KV head ``h // G``.  The softmax is evaluated
    as exp(l_t - max_t l_t) / sum_t exp(l_t - max_t l_t), which is the same
    real number as the textbook form.

    Returns float64 ``[S, Hq, D]``.
    """
    S, Hq, D, Hkv, bs, G = _check_shapes(q, k_cache, v_cache, block_tables, context_lens)
    s = float(np.float32(scale))
    q64 = upcast(q, dtype)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for b in range(S):
        n = int(context_lens[b])
        if n == 0:
            continue
        K = upcast(gather_sequence(k_cache, block_tables, b, n), dtype)  # [n, Hkv, D]
        V = upcast(gather_sequence(v_cache, block_tables, b, n), dtype)
        for g in range(Hkv):
            heads = q64[b, g * G:(g + 1) * G, :]            # [G, D]
            logits = s * (K[:, g, :] @ heads.T)              # [n, G]
            w = np.exp(logits - logits.max(axis=0, keepdims=True))
            out[b, g * G:(g + 1) * G, :] = (w.T @ V[:, g, :]) / w.sum(axis=0)[:, None]
    return out


def partition_partials(qh, K, V, scale):
    """Phase-1 statistics of one (sequence, head, partition).

    ``qh`` [D], ``K`` / ``V`` [m, D] float64 rows of the partition's tokens.
    Returns ``(max_logit, exp_sum, partial_out)`` with
    max_logit = max_t l_t, exp_sum = sum_t exp(l_t - max_logit) and
    partial_out = sum_t exp(l_t - max_logit) V_t / exp_sum, l_t = scale <qh, K_t>.
    Source: project_6 commit 96f4baf page, "Phase 1" -- QK^T, softmax and
    weighted V sum per partition, storing tmp_output / exp_sums / max_logits.
    """
    logits = scale * (K @ qh)
    m = logits.max()
    e = np.exp(logits - m)
    ssum = e.sum()
    return m, ssum, (e @ V) / ssum


def combine_partitions(max_logits, exp_sums, partial_outs):
    """Phase-2 merge of one (sequence, head), step by step as the page lists it.

    global_max = max_p max_logits[p]; rescale_p = exp(max_logits[p] - global_max)
    * exp_sums[p]; total_sum = sum_p rescale_p; output = sum_p (rescale_p /
    total_sum) * partial_outs[p].  Source: project_6 commit 96f4baf page,
    "Phase 2: Cross-partition reduction (log-sum-exp)".
    """
    m = np.asarray(max_logits, dtype=np.float64)
    s = np.asarray(exp_sums, dtype=np.float64)
    o = np.asarray(partial_outs, dtype=np.float64)
    global_max = m.max()
    rescale = np.exp(m - global_max) * s
    total_sum = rescale.sum()
    return (rescale / total_sum) @ o


def partitioned_decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
                       partition_size, max_partitions=None):
    """The two-phase V2 statement in float64, without any blocking or fusion.

    Returns ``(out, partials)`` where ``out`` is float64 [S, Hq, D] and
    ``partials`` holds float64 arrays ``tmp_out`` [S, Hq, Pmax, D],
    ``exp_sums`` and ``max_logits`` [S, Hq, Pmax] (NaN where a partition does
    not exist for that sequence).  ``Pmax`` defaults to the largest partition
    count in the batch.
    """
    S, Hq, D, Hkv, bs, G = _check_shapes(q, k_cache, v_cache, block_tables, context_lens)
    P = int(partition_size)
    s = float(np.float32(scale))
    counts = [num_partitions(int(n), P) for n in context_lens]
    Pmax = max(counts + [1]) if max_partitions is None else int(max_partitions)
    if Pmax < max(counts + [0]):
        raise ValueError("max_partitions smaller than the partition count of a sequence")
    q64 = upcast(q, dtype)
    tmp_out = np.full((S, Hq, Pmax, D), np.nan)
    exp_sums = np.full((S, Hq, Pmax), np.nan)
    max_logits = np.full((S, Hq, Pmax), np.nan)
    out = np.zeros((S, Hq, D))
    for b in range(S):
        n = int(context_lens[b])
        if n == 0:
            continue
        K = upcast(gather_sequence(k_cache, block_tables, b, n), dtype)
        V = upcast(gather_sequence(v_cache, block_tables, b, n), dtype)
        for h in range(Hq):
            g = h // G
            for p in range(counts[b]):
                lo, hi = p * P, min((p + 1) * P, n)
                m, ssum, o = partition_partials(q64[b, h], K[lo:hi, g, :], V[lo:hi, g, :], s)
                max_logits[b, h, p], exp_sums[b, h, p] = m, ssum
                tmp_out[b, h, p] = o
            out[b, h] = combine_partitions(max_logits[b, h, :counts[b]],
                                           exp_sums[b, h, :counts[b]],
                                           tmp_out[b, h, :counts[b]])
    return out, {"tmp_out": tmp_out, "exp_sums": exp_sums, "max_logits": max_logits}


def merge_partials(a, b):
    """Associative merge of two partial results over disjoint token sets.

    ``a`` and ``b`` are ``(max_logit, exp_sum, normalised_out)``; the identity is
    ``(-inf, 0, 0)``.  m = max(m1, m2), a_i = exp(m_i - m) s_i, result =
    (m, a_1 + a_2, (a_1 o_1 + a_2 o_2) / (a_1 + a_2)).  The project_6 commit
    96f4baf page (V2 plan) likens Phase 2 to merging softmax statistics computed
    on separate segments; folding this merge over the partitions gives Phase 2.
    """
    m1, s1, o1 = a
    m2, s2, o2 = b
    if m1 == -math.inf:
        return (m2, s2, np.array(o2, dtype=np.float64))
    if m2 == -math.inf:
        return (m1, s1, np.array(o1, dtype=np.float64))
    m = max(m1, m2)
    a1 = math.exp(m1 - m) * s1
    a2 = math.exp(m2 - m) * s2
    return (m, a1 + a2, (a1 * np.asarray(o1, dtype=np.float64) +
                         a2 * np.asarray(o2, dtype=np.float64)) / (a1 + a2))
