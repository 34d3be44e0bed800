"""Float64 oracle for paged prefix-prefill attention (TEST INFRASTRUCTURE ONLY).

Source: project_6 optimizations/prefix_prefill_patch.py (commit fee8f1b), the
docstring's analysis of the prefix_prefill Triton kernel: a Flash-Attention style
kernel over a grid of (batch, heads, ceil(seq_len / BLOCK_M)) query tiles, BLOCK_M
query positions per tile and K/V tiles of BLOCK_N tokens, for fp16/bf16,
head_dim 128 (256 rare) and grouped-query attention; and the "Dockerfile" commit
page (project_6 commit 96f4baf), "What CAN be optimized", item 1 (the same kernel)
and item 2 (prefill chunks of max-num-batched-tokens tokens).

The pages give the kernel's tiling, not its formula.  The plainest reading that
the tiling supports, and the one this oracle states: a prefill step appends a
chunk of L new tokens to a sequence whose first c tokens are already in the paged
KV cache (the prefix).  New token i (absolute position c + i) attends, with the
same softmax attention as decode, to every prefix token and to new tokens 0..i
(causal).  The new tokens' K and V arrive as packed tensors; the prefix is read
through the block table exactly as in decode.

Readings (also listed in the design notes):
* q, and the new tokens' k / v, are packed over the batch: [T, Hq, D] and
  [T, Hkv, D], sequence b owning rows query_start[b] .. query_start[b+1]-1;
* context_lens[b] = c_b is the prefix length (0: no prefix);
* query head h reads KV head h // G, as in decode; scale multiplies q.k;
* a query always sees at least its own key, so no row is empty.
"""
import numpy as np

from .attention import gather_sequence
from .storage import upcast


def prefill_rows(q_rows, k_all, v_all, first_pos, scale):
    """Causal softmax attention of L query rows of one head against keys 0..n-1.

    ``q_rows`` [L, D]; ``k_all`` / ``v_all`` [n, D] float64; query row i sits at
    absolute position ``first_pos + i`` and sees keys j <= first_pos + i.
    Returns float64 [L, D].
    """
    L = q_rows.shape[0]
    n = k_all.shape[0]
    logits = scale * (q_rows @ k_all.T)                       # [L, n]
    visible = np.arange(n)[None, :] <= (first_pos + np.arange(L))[:, None]
    logits = np.where(visible, logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)                                    # exp(-inf) = 0 off the mask
    return (e @ v_all) / e.sum(axis=1, keepdims=True)


def prefill_attention(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                      query_start, scale, dtype):
    """Output [T, Hq, D] float64 of a paged prefix-prefill step (see module docstring)."""
    T, Hq, D = q.shape
    Tk, Hkv, Dk = k_new.shape
    if Tk != T or Dk != D or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [T, Hkv, D] like q")
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if k_cache.shape[1] != Hkv or k_cache.shape[3] != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape does not match the new tokens")
    G = Hq // Hkv
    qs = np.asarray(query_start, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = ctx.shape[0]
    if qs.shape[0] != S + 1 or qs[0] != 0 or qs[-1] != T or np.any(np.diff(qs) < 0):
        raise ValueError("query_start must be [S+1], non-decreasing, from 0 to T")
    s = float(np.float32(scale))
    q64 = upcast(q, dtype)
    kn64 = upcast(k_new, dtype)
    vn64 = upcast(v_new, dtype)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for b in range(S):
        r0, r1 = int(qs[b]), int(qs[b + 1])
        if r1 == r0:
            continue
        c = int(ctx[b])
        kp = upcast(gather_sequence(k_cache, block_tables, b, c), dtype)   # [c, Hkv, D]
        vp = upcast(gather_sequence(v_cache, block_tables, b, c), dtype)
        k_all = np.concatenate([kp, kn64[r0:r1]], axis=0)                # [c + L, Hkv, D]
        v_all = np.concatenate([vp, vn64[r0:r1]], axis=0)
        for h in range(Hq):
            g = h // G
            out[r0:r1, h, :] = prefill_rows(q64[r0:r1, h, :], k_all[:, g, :], v_all[:, g, :],
                                            c, s)
    return out


def prefill_flops(context_lens, query_start, num_q_heads, head_dim):
    """Algorithmic FLOPs of a step: 2*D for q.k plus 2*D for p.v per visible
    (query row, key) pair, summed over heads: 4 * Hq * D * sum_b sum_i (c_b + i + 1)."""
    qs = np.asarray(query_start, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    pairs = 0
    for b in range(ctx.shape[0]):
        L = int(qs[b + 1] - qs[b])
        pairs += L * int(ctx[b]) + L * (L + 1) // 2
    return 4 * int(num_q_heads) * int(head_dim) * pairs
