"""Seeded synthetic decode workloads (shared by tests, the smoke check and the bench).

This module only *creates inputs*: it draws random values, rounds them to
the storage format and lays out a paged KV cache with a block table.  It
contains none of the attention arithmetic, so both the HIP path and the
float64 oracle can consume what it produces without sharing code.

The five named workloads follow the shapes of the decode problem as stated
for the split-KV scheme (batch 1 up to 256 sequences, contexts from 1 to
100000 tokens, GQA 4 and 8, head_dim 128 and 256, block_size 16, fp32 /
bf16 / fp16 KV).  The pages' own serving benchmark (100K max model length,
128-256 concurrent sequences of about 2K context; project_6 commit a2a5dd8
page, max-num-seqs discussion) is not available; these synthetic inputs
stand in for it.

Storage formats: ``"f32"`` float32, ``"f16"`` float16, ``"bf16"`` uint16 bit
patterns (upper half of binary32, rounded to nearest even).

Layouts:
* q                     [S, Hq, D]
* k_cache, v_cache      [NB, Hkv, 16, D]
* block_tables (int32)  [S, MB]; entries past a sequence's last block point at
  ``pad_block``, a pool block that no sequence uses.
* context_lens (int32)  [S]
"""

from dataclasses import dataclass, field
import math

import numpy as np

BLOCK_SIZE = 16


def round_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def to_storage(x, dtype):
    """Round float32 values to a storage format."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_float32(a, dtype):
    """Widen storage back to float32 (input construction only, e.g. outlier keys)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(a).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(a).astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


ELEMENT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass
class Workload:
    name: str
    dtype: str
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    scale: float
    partition_sizes: list
    pad_block: int
    seed: int
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return self.q.shape[0]

    @property
    def num_q_heads(self):
        return self.q.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def num_kv_heads(self):
        return self.k_cache.shape[1]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    @property
    def max_blocks_per_seq(self):
        return self.block_tables.shape[1]

    def used_blocks(self):
        """Physical block ids referenced by the valid part of every sequence."""
        ids = []
        for b, n in enumerate(self.context_lens):
            nb = -(-int(n) // BLOCK_SIZE)
            ids.extend(int(x) for x in self.block_tables[b, :nb])
        return ids


def make_workload(name, seed, *, context_lens, num_q_heads, num_kv_heads, head_dim, dtype,
                  sigma=1.0, scale=None, num_blocks=None, pool_factor=1.2,
                  max_blocks_per_seq=None, partition_sizes=(512,), outliers=None,
                  context_lens_fn=None):
    """Draw one seeded workload.

    Draw order from ``numpy.random.default_rng(seed)``: context lengths (only
    when ``context_lens_fn`` is given), q, the K pool, the V pool, the block
    permutation, then the outlier positions.  Values are N(0, sigma^2) drawn
    in float32 and rounded once to ``dtype``.

    ``outliers=(count, delta)`` raises the logit of ``count`` distinct token
    positions by ``delta`` for every query head of every KV head: for each KV
    head g the key of a chosen token gets the least-norm vector x with
    scale * Q_g x = delta (Q_g = that group's query rows), added before the
    key is rounded to ``dtype``.
    """
    rng = np.random.default_rng(seed)
    if context_lens_fn is not None:
        context_lens = context_lens_fn(rng)
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = len(ctx)
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    blocks_per_seq = [-(-int(n) // BLOCK_SIZE) for n in ctx]
    used = sum(blocks_per_seq)
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * used)), used + 1)
    if num_blocks < used:
        raise ValueError("pool smaller than the blocks in use")
    MB = max_blocks_per_seq if max_blocks_per_seq is not None else max(blocks_per_seq + [1])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = float(np.float32(scale))

    q32 = rng.standard_normal((S, Hq, D), dtype=np.float32) * np.float32(sigma)
    k32 = rng.standard_normal((num_blocks, Hkv, BLOCK_SIZE, D), dtype=np.float32) * np.float32(sigma)
    v32 = rng.standard_normal((num_blocks, Hkv, BLOCK_SIZE, D), dtype=np.float32) * np.float32(sigma)
    perm = rng.permutation(num_blocks)
    pad_block = int(perm[used]) if used < num_blocks else int(perm[-1])
    bt = np.full((S, MB), pad_block, dtype=np.int32)
    off = 0
    for b, nb in enumerate(blocks_per_seq):
        bt[b, :nb] = perm[off:off + nb]
        off += nb

    q = to_storage(q32, dtype)
    notes = {}
    if outliers is not None:
        count, delta = outliers
        G = Hq // Hkv
        q64 = storage_to_float32(q, dtype).astype(np.float64)
        for b in range(S):
            n = int(ctx[b])
            pos = np.sort(rng.choice(n, size=min(count, n), replace=False))
            notes.setdefault("outlier_positions", []).append(pos)
            for g in range(Hkv):
                Qg = q64[b, g * G:(g + 1) * G, :]
                rhs = np.full(G, delta / scale)
                x = Qg.T @ np.linalg.solve(Qg @ Qg.T, rhs)
                phys = bt[b, pos // BLOCK_SIZE]
                slot = pos % BLOCK_SIZE
                k32[phys, g, slot, :] += x.astype(np.float32)
    k = to_storage(k32, dtype)
    del k32
    v = to_storage(v32, dtype)
    del v32
    return Workload(name=name, dtype=dtype, q=q, k_cache=k, v_cache=v, block_tables=bt,
                    context_lens=ctx.astype(np.int32), scale=scale,
                    partition_sizes=list(partition_sizes), pad_block=pad_block, seed=seed,
                    notes=notes)


def _tiny(seed=0):
    # batch 1, 1000 tokens, 4 query heads on 1 KV head, d=128, fp32, 63 of 128 blocks.
    return make_workload("tiny", seed, context_lens=[1000], num_q_heads=4, num_kv_heads=1,
                         head_dim=128, dtype="f32", num_blocks=128, partition_sizes=(512,))


def _single(seed=1):
    # batch 1, 8192 tokens, 32/4 heads, d=128, bf16, 512 of a 4096-block pool.
    return make_workload("single_8k", seed, context_lens=[8192], num_q_heads=32,
                         num_kv_heads=4, head_dim=128, dtype="bf16", num_blocks=4096,
                         partition_sizes=(512,))


def _long(seed=2):
    # batch 1, 100000 tokens, 32/4 heads, d=128, bf16, +8 logits on 0.1% of keys.
    return make_workload("long_100k", seed, context_lens=[100000], num_q_heads=32,
                         num_kv_heads=4, head_dim=128, dtype="bf16", num_blocks=7500,
                         partition_sizes=(512,), outliers=(100, 8.0))


def _batched(seed=3):
    # 256 sequences, contexts uniform in [512, 4096], 32/4 heads, d=128, bf16, pool 1.2x.
    return make_workload("batched_256", seed, context_lens=None,
                         context_lens_fn=lambda rng: rng.integers(512, 4096, size=256,
                                                                  endpoint=True),
                         num_q_heads=32, num_kv_heads=4, head_dim=128, dtype="bf16",
                         max_blocks_per_seq=4096 // BLOCK_SIZE, partition_sizes=(512,))


def _mixed(seed=4):
    # 8 sequences of mixed length, 16/2 heads, d=256, fp16 N(0, 0.5^2), P 512 and 256.
    return make_workload("mixed_d256", seed,
                         context_lens=[65536, 32768, 16384, 8192, 2048, 512, 100, 1],
                         num_q_heads=16, num_kv_heads=2, head_dim=256, dtype="f16", sigma=0.5,
                         scale=1.0 / 16.0, partition_sizes=(512, 256))


CONFIGS = {0: _tiny, 1: _single, 2: _long, 3: _batched, 4: _mixed}
CONFIG_NAMES = {0: "tiny", 1: "single_8k", 2: "long_100k", 3: "batched_256", 4: "mixed_d256"}


def config(i):
    """Workload ``i`` of the five named decode configurations (seed = i)."""
    return CONFIGS[i]()


def kv_bytes(context_lens, num_kv_heads, head_dim, dtype):
    """Bytes of K and V that one decode step must read: each cached element once.

    sum_b n_b * Hkv * 2 (K and V) * D * element_bytes.  At D = 128, 2-byte
    elements and one KV head this is 512 bytes per token per layer, the figure
    the prefix_prefill_patch.py analysis (computility-run.yaml section) uses.
    """
    n = int(np.sum(np.asarray(context_lens, dtype=np.int64)))
    return n * int(num_kv_heads) * 2 * int(head_dim) * ELEMENT_BYTES[dtype]


# ---- paged prefix-prefill inputs ------------------------------------------------------
@dataclass
class PrefillWorkload:
    """Inputs of one prefix-prefill step: a chunk of new tokens per sequence (packed q /
    k_new / v_new over the batch) after a prefix already in the paged cache.

    Layouts: q [T, Hq, D]; k_new, v_new [T, Hkv, D]; k_cache, v_cache [NB, Hkv, 16, D];
    block_tables int32 [S, MB] (prefix blocks; padding points at ``pad_block``);
    context_lens int32 [S] (prefix lengths); query_start int32 [S+1] (sequence b owns
    rows query_start[b] .. query_start[b+1]-1)."""
    name: str
    dtype: str
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    query_start: np.ndarray
    scale: float
    pad_block: int
    seed: int

    @property
    def num_seqs(self):
        return self.context_lens.shape[0]

    @property
    def num_tokens(self):
        return self.q.shape[0]

    @property
    def num_q_heads(self):
        return self.q.shape[1]

    @property
    def num_kv_heads(self):
        return self.k_new.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def max_query_len(self):
        return int(np.max(np.diff(self.query_start))) if self.num_seqs else 0


def make_prefill_workload(name, seed, *, context_lens, query_lens, num_q_heads, num_kv_heads,
                          head_dim, dtype, sigma=1.0, scale=None, pool_factor=1.2):
    """Draw one seeded prefill step.  Draw order: q, k_new, v_new, K pool, V pool, block
    permutation; values N(0, sigma^2) in float32, rounded once to the storage dtype."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(query_lens, dtype=np.int64)
    S = ctx.shape[0]
    if ql.shape[0] != S:
        raise ValueError("one query length per sequence")
    T = int(ql.sum())
    Hq, Hkv, D = int(num_q_heads), int(num_kv_heads), int(head_dim)
    nblk = [-(-int(c) // BLOCK_SIZE) for c in ctx]
    MB = max(1, max(nblk) if S else 1)
    used = int(sum(nblk))
    NB = max(used + 1, int(math.ceil(used * pool_factor)) + 1)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    q = to_storage(rng.standard_normal((T, Hq, D), dtype=np.float32) * sigma, dtype)
    k_new = to_storage(rng.standard_normal((T, Hkv, D), dtype=np.float32) * sigma, dtype)
    v_new = to_storage(rng.standard_normal((T, Hkv, D), dtype=np.float32) * sigma, dtype)
    k_cache = to_storage(rng.standard_normal((NB, Hkv, BLOCK_SIZE, D), dtype=np.float32) * sigma,
                         dtype)
    v_cache = to_storage(rng.standard_normal((NB, Hkv, BLOCK_SIZE, D), dtype=np.float32) * sigma,
                         dtype)
    perm = rng.permutation(NB)
    pad_block = int(perm[used])
    bt = np.full((max(S, 0), MB), pad_block, dtype=np.int32)
    o = 0
    for b in range(S):
        bt[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    qs = np.zeros(S + 1, dtype=np.int32)
    qs[1:] = np.cumsum(ql)
    return PrefillWorkload(name=name, dtype=dtype, q=q, k_new=k_new, v_new=v_new,
                           k_cache=k_cache, v_cache=v_cache, block_tables=bt,
                           context_lens=ctx.astype(np.int32), query_start=qs,
                           scale=float(np.float32(scale)), pad_block=pad_block, seed=seed)


def _pf_small(seed=10):
    # 3 sequences: no prefix, a prefix ending mid-block, a 200-token prefix; GQA 4.
    return make_prefill_workload("pf_small", seed, context_lens=[0, 37, 200],
                                 query_lens=[17, 64, 5], num_q_heads=8, num_kv_heads=2,
                                 head_dim=128, dtype="bf16")


def _pf_chunk(seed=11):
    # One 8192-token prefill chunk (the pages' max-num-batched-tokens) after a 65536-token
    # cached prefix; 32/4 heads, head_dim 128, bf16.
    return make_prefill_workload("pf_chunk_8k_at_64k", seed, context_lens=[65536],
                                 query_lens=[8192], num_q_heads=32, num_kv_heads=4,
                                 head_dim=128, dtype="bf16")


def _pf_batch(seed=12):
    # 4 sequences of mixed prefix and chunk lengths, GQA 8, fp16.
    return make_prefill_workload("pf_batch_mixed", seed, context_lens=[4096, 0, 1000, 16384],
                                 query_lens=[1024, 2048, 333, 512], num_q_heads=32,
                                 num_kv_heads=4, head_dim=128, dtype="f16")


def _pf_d256(seed=13):
    # head_dim 256 (the pages' rarer head size, as in the mixed decode workload): a
    # 4096-token chunk after a 16384-token prefix, 16/2 heads, fp16, values N(0, 0.5^2).
    return make_prefill_workload("pf_chunk_4k_at_16k_d256", seed, context_lens=[16384],
                                 query_lens=[4096], num_q_heads=16, num_kv_heads=2,
                                 head_dim=256, dtype="f16", sigma=0.5)


PREFILL_CONFIGS = {0: _pf_small, 1: _pf_chunk, 2: _pf_batch, 3: _pf_d256}
PREFILL_CONFIG_NAMES = {0: "pf_small", 1: "pf_chunk_8k_at_64k", 2: "pf_batch_mixed",
                        3: "pf_chunk_4k_at_16k_d256"}


def prefill_config(i):
    """Prefill workload ``i`` (seed = 10 + i)."""
    return PREFILL_CONFIGS[i]()
