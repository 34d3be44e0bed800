"""Pins of oracle.prefill_attention (no GPU), each against something other than the
oracle's own formula: pure-Python loops, torch's causal SDPA in float64, the decode
oracle, causality and chunking invariants, closed forms and planted mistakes."""
import math

import numpy as np
import pytest

import oracle
from oracle.storage import upcast
from paged_split_kv_pa_amd import workloads as wl

torch = pytest.importorskip("torch")


def tiny(seed, ctx, ql, Hq=4, Hkv=2, D=8, dtype="f32", **kw):
    return wl.make_prefill_workload("t", seed, context_lens=ctx, query_lens=ql, num_q_heads=Hq,
                                    num_kv_heads=Hkv, head_dim=D, dtype=dtype, **kw)


def run(w):
    return oracle.prefill_attention(w.q, w.k_new, w.v_new, w.k_cache, w.v_cache,
                                    w.block_tables, w.context_lens, w.query_start, w.scale,
                                    w.dtype)


def indep_upcast(a, dtype):
    """float64 values of storage arrays via torch (independent of oracle.storage)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(torch.float64).numpy()
    return np.asarray(a).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_brute_force_loops(dtype):
    w = tiny(1, [5, 0, 19], [3, 4, 2], dtype=dtype)
    got = run(w)
    q = indep_upcast(w.q, dtype)
    kn, vn = indep_upcast(w.k_new, dtype), indep_upcast(w.v_new, dtype)
    kc, vc = indep_upcast(w.k_cache, dtype), indep_upcast(w.v_cache, dtype)
    G = w.num_q_heads // w.num_kv_heads
    s = float(np.float32(w.scale))
    for b in range(w.num_seqs):
        c = int(w.context_lens[b])
        r0, r1 = int(w.query_start[b]), int(w.query_start[b + 1])
        for i in range(r1 - r0):
            for h in range(w.num_q_heads):
                g = h // G
                keys, vals = [], []
                for t in range(c):  # the prefix, block by block
                    blk = int(w.block_tables[b, t // 16])
                    keys.append(kc[blk, g, t % 16])
                    vals.append(vc[blk, g, t % 16])
                for j in range(i + 1):  # new tokens 0..i
                    keys.append(kn[r0 + j, g])
                    vals.append(vn[r0 + j, g])
                lg = [s * math.fsum(float(x) * float(y) for x, y in zip(q[r0 + i, h], k))
                      for k in keys]
                m = max(lg)
                e = [math.exp(x - m) for x in lg]
                tot = math.fsum(e)
                for d in range(w.head_dim):
                    ref = math.fsum(e[t] * float(vals[t][d]) for t in range(len(e))) / tot
                    assert abs(got[r0 + i, h, d] - ref) <= 1e-12 * (1 + abs(ref))


def test_no_prefix_equals_causal_sdpa():
    w = tiny(2, [0, 0], [33, 7], Hq=8, Hkv=2, D=16)
    got = run(w)
    G = 4
    for b in range(2):
        r0, r1 = int(w.query_start[b]), int(w.query_start[b + 1])
        q = torch.from_numpy(upcast(w.q[r0:r1], "f32")).permute(1, 0, 2)          # [Hq, L, D]
        k = torch.from_numpy(upcast(w.k_new[r0:r1], "f32")).permute(1, 0, 2)
        v = torch.from_numpy(upcast(w.v_new[r0:r1], "f32")).permute(1, 0, 2)
        k = k.repeat_interleave(G, dim=0)
        v = v.repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], is_causal=True, scale=float(np.float32(w.scale)))[0]
        assert np.allclose(got[r0:r1], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_one_new_token_equals_decode_with_the_token_cached():
    """L = 1: the new token attends to the prefix and itself = decode over c + 1 cached
    tokens once its K/V are written into the cache (block table extended)."""
    w = tiny(3, [21, 0, 47], [1, 1, 1], Hq=6, Hkv=3, D=8)
    got = run(w)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    S = w.num_seqs
    bt = np.zeros((S, 4), dtype=np.int32)
    free = [x for x in range(kc.shape[0]) if x not in set(w.block_tables.ravel())]
    nxt = 0
    for b in range(S):
        c = int(w.context_lens[b])
        nb = -(-c // 16)
        bt[b, :nb] = w.block_tables[b, :nb]
        if c % 16 == 0:  # the token starts a new block
            bt[b, nb] = free[nxt]
            nxt += 1
        blk = bt[b, c // 16]
        kc[blk, :, c % 16] = w.k_new[b]
        vc[blk, :, c % 16] = w.v_new[b]
    ref = oracle.decode_attention(w.q, kc, vc, bt, w.context_lens + 1, w.scale, w.dtype)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_causality_and_prefix_bounds():
    w = tiny(4, [30, 9], [12, 6], D=8)
    base = run(w)
    # later new tokens do not influence earlier rows
    w.k_new[5:12] = 0
    w.v_new[5:12] = 7
    changed = run(w)
    assert np.array_equal(base[:5], changed[:5])
    assert not np.allclose(base[5:12], changed[5:12])
    # cache contents outside the prefix (pool blocks not in the table, tail slots) are not read
    w2 = tiny(4, [30, 9], [12, 6], D=8)
    used = set()
    for b in range(2):
        c = int(w2.context_lens[b])
        used |= {int(x) for x in w2.block_tables[b, :-(-c // 16)]}
    for blk in range(w2.k_cache.shape[0]):
        if blk not in used:
            w2.k_cache[blk] = np.nan
            w2.v_cache[blk] = np.nan
    w2.k_cache[w2.block_tables[0, 1], :, 14:] = np.nan  # tokens 30, 31 of sequence 0
    assert np.array_equal(run(w2), base)


def test_chunked_prefill_is_consistent():
    """Rows [0, L1) with prefix c and rows [L1, L) with prefix c + L1 (the first L1 new
    tokens moved into the cache) give the one-chunk result."""
    c, L, L1 = 20, 25, 12
    w = tiny(5, [c], [L], Hq=4, Hkv=1, D=8)
    full = run(w)
    first = wl.make_prefill_workload("a", 5, context_lens=[c], query_lens=[L1], num_q_heads=4,
                                     num_kv_heads=1, head_dim=8, dtype="f32")
    for name in ("q", "k_new", "v_new"):
        getattr(first, name)[...] = getattr(w, name)[:L1]
    first.k_cache, first.v_cache, first.block_tables = w.k_cache, w.v_cache, w.block_tables
    assert np.allclose(run(first), full[:L1], rtol=1e-13, atol=1e-14)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    bt = np.zeros((1, 4), dtype=np.int32)
    bt[0, :2] = w.block_tables[0, :2]
    bt[0, 2] = [x for x in range(kc.shape[0]) if x not in set(w.block_tables.ravel())][0]
    for t in range(L1):
        pos = c + t
        kc[bt[0, pos // 16], :, pos % 16] = w.k_new[t]
        vc[bt[0, pos // 16], :, pos % 16] = w.v_new[t]
    second = oracle.prefill_attention(w.q[L1:], w.k_new[L1:], w.v_new[L1:], kc, vc, bt,
                                      np.array([c + L1]), np.array([0, L - L1]), w.scale, "f32")
    assert np.allclose(second, full[L1:], rtol=1e-12, atol=1e-13)


def test_closed_forms():
    w = tiny(6, [0], [1], D=8)
    out = run(w)  # one token, no prefix: the output is its own V, exactly
    G = 2
    for h in range(4):
        assert np.array_equal(out[0, h], upcast(w.v_new[0, h // G], "f32"))
    w = tiny(7, [40], [9], D=8)
    w.v_cache[...] = 3.25
    w.v_new[...] = 3.25
    assert np.allclose(run(w), 3.25, rtol=1e-14, atol=0)
    w = tiny(8, [40], [9], D=8, scale=0.0)  # scale 0: the mean of the visible V rows
    out = run(w)
    vp = upcast(oracle.gather_sequence(w.v_cache, w.block_tables, 0, 40), "f32")
    vn = upcast(w.v_new, "f32")
    for i in range(9):
        allv = np.concatenate([vp, vn[:i + 1]], axis=0)
        assert np.allclose(out[i, 0], allv[:, 0].mean(axis=0), rtol=1e-13)


def test_flop_count():
    # 4 * Hq * D * (L*c + L(L+1)/2) summed over sequences
    assert oracle.prefill_flops([65536], [0, 8192], 32, 128) == \
        4 * 32 * 128 * (8192 * 65536 + 8192 * 8193 // 2)
    assert oracle.prefill_flops([0, 5], [0, 1, 3], 2, 8) == 4 * 2 * 8 * (1 + (2 * 5 + 3))


def test_planted_mistakes_are_caught():
    """Off-by-one causal mask, a dropped prefix, h % Hkv grouping, a missing scale: each
    changes the result of a small case."""
    w = tiny(9, [18, 3], [7, 5], Hq=4, Hkv=2, D=8)
    good = run(w)
    q64, kn, vn = upcast(w.q, "f32"), upcast(w.k_new, "f32"), upcast(w.v_new, "f32")
    s = float(np.float32(w.scale))

    def variant(shift=0, prefix=True, grouping=lambda h: h // 2, scale=s):
        out = np.zeros_like(good)
        for b in range(2):
            c = int(w.context_lens[b])
            r0, r1 = int(w.query_start[b]), int(w.query_start[b + 1])
            kp = upcast(oracle.gather_sequence(w.k_cache, w.block_tables, b, c), "f32")
            vp = upcast(oracle.gather_sequence(w.v_cache, w.block_tables, b, c), "f32")
            if not prefix:
                kp, vp, c = kp[:0], vp[:0], 0
            ka = np.concatenate([kp, kn[r0:r1]])
            va = np.concatenate([vp, vn[r0:r1]])
            for h in range(4):
                g = grouping(h)
                out[r0:r1, h] = oracle.prefill_rows(q64[r0:r1, h], ka[:, g], va[:, g],
                                                    c + shift, scale)
        return out

    assert np.allclose(variant(), good, rtol=1e-13)
    for bad in (variant(shift=-1), variant(shift=1), variant(prefix=False),
                variant(grouping=lambda h: h % 2), variant(scale=1.0)):
        assert not np.allclose(bad, good, rtol=1e-6)
