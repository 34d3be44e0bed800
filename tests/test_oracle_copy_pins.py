"""Pins of oracle.copy_blocks against element-by-element loops and the readings
stated in its docstring (no GPU)."""
import numpy as np
import pytest

import oracle


def loop_copy(k, v, pairs):
    """Element-wise brute force over a snapshot (pure Python loops)."""
    nb = k.shape[0]
    k2, v2 = k.copy(), v.copy()
    snap_k, snap_v = k.copy(), v.copy()
    for s, d in pairs:
        if not (0 <= s < nb and 0 <= d < nb):
            continue
        for idx in np.ndindex(*k.shape[1:]):
            k2[(d,) + idx] = snap_k[(s,) + idx]
            v2[(d,) + idx] = snap_v[(s,) + idx]
    return k2, v2


@pytest.mark.parametrize("dtype", [np.float32, np.float16, np.uint16])
def test_matches_element_loops(dtype):
    rng = np.random.default_rng(5)
    k = (rng.integers(0, 1 << 16, size=(9, 2, 4, 3))).astype(dtype)
    v = (rng.integers(0, 1 << 16, size=(9, 2, 4, 3))).astype(dtype)
    pairs = [(0, 5), (3, 7), (8, 1), (2, 2), (4, 9), (-1, 3), (6, 0)]
    got = oracle.copy_blocks(k, v, pairs)
    want = loop_copy(k, v, pairs)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    # the inputs are not modified
    assert not np.shares_memory(got[0], k)


def test_bitwise_including_nan_payloads():
    k = np.full((3, 1, 2, 2), np.nan, dtype=np.float32)
    k.view(np.uint32)[0] = 0x7fc00123  # a NaN with a payload survives a bitwise copy
    v = np.zeros_like(k)
    v[0] = -0.0
    k2, v2 = oracle.copy_blocks(k, v, [(0, 2)])
    assert np.array_equal(k2.view(np.uint32)[2], k.view(np.uint32)[0])
    assert np.signbit(v2[2]).all()


def test_untouched_blocks_and_identity_pairs():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((6, 2, 16, 8)).astype(np.float32)
    v = rng.standard_normal((6, 2, 16, 8)).astype(np.float32)
    k2, v2 = oracle.copy_blocks(k, v, [(1, 1), (4, 4)])
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    k3, v3 = oracle.copy_blocks(k, v, [(0, 3)])
    for b in (0, 1, 2, 4, 5):
        assert np.array_equal(k3[b], k[b]) and np.array_equal(v3[b], v[b])
    assert np.array_equal(k3[3], k[0]) and np.array_equal(v3[3], v[0])


def test_reads_precede_writes():
    # A chain 0 -> 1, 1 -> 2: block 2 receives the old block 1 (snapshot semantics).
    k = np.arange(3 * 4, dtype=np.float32).reshape(3, 1, 1, 4)
    k2, _ = oracle.copy_blocks(k, k.copy(), [(0, 1), (1, 2)])
    assert np.array_equal(k2[2], k[1]) and np.array_equal(k2[1], k[0])


def test_out_of_range_pairs_are_skipped_and_empty_list_is_identity():
    k = np.ones((4, 1, 2, 2), dtype=np.float16)
    v = np.zeros((4, 1, 2, 2), dtype=np.float16)
    for pairs in ([(4, 0)], [(0, 4)], [(-1, 0)], [(0, -2)], np.zeros((0, 2), dtype=np.int32)):
        k2, v2 = oracle.copy_blocks(k, v, pairs)
        assert np.array_equal(k2, k) and np.array_equal(v2, v)


def test_planted_mistakes_are_caught():
    """K and V swapped, src/dst swapped, or an in-place sequential copy: each fails a pin."""
    k = np.arange(3 * 2, dtype=np.float32).reshape(3, 1, 1, 2)
    v = -k
    pairs = [(0, 1), (1, 2)]
    want_k, want_v = loop_copy(k, v, pairs)

    def swapped_kv(k, v, p):
        a, b = oracle.copy_blocks(k, v, p)
        return b, a

    def swapped_dir(k, v, p):
        return oracle.copy_blocks(k, v, [(d, s) for s, d in p])

    def sequential(k, v, p):
        k2, v2 = k.copy(), v.copy()
        for s, d in p:
            k2[d] = k2[s]
            v2[d] = v2[s]
        return k2, v2

    for bad in (swapped_kv, swapped_dir, sequential):
        got = bad(k, v, pairs)
        assert not (np.array_equal(got[0], want_k) and np.array_equal(got[1], want_v)), bad
