"""GPU parity of pa_copy_blocks (prefix-caching block copy) against oracle.copy_blocks:
bit-exact, whole pools compared (copied blocks, untouched blocks, skipped pairs)."""
import sys

import numpy as np
import pytest

import oracle
from paged_split_kv_pa_amd import binding as B

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


NP_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}
TORCH_BITS = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}


def pools(seed, NB, Hkv, D, dtype):
    """Random bit patterns (NaN and Inf payloads included): a bitwise copy must keep them."""
    rng = np.random.default_rng(seed)
    bits = NP_BITS[dtype]
    k = rng.integers(0, np.iinfo(bits).max, size=(NB, Hkv, 16, D), dtype=np.uint64).astype(bits)
    v = rng.integers(0, np.iinfo(bits).max, size=(NB, Hkv, 16, D), dtype=np.uint64).astype(bits)
    return k, v


def disjoint_pairs(seed, NB, n):
    rng = np.random.default_rng(seed)
    ids = rng.permutation(NB)[:2 * n]
    return np.stack([ids[:n], ids[n:]], axis=1).astype(np.int32)


def run(k, v, pairs, dtype, with_v=True):
    dk = torch.from_numpy(k.view(np.int32 if dtype == "f32" else np.int16).copy()).cuda()
    dv = torch.from_numpy(v.view(np.int32 if dtype == "f32" else np.int16).copy()).cuda()
    dp = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32)).cuda()
    B.pa_copy_blocks(dk, dv if with_v else None, dp)
    torch.cuda.synchronize()
    return (dk.cpu().numpy().view(k.dtype), dv.cpu().numpy().view(v.dtype))


CASES = [("bf16", 4, 128, 300, 97), ("f16", 8, 256, 64, 20), ("f32", 1, 128, 50, 25),
         ("f32", 2, 256, 40, 11), ("bf16", 16, 128, 33, 16)]


@pytest.mark.parametrize("dtype,Hkv,D,NB,n", CASES,
                         ids=[f"{a}-h{b}-d{c}-nb{d}-n{e}" for a, b, c, d, e in CASES])
def test_copy_matches_oracle_bitwise(dtype, Hkv, D, NB, n):
    k, v = pools(Hkv + D + NB, NB, Hkv, D, dtype)
    pairs = disjoint_pairs(n, NB, n)
    say(f"copy dtype={dtype} Hkv={Hkv} D={D} NB={NB} pairs={n} block_bytes="
        f"{Hkv * 16 * D * k.itemsize}")
    got_k, got_v = run(k, v, pairs, dtype)
    want_k, want_v = oracle.copy_blocks(k, v, pairs)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)


def test_skipped_pairs_identity_pairs_and_k_only():
    k, v = pools(3, 40, 4, 128, "bf16")
    pairs = np.array([[0, 5], [40, 6], [7, -1], [-3, 8], [9, 9], [10, 11], [2147483647, 1]],
                     dtype=np.int32)
    say("copy with out-of-range and identity pairs")
    got_k, got_v = run(k, v, pairs, "bf16")
    want_k, want_v = oracle.copy_blocks(k, v, pairs)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)
    say("copy K only")
    got_k, got_v = run(k, v, pairs, "bf16", with_v=False)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, v)


def test_block_bytes_not_a_multiple_of_the_chunk():
    # 3 KV heads x 16 x 128 x 2 B = 12 KiB per block (one short chunk) and 5 x 16 x 128 x
    # 4 B = 40 KiB (two whole 16 KiB chunks and a short one).
    for dtype, Hkv, D in (("bf16", 3, 128), ("f32", 5, 128)):
        k, v = pools(Hkv, 12, Hkv, D, dtype)
        pairs = disjoint_pairs(1, 12, 5)
        say(f"copy ragged chunks dtype={dtype} Hkv={Hkv} D={D}")
        got_k, got_v = run(k, v, pairs, dtype)
        want_k, want_v = oracle.copy_blocks(k, v, pairs)
        assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)


def test_empty_pair_list_is_a_no_op():
    k, v = pools(4, 8, 2, 128, "f16")
    got_k, got_v = run(k, v, np.zeros((0, 2), dtype=np.int32), "f16")
    assert np.array_equal(got_k, k) and np.array_equal(got_v, v)
