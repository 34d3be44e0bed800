"""GPU parity of pa_prefill (paged prefix-prefill attention) against the float64 oracle.

Same bar as decode (fp16/bf16 inputs, fp32 accumulation): |gpu - ref| <= 2e-3 + 1e-2 |ref|
element-wise and per-(row, head) relative L2 <= 1e-2, against the unrounded oracle;
bitwise determinism and block-placement invariance; cache contents outside the prefix
never read."""
import sys

import numpy as np
import pytest

import oracle
from paged_split_kv_pa_amd import binding as B
from paged_split_kv_pa_amd import workloads as wl

from helpers import check_close, to_device, to_f64

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


def upload(w):
    d = {n: to_device(getattr(w, n), w.dtype) for n in ("q", "k_new", "v_new", "k_cache",
                                                          "v_cache")}
    for n in ("block_tables", "context_lens", "query_start"):
        d[n] = torch.from_numpy(np.ascontiguousarray(getattr(w, n), dtype=np.int32)).cuda()
    return d


def run(w, dev, max_query_len=0, out=None):
    if out is None:
        out = torch.empty_like(dev["q"])
    B.pa_prefill(out, dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                 dev["block_tables"], dev["context_lens"], dev["query_start"], w.scale,
                 max_query_len=max_query_len)
    torch.cuda.synchronize()
    return out


def reference(w):
    return oracle.prefill_attention(w.q, w.k_new, w.v_new, w.k_cache, w.v_cache,
                                    w.block_tables, w.context_lens, w.query_start, w.scale,
                                    w.dtype)


def check_rows(got, ref, what):
    """check_close on [T, Hq, D] treated as (row, head) pairs."""
    check_close(got.reshape(1, -1, got.shape[-1]), ref.reshape(1, -1, ref.shape[-1]), what)


def test_pf_small():
    w = wl.prefill_config(0)
    say(f"prefill {w.name}")
    check_rows(to_f64(run(w, upload(w))), reference(w), "pf_small")


EDGE = [(dt, G) for dt in ("bf16", "f16") for G in (1, 2, 4, 8, 16)]


@pytest.mark.parametrize("dtype,G", EDGE, ids=[f"{a}-g{b}" for a, b in EDGE])
def test_edge_shapes(dtype, G):
    ctx = [0, 1, 15, 16, 17, 63, 64, 65, 300, 0]
    ql = [1, 2, 17, 64, 65, 100, 257, 3, 1, 0]
    w = wl.make_prefill_workload("edge", 500 + G, context_lens=ctx, query_lens=ql,
                                 num_q_heads=2 * G, num_kv_heads=2, head_dim=128, dtype=dtype)
    say(f"prefill edge dtype={dtype} G={G} T={w.num_tokens}")
    check_rows(to_f64(run(w, upload(w))), reference(w), f"prefill edge {dtype} G={G}")


def test_pf_batch_mixed():
    w = wl.prefill_config(2)
    say(f"prefill {w.name} T={w.num_tokens}")
    check_rows(to_f64(run(w, upload(w))), reference(w), "pf_batch_mixed")


def test_pf_batch_mixed_rows_equal_single_sequence_runs():
    """Without the planned schedule (pa_set_prefill_split(0)) the work-groups take
    sequences most keys first (the longest prefix plus chunk first) and position blocks
    last first; every sequence's rows must be bitwise those of a prefill of that sequence
    alone (one sequence: grid order)."""
    w = wl.prefill_config(2)
    dev = upload(w)
    old = B.pa_get_prefill_split()
    B.pa_set_prefill_split(0)
    try:
        _rows_equal_single(w, dev)
    finally:
        B.pa_set_prefill_split(old)


def _rows_equal_single(w, dev):
    batch = run(w, dev)
    qs = np.asarray(w.query_start)
    for b in range(len(w.context_lens)):
        r0, r1 = int(qs[b]), int(qs[b + 1])
        say(f"prefill {w.name}: sequence {b} alone (rows {r0}..{r1})")
        one = {n: dev[n][r0:r1].clone() for n in ("q", "k_new", "v_new")}
        one["k_cache"], one["v_cache"] = dev["k_cache"], dev["v_cache"]
        one["block_tables"] = dev["block_tables"][b:b + 1].clone()
        one["context_lens"] = dev["context_lens"][b:b + 1].clone()
        one["query_start"] = torch.tensor([0, r1 - r0], dtype=torch.int32, device="cuda")
        got = run(w, one)
        assert torch.equal(got, batch[r0:r1]), f"sequence {b}"


def test_pf_chunk_sampled_rows():
    """The 8192-token chunk after a 65536-token prefix: 96 sampled (row, head) outputs
    against the oracle's causal rows, one at a time."""
    w = wl.prefill_config(1)
    say(f"prefill {w.name} (sampled rows)")
    got = to_f64(run(w, upload(w)))
    c = int(w.context_lens[0])
    G = w.num_q_heads // w.num_kv_heads
    from oracle.storage import upcast
    rng = np.random.default_rng(0)
    rows = np.concatenate([[0, 1, 255, 256, 8191], rng.integers(0, w.num_tokens, 91)])
    heads = rng.integers(0, w.num_q_heads, rows.shape[0])
    kp = upcast(oracle.gather_sequence(w.k_cache, w.block_tables, 0, c), w.dtype)
    vp = upcast(oracle.gather_sequence(w.v_cache, w.block_tables, 0, c), w.dtype)
    kn, vn = upcast(w.k_new, w.dtype), upcast(w.v_new, w.dtype)
    q = upcast(w.q, w.dtype)
    s = float(np.float32(w.scale))
    ref = np.zeros((rows.shape[0], w.head_dim))
    gs = np.zeros((rows.shape[0], w.head_dim))
    for n, (i, h) in enumerate(zip(rows, heads)):
        g = h // G
        ka = np.concatenate([kp[:, g], kn[:i + 1, g]])
        va = np.concatenate([vp[:, g], vn[:i + 1, g]])
        ref[n] = oracle.prefill_rows(q[i:i + 1, h], ka, va, c + i, s)[0]
        gs[n] = got[i, h]
    check_close(gs[None], ref[None], "pf_chunk sampled rows")


def test_determinism_placement_and_poison():
    w = wl.make_prefill_workload("pp", 77, context_lens=[70, 33, 128], query_lens=[40, 90, 7],
                                 num_q_heads=16, num_kv_heads=2, head_dim=128, dtype="bf16")
    dev = upload(w)
    a = run(w, dev)
    b = run(w, dev)
    assert torch.equal(a, b), "runs must be bitwise deterministic"
    # same logical cache, different physical blocks
    rng = np.random.default_rng(3)
    perm = rng.permutation(w.k_cache.shape[0])
    k2 = np.empty_like(w.k_cache)
    v2 = np.empty_like(w.v_cache)
    k2[perm] = w.k_cache
    v2[perm] = w.v_cache
    w2 = wl.PrefillWorkload(w.name, w.dtype, w.q, w.k_new, w.v_new, k2, v2,
                            perm[w.block_tables].astype(np.int32), w.context_lens,
                            w.query_start, w.scale, int(perm[w.pad_block]), w.seed)
    assert torch.equal(run(w2, upload(w2)), a), "block placement must not change the bits"
    # NaN in every pool block the prefixes do not use and in the tail slots after them
    used = set()
    for bb, c in enumerate(w.context_lens):
        used |= {int(x) for x in w.block_tables[bb, :-(-int(c) // 16)]}
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    nan = np.uint16(0x7FC0)
    for blk in range(kp.shape[0]):
        if blk not in used:
            kp[blk] = nan
            vp[blk] = nan
    for bb, c in enumerate(w.context_lens):
        c = int(c)
        if c % 16:
            kp[w.block_tables[bb, c // 16], :, c % 16:] = nan
            vp[w.block_tables[bb, c // 16], :, c % 16:] = nan
    w3 = wl.PrefillWorkload(w.name, w.dtype, w.q, w.k_new, w.v_new, kp, vp, w.block_tables,
                            w.context_lens, w.query_start, w.scale, w.pad_block, w.seed)
    assert torch.equal(run(w3, upload(w3)), a), "cache contents outside the prefix were read"


def test_out_of_range_block_ids_read_as_zero_rows():
    """A prefix block id outside [0, NB) (-1, NB, NB + 1000, 2^31 - 1) reads its tokens as
    zero keys and values, as the header states: the output equals the oracle's on a pool
    with an all-zero block at those table entries.  The broken blocks sit in whole-wave
    prefix rows, in a wave whose rows run from the prefix into the new tokens, and in
    the first block of a prefix."""
    w = wl.make_prefill_workload("badid", 91, context_lens=[200, 77, 40], query_lens=[33, 20, 64],
                                 num_q_heads=16, num_kv_heads=2, head_dim=128, dtype="bf16")
    NB = w.k_cache.shape[0]
    bad = [(0, 2, -1), (0, 5, NB), (1, 4, NB + 1000), (2, 0, 2**31 - 1)]
    bt_gpu = w.block_tables.copy()
    bt_ref = w.block_tables.copy()
    for b, j, bid in bad:
        assert j < -(-int(w.context_lens[b]) // 16), "the broken block must lie in the prefix"
        bt_gpu[b, j] = bid
        bt_ref[b, j] = NB  # the appended zero block
    kz = np.concatenate([w.k_cache, np.zeros_like(w.k_cache[:1])])
    vz = np.concatenate([w.v_cache, np.zeros_like(w.v_cache[:1])])
    w_gpu = wl.PrefillWorkload(w.name, w.dtype, w.q, w.k_new, w.v_new, w.k_cache, w.v_cache,
                               bt_gpu, w.context_lens, w.query_start, w.scale, w.pad_block,
                               w.seed)
    w_ref = wl.PrefillWorkload(w.name, w.dtype, w.q, w.k_new, w.v_new, kz, vz, bt_ref,
                               w.context_lens, w.query_start, w.scale, w.pad_block, w.seed)
    say("prefill out-of-range block ids")
    got = to_f64(run(w_gpu, upload(w_gpu)))
    assert np.isfinite(got).all()
    check_rows(got, reference(w_ref), "prefill out-of-range block ids")


def test_max_query_len_bounds_the_rows_written():
    w = wl.make_prefill_workload("mq", 78, context_lens=[20, 5], query_lens=[300, 40],
                                 num_q_heads=8, num_kv_heads=1, head_dim=128, dtype="f16")
    dev = upload(w)
    out = torch.full_like(dev["q"], 7.0)
    run(w, dev, max_query_len=64, out=out)
    got = to_f64(out)
    ref = reference(w)
    qs = w.query_start
    for b, L in enumerate((300, 40)):
        r0 = int(qs[b])
        k = min(L, 64)
        check_rows(got[r0:r0 + k], ref[r0:r0 + k], f"max_query_len seq {b}")
        assert np.all(got[r0 + k:r0 + L] == 7.0), "rows past max_query_len must be untouched"


@pytest.mark.parametrize("scale", [-0.3, -0.09, 0.0, 0.09, 0.3])
def test_scale_sign_and_zero(scale):
    """A negative scale (carried as a sign flip of q in the kernel), scale 0 (uniform
    weights over the visible keys) and |scale| 0.3 (logits 3.4x wider than at
    1/sqrt(128), a peaky softmax) against the oracle, N(0, 1) inputs."""
    w = wl.make_prefill_workload("sc", 90, context_lens=[50, 0], query_lens=[37, 70],
                                 num_q_heads=16, num_kv_heads=2, head_dim=128, dtype="bf16",
                                 scale=scale)
    say(f"prefill scale={scale}")
    check_rows(to_f64(run(w, upload(w))), reference(w), f"scale {scale}")


EDGE256 = [(dt, G) for dt in ("bf16", "f16") for G in (1, 4, 16)]


@pytest.mark.parametrize("dtype,G", EDGE256, ids=[f"{a}-g{b}" for a, b in EDGE256])
def test_head_dim_256(dtype, G):
    """head_dim 256 (one 16-row column group per wave, 128 rows per work-group): ragged
    prefixes and chunks around the 64-key tile and the 128/G-position work-group edges.
    Values N(0, 1)."""
    ctx = [0, 1, 63, 64, 65, 300, 1000]
    ql = [1, 130, 17, 64, 129, 3, 200]
    w = wl.make_prefill_workload("d256", 700 + G, context_lens=ctx, query_lens=ql,
                                 num_q_heads=2 * G, num_kv_heads=2, head_dim=256, dtype=dtype)
    say(f"prefill d256 dtype={dtype} G={G} T={w.num_tokens}")
    check_rows(to_f64(run(w, upload(w))), reference(w), f"prefill d256 {dtype} G={G}")


def test_head_dim_256_long_chunk_sampled_rows():
    """The head_dim 256 bench workload (4096 new tokens after a 16384-token prefix):
    48 sampled (row, head) outputs against the oracle's causal rows."""
    w = wl.prefill_config(3)
    say(f"prefill {w.name} (sampled rows)")
    got = to_f64(run(w, upload(w)))
    c = int(w.context_lens[0])
    G = w.num_q_heads // w.num_kv_heads
    from oracle.storage import upcast
    rng = np.random.default_rng(5)
    rows = np.concatenate([[0, 1, 127, 128, 4095], rng.integers(0, w.num_tokens, 43)])
    heads = rng.integers(0, w.num_q_heads, rows.shape[0])
    kp = upcast(oracle.gather_sequence(w.k_cache, w.block_tables, 0, c), w.dtype)
    vp = upcast(oracle.gather_sequence(w.v_cache, w.block_tables, 0, c), w.dtype)
    kn, vn = upcast(w.k_new, w.dtype), upcast(w.v_new, w.dtype)
    q = upcast(w.q, w.dtype)
    s = float(np.float32(w.scale))
    ref = np.zeros((rows.shape[0], w.head_dim))
    gs = np.zeros((rows.shape[0], w.head_dim))
    for n, (i, h) in enumerate(zip(rows, heads)):
        g = h // G
        ka = np.concatenate([kp[:, g], kn[:i + 1, g]])
        va = np.concatenate([vp[:, g], vn[:i + 1, g]])
        ref[n] = oracle.prefill_rows(q[i:i + 1, h], ka, va, c + i, s)[0]
        gs[n] = got[i, h]
    check_close(gs[None], ref[None], "pf_chunk_d256 sampled rows")



PREC = [(D, dt, G, sc) for D in (128, 256) for dt in ("bf16", "f16") for G in (1, 4, 8, 16)
        for sc in ("pages", "0.3")]


@pytest.mark.parametrize("D,dtype,G,scale_kind", PREC,
                         ids=[f"D{d}-{t}-G{g}-scale_{s}" for d, t, g, s in PREC])
def test_precision_sweep(D, dtype, G, scale_kind):
    """N(0, 1) inputs, short prefixes and chunks (rows that see 1 to ~150 keys: few keys
    carry the weight, where the rounding of the probabilities matters most), both head
    dims and element types, the pages' scale 1/sqrt(D) and 0.3, against the oracle at the
    decode tolerance."""
    scale = 1.0 / np.sqrt(D) if scale_kind == "pages" else 0.3
    seed = 2000 + PREC.index((D, dtype, G, scale_kind))
    rng = np.random.default_rng(seed)
    ctx = [int(x) for x in rng.integers(0, 100, size=4)]
    ql = [int(x) for x in rng.integers(1, 80, size=4)]
    w = wl.make_prefill_workload("prec", seed, context_lens=ctx, query_lens=ql,
                                 num_q_heads=2 * G, num_kv_heads=2, head_dim=D, dtype=dtype,
                                 scale=scale)
    say(f"prefill precision D={D} {dtype} G={G} scale={w.scale:.4f} ctx={ctx} ql={ql}")
    check_rows(to_f64(run(w, upload(w))), reference(w), f"prefill D={D} {dtype} G={G} {scale}")
