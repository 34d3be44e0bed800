"""GPU parity of the HIP path against the float64 oracle (needs an MI355X).

Every call goes through the C ABI (paged_split_kv_pa_amd.binding -> libpa_decode.so).
The bar: fp16/bf16 results within |gpu - ref| <= 2e-3 + 1e-2 |ref| element-wise and a
per-(sequence, head) relative L2 error <= 1e-2 against the unrounded float64 oracle;
block-table indexing bit-exact (placement and poison tests); runs bitwise deterministic.
"""
import sys

import numpy as np
import pytest

import oracle
from paged_split_kv_pa_amd import binding as B
from paged_split_kv_pa_amd import workloads as wl

from helpers import check_close, fused_mode, small_workload, to_f64, upload, work_split

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


_CACHE = {}


def config_case(i):
    """Workload i, its device tensors and the oracle output (cached per module)."""
    if i not in _CACHE:
        w = wl.config(i)
        ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables,
                                      w.context_lens, w.scale, w.dtype)
        _CACHE[i] = (w, upload(w), ref)
    return _CACHE[i]


def run_path(w, dev, path, P, variant=None, max_context_len=0):
    out = torch.empty_like(dev["q"])
    ws = None
    if path != B.PA_PATH_V1:
        nbytes = B.pa_workspace_bytes(dev["q"], dev["k_cache"], dev["block_tables"],
                                      max_context_len, P)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    if variant is not None:
        B.pa_set_mfma_variant(variant)
    B.pa_decode_ex(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                   dev["context_lens"], w.scale, P, workspace=ws,
                   max_context_len=max_context_len, path=path)
    torch.cuda.synchronize()
    return out


CONFIG_CASES = []
for _i in range(5):
    _Ps = (512, 256) if _i == 4 else (512,)
    for _P in _Ps:
        for _path in (B.PA_PATH_AUTO, B.PA_PATH_V1, B.PA_PATH_V2):
            CONFIG_CASES.append((_i, _P, _path))


@pytest.mark.parametrize("cfg,P,path", CONFIG_CASES,
                         ids=[f"{wl.CONFIG_NAMES[c]}-P{p}-{['auto', 'v1', 'v2'][q]}"
                              for c, p, q in CONFIG_CASES])
def test_config_parity(cfg, P, path):
    w, dev, ref = config_case(cfg)
    say(f"config {wl.CONFIG_NAMES[cfg]} P={P} path={path} dtype={w.dtype} "
        f"S={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim}")
    out = run_path(w, dev, path, P)
    check_close(to_f64(out), ref, f"{wl.CONFIG_NAMES[cfg]} P={P} path={path}")


@pytest.mark.parametrize("variant", [0, 1, 2, 3, -1])
@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_mfma_variants(cfg, variant):
    w, dev, ref = config_case(cfg)
    old = B.pa_get_mfma_variant()
    try:
        say(f"variant {variant} on {wl.CONFIG_NAMES[cfg]}")
        out = run_path(w, dev, B.PA_PATH_V2, 512, variant=variant)
    finally:
        B.pa_set_mfma_variant(old)
    check_close(to_f64(out), ref, f"variant {variant}")


@pytest.mark.parametrize("cfg,P", [(0, 512), (1, 512), (4, 256), (4, 512)])
def test_phase1_partials_match_partitioned_oracle(cfg, P):
    """Partial outputs, exp-sums and max logits of every partition (Phase 1)."""
    w, dev, _ = config_case(cfg)
    say(f"partials {wl.CONFIG_NAMES[cfg]} P={P}")
    lay = B.workspace_layout(dev["q"], dev["k_cache"], dev["block_tables"], 0, P)
    ws = torch.zeros(lay["bytes"], dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    B.pa_v2_partition(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                      dev["context_lens"], w.scale, ws, P)
    torch.cuda.synchronize()
    _, parts = oracle.partitioned_decode(w.q, w.k_cache, w.v_cache, w.block_tables,
                                         w.context_lens, w.scale, w.dtype, P,
                                         max_partitions=lay["pmax"])
    raw = ws.cpu().numpy()

    def view(name):
        off, shape = lay[name]
        n = int(np.prod(shape))
        return raw[off:off + 4 * n].view(np.float32).reshape(shape).astype(np.float64)

    tmp, ml, es = view("tmp_out"), view("max_logits"), view("exp_sums")
    for b, n in enumerate(w.context_lens):
        cnt = oracle.num_partitions(int(n), P)
        if cnt <= 1:
            continue  # single-partition sequences write the final output instead
        np.testing.assert_allclose(ml[b, :, :cnt], parts["max_logits"][b, :, :cnt],
                                   rtol=1e-5, atol=1e-4)
        np.testing.assert_allclose(es[b, :, :cnt], parts["exp_sums"][b, :, :cnt], rtol=2e-4)
        check_close(tmp[b, :, :cnt], parts["tmp_out"][b, :, :cnt], f"tmp_out seq {b}")


# ---- edge cases across both kernels: dtypes, head dims, GQA groups, ragged contexts ----
EDGE = []
for _dt in ("f32", "f16", "bf16"):
    for _D in (128, 256):
        for _G in (1, 2, 4, 8, 16):
            EDGE.append((_dt, _D, _G))


@pytest.mark.parametrize("dtype,D,G", EDGE, ids=[f"{a}-d{b}-g{c}" for a, b, c in EDGE])
def test_edge_contexts(dtype, D, G):
    ctx = [0, 1, 15, 16, 17, 63, 64, 65, 200, 1000]
    w = small_workload(100 + G + D, ctx, Hq=2 * G, Hkv=2, D=D, dtype=dtype)
    dev = upload(w)
    ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                  w.scale, w.dtype)
    for path, P in ((B.PA_PATH_V1, 0), (B.PA_PATH_V2, 64), (B.PA_PATH_V2, 256)):
        say(f"edge dtype={dtype} D={D} G={G} path={path} P={P}")
        out = run_path(w, dev, path, P if P else 512)
        got = to_f64(out)
        check_close(got, ref, f"edge {dtype} D={D} G={G} path={path} P={P}")
        assert np.all(got[0] == 0), "empty sequence must give 0"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("G", [1, 8])
def test_single_token_is_exact(dtype, G):
    """n = 1: the softmax weight is exactly 1, so out must equal V_0 bit for bit."""
    w = small_workload(7, [1, 1, 1], Hq=2 * G, Hkv=2, D=128, dtype=dtype)
    dev = upload(w)
    for path in (B.PA_PATH_V1, B.PA_PATH_V2):
        say(f"single token dtype={dtype} G={G} path={path}")
        got = run_path(w, dev, path, 512)
        expect = torch.stack([dev["v_cache"][int(w.block_tables[b, 0]), h // G, 0]
                              for b in range(3) for h in range(2 * G)]).view_as(got)
        assert torch.equal(got, expect)


def _relocate(w, seed):
    """Same logical KV, different physical blocks: a new permutation of the pool."""
    rng = np.random.default_rng(seed)
    NB = w.num_blocks
    perm = rng.permutation(NB)          # old physical id -> new physical id
    k = np.empty_like(w.k_cache)
    v = np.empty_like(w.v_cache)
    k[perm] = w.k_cache
    v[perm] = w.v_cache
    bt = perm[w.block_tables].astype(np.int32)
    w2 = wl.Workload(w.name, w.dtype, w.q, k, v, bt, w.context_lens, w.scale,
                     w.partition_sizes, int(perm[w.pad_block]), w.seed)
    return w2


@pytest.mark.parametrize("dtype,G", [("bf16", 8), ("f16", 4), ("f32", 4), ("bf16", 1)])
def test_block_placement_is_bitwise_invariant(dtype, G):
    ctx = [5000, 1, 777, 2048, 31]
    w = small_workload(11, ctx, Hq=4 * G, Hkv=4, D=128, dtype=dtype, pool_factor=1.5)
    w2 = _relocate(w, 99)
    for path in (B.PA_PATH_V1, B.PA_PATH_V2):
        say(f"placement dtype={dtype} G={G} path={path}")
        a = run_path(w, upload(w), path, 512)
        b = run_path(w2, upload(w2), path, 512)
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,G,D", [("bf16", 8, 128), ("f16", 8, 256), ("f32", 4, 128),
                                       ("bf16", 2, 128)])
def test_nan_poison_outside_context_is_never_read(dtype, G, D):
    ctx = [1000, 17, 530, 1]
    w = small_workload(12, ctx, Hq=2 * G, Hkv=2, D=D, dtype=dtype, pool_factor=1.5)
    clean = {path: run_path(w, upload(w), path, 512) for path in (B.PA_PATH_V1, B.PA_PATH_V2)}
    used = set(w.used_blocks())
    k, v = w.k_cache.copy(), w.v_cache.copy()
    nan = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]
    for blk in range(w.num_blocks):
        if blk not in used:
            k[blk] = nan
            v[blk] = nan
    for b, n in enumerate(ctx):       # tail slots of each sequence's last block
        nb = -(-n // 16)
        last = int(w.block_tables[b, nb - 1])
        k[last, :, n - (nb - 1) * 16:] = nan
        v[last, :, n - (nb - 1) * 16:] = nan
    wp = wl.Workload(w.name, w.dtype, w.q, k, v, w.block_tables, w.context_lens, w.scale,
                     w.partition_sizes, w.pad_block, w.seed)
    devp = upload(wp)
    for path in (B.PA_PATH_V1, B.PA_PATH_V2):
        say(f"poison dtype={dtype} G={G} D={D} path={path}")
        got = run_path(wp, devp, path, 512)
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, clean[path])


@pytest.mark.parametrize("dtype,G,D", [("bf16", 8, 128), ("f16", 8, 256), ("f32", 4, 128),
                                       ("bf16", 2, 128)])
def test_table_entries_past_the_context_are_never_dereferenced(dtype, G, D):
    """Block ids past each sequence's last block are fetched ahead of the context length
    but must never select a block: out-of-range ids there leave the output unchanged."""
    ctx = [1000, 17, 530, 1, 0, 520]
    w = small_workload(13, ctx, Hq=2 * G, Hkv=2, D=D, dtype=dtype, pool_factor=1.5)
    dev = upload(w)
    bt = w.block_tables.copy()
    junk = np.array([-1, 2**31 - 1, w.num_blocks, -2**31, 7 * w.num_blocks + 3], np.int32)
    for b, n in enumerate(ctx):
        nb = -(-n // 16)
        tail = bt.shape[1] - nb
        bt[b, nb:] = junk[np.arange(tail) % len(junk)]
    devj = dict(dev)
    devj["block_tables"] = torch.from_numpy(bt).to("cuda")
    for path, P in ((B.PA_PATH_V1, 512), (B.PA_PATH_V2, 512), (B.PA_PATH_V2, 64)):
        say(f"table junk dtype={dtype} G={G} D={D} path={path} P={P}")
        clean = run_path(w, dev, path, P)
        got = run_path(w, devj, path, P)
        assert torch.equal(got, clean)
    say(f"table junk dtype={dtype} G={G} D={D} split into 8 pieces")
    with work_split(8):
        clean = run_path(w, dev, B.PA_PATH_V2, 512)
        got = run_path(w, devj, B.PA_PATH_V2, 512)
    assert torch.equal(got, clean)


@pytest.mark.parametrize("S,dtype,G", [(300, "bf16", 8), (512, "f16", 4), (513, "bf16", 8)])
def test_v1_many_sequences_in_longest_first_order(S, dtype, G):
    """V1 over many sequences (from 256 (sequence, KV head) items up to 512 sequences,
    with contexts bounded above 1024 tokens, the work-groups take sequences longest
    context first; 513 is past that limit): parity with the oracle, ties and empty
    sequences included, and every sequence's rows bitwise equal to a decode of that
    sequence alone with the same kernel shape."""
    rng = np.random.default_rng(S)
    ctx = rng.integers(1, 1400, size=S)
    ctx[1] = 1399    # table bound > 1024 tokens
    ctx[::7] = 333   # ties
    ctx[3::11] = 0   # empty sequences
    ctx[5] = 1
    w = small_workload(40 + S, ctx.tolist(), Hq=2 * G, Hkv=2, D=128, dtype=dtype)
    dev = upload(w)
    ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                  w.scale, w.dtype)
    old = B.pa_get_mfma_variant()
    try:
        say(f"v1 order S={S} dtype={dtype} G={G}")
        out = run_path(w, dev, B.PA_PATH_V1, 512, variant=2)
        check_close(to_f64(out), ref, f"v1 order S={S}")
        assert torch.all(out[ctx == 0] == 0)
        for b in [0, 3, 5, 7, int(np.argmax(ctx)), int(np.argmin(ctx)), S // 2, S - 1]:
            say(f"v1 order S={S}: sequence {b} alone")
            q1 = dev["q"][b:b + 1].clone()  # fresh (16-byte aligned) single-sequence inputs
            one = torch.empty_like(q1)
            B.pa_decode_ex(one, q1, dev["k_cache"], dev["v_cache"],
                           dev["block_tables"][b:b + 1].clone(),
                           dev["context_lens"][b:b + 1].clone(), w.scale, 512,
                           path=B.PA_PATH_V1)
            torch.cuda.synchronize()
            assert torch.equal(one[0], out[b]), f"sequence {b}"
    finally:
        B.pa_set_mfma_variant(old)


@pytest.mark.parametrize("dtype,G,D,P", [("bf16", 8, 128, 512), ("f16", 8, 256, 256),
                                         ("bf16", 4, 128, 64), ("f32", 4, 128, 512),
                                         ("bf16", 2, 256, 256)])
def test_v2_compacted_order_matches_single_sequence_runs(dtype, G, D, P):
    """V2 over several sequences takes the non-empty (sequence, head, partition) items in a
    compacted order; every sequence's rows must be bitwise those of a V2 decode of that
    sequence alone (one sequence: grid order) with the same kernel shape (the automatic
    shape depends on the grid size), and empty sequences give exact zeros."""
    ctx = [3000, 0, 1, 700, 5000, 16, 0, 1033]
    w = small_workload(61 + D + P, ctx, Hq=2 * G, Hkv=2, D=D, dtype=dtype)
    dev = upload(w)
    ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                  w.scale, w.dtype)
    old = B.pa_get_mfma_variant()
    B.pa_set_mfma_variant(1)
    try:
        with work_split(0):
            say(f"v2 compacted dtype={dtype} G={G} D={D} P={P}")
            out = run_path(w, dev, B.PA_PATH_V2, P)
            check_close(to_f64(out), ref, f"v2 compacted P={P}")
            assert torch.all(out[np.asarray(ctx) == 0] == 0)
            for b in range(len(ctx)):
                q1 = dev["q"][b:b + 1].clone()
                one = torch.empty_like(q1)
                bt1 = dev["block_tables"][b:b + 1].clone()
                ws = torch.zeros(B.pa_workspace_bytes(q1, dev["k_cache"], bt1, 0, P),
                                 dtype=torch.uint8, device="cuda")
                B.pa_decode_ex(one, q1, dev["k_cache"], dev["v_cache"], bt1,
                               dev["context_lens"][b:b + 1].clone(), w.scale, P,
                               workspace=ws, path=B.PA_PATH_V2)
                torch.cuda.synchronize()
                assert torch.equal(one[0], out[b]), f"sequence {b}"
    finally:
        B.pa_set_mfma_variant(old)


def test_identity_coded_values_select_exact_rows():
    """fp32 V = physical_block*16 + slot, q = 0: out is the mean of the selected codes."""
    ctx = [1000, 333, 16, 1]
    w = small_workload(13, ctx, Hq=4, Hkv=1, D=128, dtype="f32", num_blocks=128)
    codes = (np.arange(128)[:, None] * 16 + np.arange(16)[None, :]).astype(np.float32)
    w.v_cache[...] = codes[:, None, :, None]
    w.q[...] = 0
    dev = upload(w)
    for path in (B.PA_PATH_V1, B.PA_PATH_V2):
        say(f"identity codes path={path}")
        got = to_f64(run_path(w, dev, path, 512))
        for b, n in enumerate(ctx):
            sel = [int(w.block_tables[b, t // 16]) * 16 + t % 16 for t in range(n)]
            np.testing.assert_allclose(got[b], np.mean(sel), rtol=2e-6)
            # a wrong block or slot would move the mean by at least 1/n
            assert np.abs(got[b] - np.mean(sel)).max() < 0.5 / n


@pytest.mark.parametrize("cfg", [1, 3, 4])
def test_runs_are_bitwise_deterministic(cfg):
    w, dev, _ = config_case(cfg)
    say(f"determinism {wl.CONFIG_NAMES[cfg]}")
    a = run_path(w, dev, B.PA_PATH_V2, 512)
    b = run_path(w, dev, B.PA_PATH_V2, 512)
    assert torch.equal(a, b)


def test_pa_decode_equals_its_two_phases():
    """pa_decode (library workspace, two launches) == pa_decode_ex V2 == pa_v2_partition +
    pa_v2_reduce, bit for bit with the work split off (the phase entry points never cut),
    and within tolerance of the oracle."""
    w, dev, ref = config_case(2)
    say("pa_decode vs pa_decode_ex vs the two phases on long_100k")
    out1 = torch.empty_like(dev["q"])
    with work_split(0), fused_mode(0):
        B.pa_decode(out1, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                    dev["context_lens"], w.scale, 512)
        out0 = run_path(w, dev, B.PA_PATH_V2, 512)
    lay = B.workspace_layout(dev["q"], dev["k_cache"], dev["block_tables"], 0, 512)
    ws = torch.empty(lay["bytes"], dtype=torch.uint8, device="cuda")
    out2 = torch.empty_like(dev["q"])
    B.pa_v2_partition(out2, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                      dev["context_lens"], w.scale, ws, 512)
    B.pa_v2_reduce(out2, dev["q"], dev["k_cache"], dev["block_tables"], dev["context_lens"], ws,
                   512)
    torch.cuda.synchronize()
    assert torch.equal(out1, out0)
    assert torch.equal(out1, out2)
    check_close(to_f64(out1), ref, "pa_decode long_100k")


def test_workspace_reuse_across_shapes():
    """One workspace, consecutive calls whose partition counts differ per sequence."""
    P = 64
    big = small_workload(41, [3000, 640, 65, 1, 0, 2000], Hq=16, Hkv=2, D=128, dtype="bf16",
                         max_blocks_per_seq=200)
    dev = upload(big)
    lay = B.workspace_layout(dev["q"], dev["k_cache"], dev["block_tables"], 0, P)
    ws = torch.empty(lay["bytes"], dtype=torch.uint8, device="cuda")
    for step, lens in enumerate(([3000, 640, 65, 1, 0, 2000], [100, 3199, 64, 700, 5, 1],
                                 [3200, 3200, 3200, 3200, 3200, 3200], [0, 0, 1, 0, 0, 17])):
        say(f"workspace reuse step {step} lens={lens}")
        ctx = np.array(lens, dtype=np.int32)
        ref = oracle.decode_attention(big.q, big.k_cache, big.v_cache, big.block_tables, ctx,
                                      big.scale, big.dtype)
        out = torch.empty_like(dev["q"])
        B.pa_decode_ex(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                       torch.from_numpy(ctx).cuda(), big.scale, P, workspace=ws,
                       path=B.PA_PATH_V2)
        torch.cuda.synchronize()
        check_close(to_f64(out), ref, f"reuse step {step}")


def test_context_hint_and_side_stream():
    """A context hint only trims idle work-groups: same bits as without it (work split
    off: the hint changes the item count, hence which items an automatic split cuts)."""
    w, dev, ref = config_case(3)
    say("context hint + side stream on batched_256")
    hint = int(w.context_lens.max())
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        auto = run_path(w, dev, B.PA_PATH_V2, 512, max_context_len=hint)
    s.synchronize()
    check_close(to_f64(auto), ref, "hinted, automatic split")
    with work_split(0):
        with torch.cuda.stream(s):
            out = run_path(w, dev, B.PA_PATH_V2, 512, max_context_len=hint)
        s.synchronize()
        check_close(to_f64(out), ref, "hinted")
        full = run_path(w, dev, B.PA_PATH_V2, 512)
    assert torch.equal(out, full)

