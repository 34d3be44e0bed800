"""pa_prefill's planned schedule on the GPU (see pa_set_prefill_split).

A plan kernel cuts long row blocks' key ranges into chunks, the prefill kernel takes the
items longest first, and a merge kernel folds each cut row block's chunks with the
log-sum-exp rule (the combination rule of the pages' Phase 2, project_6 commit 96f4baf
page, V2 plan, applied to key ranges of one prefill row block).  Checked against the
float64 oracle at the decode tolerance: automatic chunks on the bench workloads and on a
short chunk after a long prefix (the case the plan is for); fixed small chunks (4 to 16
tiles) on ragged shapes at every group size and both head dims, including chunks that
start inside the causal part; more than 512 row blocks; several hundred sequences; 513
sequences (beyond the plan: the grid schedule); results independent of the rest of the
batch with a fixed chunk length (bitwise); the schedule off; a captured graph replayed;
bf16 values beyond fp16 in a cut row block (the two-part recompute)."""
import contextlib
import sys

import numpy as np
import pytest

import oracle
from paged_split_kv_pa_amd import binding as B
from paged_split_kv_pa_amd import workloads as wl

from helpers import check_close, prefill_mode, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@contextlib.contextmanager
def split(chunk):
    old = B.pa_get_prefill_split()
    B.pa_set_prefill_split(chunk)
    try:
        yield
    finally:
        B.pa_set_prefill_split(old)


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    with prefill_mode(0), split(-1):
        yield


def upload(w):
    d = {n: to_device(getattr(w, n), w.dtype) for n in ("q", "k_new", "v_new", "k_cache",
                                                          "v_cache")}
    for n in ("block_tables", "context_lens", "query_start"):
        d[n] = torch.from_numpy(np.ascontiguousarray(getattr(w, n), dtype=np.int32)).cuda()
    return d


def run(w, dev, out=None, stream=None):
    if out is None:
        out = torch.empty_like(dev["q"])
    B.pa_prefill(out, dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                 dev["block_tables"], dev["context_lens"], dev["query_start"], w.scale,
                 stream=stream)
    torch.cuda.synchronize()
    return out


def reference(w):
    return oracle.prefill_attention(w.q, w.k_new, w.v_new, w.k_cache, w.v_cache,
                                    w.block_tables, w.context_lens, w.query_start, w.scale,
                                    w.dtype)


def check_rows(got, ref, what):
    check_close(got.reshape(1, -1, got.shape[-1]), ref.reshape(1, -1, ref.shape[-1]), what)


def test_batch_mixed_automatic():
    w = wl.prefill_config(2)
    say(f"planned prefill {w.name}")
    check_rows(to_f64(run(w, upload(w))), reference(w), "pf_batch_mixed planned")


def test_short_chunk_after_long_prefix():
    """One sequence, 100 new tokens after a 20000-token prefix: 4 row blocks per KV head
    of ~315 tiles each, cut into chunks over the whole chip."""
    w = wl.make_prefill_workload("short_after_long", 3600, context_lens=[20000],
                                 query_lens=[100], num_q_heads=32, num_kv_heads=4,
                                 head_dim=128, dtype="bf16")
    say("planned prefill: 100 tokens after 20000")
    check_rows(to_f64(run(w, upload(w))), reference(w), "short after long")


FIXED = [(G, D, dt, ch) for G, D, dt, ch in
         [(1, 128, "bf16", 4), (2, 128, "f16", 5), (4, 128, "bf16", 8), (8, 128, "f16", 4),
          (16, 128, "bf16", 16), (1, 256, "f16", 4), (4, 256, "bf16", 6), (16, 256, "f16", 4)]]


@pytest.mark.parametrize("G,D,dtype,chunk", FIXED,
                         ids=[f"G{g}-D{d}-{t}-c{c}" for g, d, t, c in FIXED])
def test_fixed_chunks_ragged(G, D, dtype, chunk):
    """Chunks of at most `chunk` tiles: with 1-2 query heads per KV head a row block holds
    128-256 positions, so the last chunk of a row block starts inside the causal part and
    some rows see none of its keys."""
    ctx = [0, 1, 700, 64, 1500, 300, 0]
    ql = [1, 300, 17, 520, 65, 129, 640]
    w = wl.make_prefill_workload("fixed", 3700 + G + D, context_lens=ctx, query_lens=ql,
                                 num_q_heads=2 * G, num_kv_heads=2, head_dim=D, dtype=dtype)
    say(f"planned prefill fixed chunks {chunk} G={G} D={D} {dtype} T={w.num_tokens}")
    with split(chunk):
        got = run(w, upload(w))
    check_rows(to_f64(got), reference(w), f"fixed chunks {chunk} G={G} D={D}")


def test_rows_independent_of_the_batch():
    """With a fixed chunk length every row block is cut the same way in any batch, so each
    sequence's rows equal a prefill of that sequence alone, bitwise."""
    w = wl.prefill_config(2)
    dev = upload(w)
    with split(24):
        batch = run(w, dev)
        qs = np.asarray(w.query_start)
        for b in range(len(w.context_lens)):
            r0, r1 = int(qs[b]), int(qs[b + 1])
            say(f"planned prefill {w.name}: sequence {b} alone")
            one = {n: dev[n][r0:r1].clone() for n in ("q", "k_new", "v_new")}
            one["k_cache"], one["v_cache"] = dev["k_cache"], dev["v_cache"]
            one["block_tables"] = dev["block_tables"][b:b + 1].clone()
            one["context_lens"] = dev["context_lens"][b:b + 1].clone()
            one["query_start"] = torch.tensor([0, r1 - r0], dtype=torch.int32, device="cuda")
            assert torch.equal(run(w, one), batch[r0:r1]), f"sequence {b}"
    check_rows(to_f64(batch), reference(w), "fixed 24 batch")


@pytest.mark.parametrize("S", (300, 513))
def test_many_sequences(S):
    """300 sequences (the plan, with ranks over all of them) and 513 (past the plan's
    512: the grid schedule)."""
    rng = np.random.default_rng(3800 + S)
    ctx = [int(x) for x in rng.integers(0, 3000, size=S)]
    ql = [int(x) for x in rng.integers(0, 40, size=S)]
    ctx[7], ql[7] = 6000, 33  # one long row block among short ones
    w = wl.make_prefill_workload("many", 3800 + S, context_lens=ctx, query_lens=ql,
                                 num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="f16")
    say(f"planned prefill {S} sequences T={w.num_tokens}")
    with split(8):
        got = run(w, upload(w))
    check_rows(to_f64(got), reference(w), f"{S} sequences")


@pytest.mark.parametrize("chunk", (16, -1), ids=("c16", "auto"))
def test_more_than_512_row_blocks(chunk):
    """Two sequences whose chunks hold 519 + 40 row blocks of 16 positions (16 query heads
    per KV head): the plan kernel's per-row-block loops, the tile total among them, run in
    two rounds of its 512 threads.  Sampled (row, head) outputs against the oracle's causal
    rows, one at a time."""
    ctx, ql = [300, 5000], [8300, 640]
    w = wl.make_prefill_workload("rb", 3900, context_lens=ctx, query_lens=ql, num_q_heads=16,
                                 num_kv_heads=1, head_dim=128, dtype="bf16")
    say(f"planned prefill {sum(-(-n // 16) for n in ql)} row blocks chunk {chunk}")
    with split(chunk):
        got = to_f64(run(w, upload(w)))
    from oracle.storage import upcast
    rng = np.random.default_rng(3901)
    q, kn, vn = upcast(w.q, w.dtype), upcast(w.k_new, w.dtype), upcast(w.v_new, w.dtype)
    s = float(np.float32(w.scale))
    picks = [(0, 0), (0, 8299), (1, 0), (1, 639)] + [
        (int(b), int(rng.integers(0, ql[int(b)]))) for b in rng.integers(0, 2, 40)]
    ref, gs = [], []
    for b, i in picks:
        c, r0 = ctx[b], int(w.query_start[b])
        kp = upcast(oracle.gather_sequence(w.k_cache, w.block_tables, b, c), w.dtype)[:, 0]
        vp = upcast(oracle.gather_sequence(w.v_cache, w.block_tables, b, c), w.dtype)[:, 0]
        h = int(rng.integers(0, 16))
        ka = np.concatenate([kp, kn[r0:r0 + i + 1, 0]])
        va = np.concatenate([vp, vn[r0:r0 + i + 1, 0]])
        ref.append(oracle.prefill_rows(q[r0 + i:r0 + i + 1, h], ka, va, c + i, s)[0])
        gs.append(got[r0 + i, h])
    check_close(np.array(gs)[None], np.array(ref)[None], f"{len(picks)} sampled rows, chunk {chunk}")


def test_off_matches_oracle_and_planned_agrees():
    w = wl.make_prefill_workload("off", 3900, context_lens=[5000, 40], query_lens=[200, 300],
                                 num_q_heads=16, num_kv_heads=2, head_dim=128, dtype="bf16")
    dev = upload(w)
    ref = reference(w)
    say("prefill, schedule off and automatic")
    with split(0):
        off = run(w, dev)
    check_rows(to_f64(off), ref, "schedule off")
    with split(4):
        cut = run(w, dev)
    check_rows(to_f64(cut), ref, "chunks of 4")


def test_graph_replays():
    w = wl.make_prefill_workload("graph", 3950, context_lens=[9000, 100], query_lens=[64, 500],
                                 num_q_heads=32, num_kv_heads=4, head_dim=128, dtype="bf16")
    dev = upload(w)
    with split(8):
        eager = run(w, dev)
        out = torch.empty_like(dev["q"])
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run(w, dev, out=out, stream=s)  # warm-up on the capture stream: workspace exists
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            B.pa_prefill(out, dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"],
                         dev["v_cache"], dev["block_tables"], dev["context_lens"],
                         dev["query_start"], w.scale, stream=s)
        for i in range(4):
            out.fill_(3.0)
            torch.cuda.synchronize()
            say(f"planned prefill graph replay {i}")
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {i}"
            run(w, dev)  # an eager call between replays
    check_rows(to_f64(eager), reference(w), "graph workload")


def test_bf16_beyond_fp16_in_a_cut_row_block():
    w = wl.make_prefill_workload("ovf", 3990, context_lens=[4000], query_lens=[40],
                                 num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16")
    vc = w.v_cache.copy()
    big = wl.to_storage(np.array([80000.0], dtype=np.float32), "bf16")[0]
    for n in range(4):
        key = 1000 * n + 17
        vc[w.block_tables[0, key // 16], n % 2, key % 16, 11 * n + 3] = big
    import dataclasses
    w = dataclasses.replace(w, v_cache=vc)
    dev = upload(w)
    say("planned prefill, bf16 V beyond fp16 in a cut row block")
    with split(8):
        got = run(w, dev)
    check_rows(to_f64(got), reference(w), "overflow recompute")
    with prefill_mode(1):
        two = run(w, dev)
    assert torch.equal(got, two)


def test_caller_workspace_matches_library_workspace():
    """pa_prefill_ex with a zeroed workspace of pa_prefill_workspace_bytes: bitwise the
    library-workspace result, twice in a row (the counters are left at zero); a workspace
    one byte short is refused."""
    w = wl.prefill_config(2)
    dev = upload(w)
    want = run(w, dev)
    nbytes = B.pa_prefill_workspace_bytes(dev["q"], dev["k_new"], dev["k_cache"],
                                          dev["block_tables"], dev["context_lens"])
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for i in range(2):
        say(f"pa_prefill_ex call {i} ({nbytes} bytes of workspace)")
        out = torch.empty_like(dev["q"])
        B.pa_prefill(out, dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                     dev["block_tables"], dev["context_lens"], dev["query_start"], w.scale,
                     workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"call {i}"
    with pytest.raises(B.PaError) as e:
        B.pa_prefill(torch.empty_like(dev["q"]), dev["q"], dev["k_new"], dev["v_new"],
                     dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                     dev["query_start"], w.scale, workspace=ws[:nbytes - 1])
    assert e.value.status == -7


def test_decode_and_prefills_overlap_on_three_streams():
    """A decode (library workspace) and two prefills (one on the library's prefill
    workspace, one on a caller workspace) enqueued on three streams with no waits between
    them: every result bitwise equal to the same call made alone."""
    from helpers import small_workload, upload as upload_decode
    wd = small_workload(3970, [60000, 7000], 32, 4, 128, "bf16")
    ddev = upload_decode(wd)
    w1 = wl.prefill_config(2)
    w2 = wl.make_prefill_workload("overlap", 3971, context_lens=[12000, 300], query_lens=[70, 400],
                                  num_q_heads=32, num_kv_heads=4, head_dim=128, dtype="bf16")
    d1, d2 = upload(w1), upload(w2)

    def decode(out, stream=None):
        B.pa_decode(out, ddev["q"], ddev["k_cache"], ddev["v_cache"], ddev["block_tables"],
                    ddev["context_lens"], wd.scale, 512, stream=stream)

    alone_d = torch.empty_like(ddev["q"])
    decode(alone_d)
    alone_1 = run(w1, d1)
    nbytes = B.pa_prefill_workspace_bytes(d2["q"], d2["k_new"], d2["k_cache"],
                                          d2["block_tables"], d2["context_lens"])
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    alone_2 = torch.empty_like(d2["q"])
    B.pa_prefill(alone_2, d2["q"], d2["k_new"], d2["v_new"], d2["k_cache"], d2["v_cache"],
                 d2["block_tables"], d2["context_lens"], d2["query_start"], w2.scale, workspace=ws)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(3):
        say(f"decode + two prefills on three streams, round {rep}")
        od, o1, o2 = torch.empty_like(alone_d), torch.empty_like(alone_1), torch.empty_like(alone_2)
        torch.cuda.synchronize()
        decode(od, stream=streams[0])
        B.pa_prefill(o1, d1["q"], d1["k_new"], d1["v_new"], d1["k_cache"], d1["v_cache"],
                     d1["block_tables"], d1["context_lens"], d1["query_start"], w1.scale,
                     stream=streams[1])
        B.pa_prefill(o2, d2["q"], d2["k_new"], d2["v_new"], d2["k_cache"], d2["v_cache"],
                     d2["block_tables"], d2["context_lens"], d2["query_start"], w2.scale,
                     stream=streams[2], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(od, alone_d), "decode"
        assert torch.equal(o1, alone_1), "prefill on the library workspace"
        assert torch.equal(o2, alone_2), "prefill on the caller workspace"
