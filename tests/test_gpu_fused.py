"""Single-launch V2 (GPU): phase 1 and the log-sum-exp merge in one grid.

pa_decode with the library's workspace runs the "Phase 1" partials and the "Phase 2"
merge (project_6 commit 96f4baf page, V2 plan) in one launch: merge work-groups of the
same grid wait for every partition of their (sequence, KV head), counted by arrival
counters that the launch leaves at zero.  Checked here: the oracle's tolerance on the
workloads and on ragged, empty and short sequences, forced work splits (which put
early-exit and empty-piece work-groups in the count), the vector-ALU kernel, many calls
in a row over changing shapes (a counter left non-zero would stall a later merge until
its wall-clock limit and show as NaN), bitwise determinism, and agreement with the
two-launch path.
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
    with fused_mode(1):  # the single launch is opt-in
        yield


def reference(w):
    return oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                   w.scale, w.dtype)


def decode(dev, w, P):
    out = torch.full_like(dev["q"], 9.0)
    B.pa_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                dev["context_lens"], w.scale, P)
    torch.cuda.synchronize()
    return out


def bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def check_fused(w, P, what, expect_fused=True):
    dev = upload(w)
    applies = B.pa_fused_applies(dev["q"], dev["k_cache"], dev["block_tables"], P)
    assert applies == expect_fused, f"{what}: single launch {'not ' if expect_fused else ''}taken"
    ref = reference(w)
    a = decode(dev, w, P)
    b = decode(dev, w, P)
    check_close(to_f64(a), ref, what)
    assert torch.equal(bits(a), bits(b)), f"{what}: runs differ"
    with fused_mode(0):
        two = decode(dev, w, P)
    check_close(to_f64(two), ref, what + " (two launches)")
    return a


@pytest.mark.parametrize("cfg,P", [(1, 512), (2, 512), (4, 512), (4, 256)],
                         ids=["single_8k", "long_100k", "mixed_d256-P512", "mixed_d256-P256"])
def test_workloads(cfg, P):
    w = wl.config(cfg)
    say(f"single launch {wl.CONFIG_NAMES[cfg]} P={P}")
    check_fused(w, P, f"{wl.CONFIG_NAMES[cfg]} P={P}")


SHAPES = [
    # (name, contexts, Hq, Hkv, D, dtype, P, max_blocks_per_seq)
    ("ragged-empty-bf16", [0, 1, 15, 513, 40000, 0, 2048], 32, 4, 128, "bf16", 512, None),
    ("short-than-table-f16-d256", [9000, 3000], 16, 2, 256, "f16", 256, 1200),
    ("valu-f32-g4", [60000], 4, 1, 128, "f32", 512, None),
    ("valu-bf16-g2", [30000, 5000], 8, 4, 128, "bf16", 512, None),
    ("g16-bf16", [70000], 32, 2, 128, "bf16", 512, None),
]


@pytest.mark.parametrize("name,ctx,Hq,Hkv,D,dtype,P,MB", SHAPES, ids=[s[0] for s in SHAPES])
def test_shapes(name, ctx, Hq, Hkv, D, dtype, P, MB):
    w = small_workload(51, ctx, Hq, Hkv, D, dtype, max_blocks_per_seq=MB,
                       sigma=0.5 if dtype == "f16" else 1.0)
    say(f"single launch {name}")
    check_fused(w, P, name)


@pytest.mark.parametrize("pieces", [2, 4, 16])
def test_forced_splits(pieces):
    """Every item cut from item 5 on: pieces past a short context and partitions past a
    sequence's last one exit early and must still be counted."""
    w = small_workload(52, [33000, 700, 12000], 32, 4, 128, "bf16", max_blocks_per_seq=2500)
    say(f"single launch, split {pieces} from item 5")
    with work_split(pieces, 5):
        check_fused(w, 512, f"split {pieces}")


def test_many_calls_leave_the_counters_at_zero():
    """Twelve calls in a row over four shapes (different (sequence, KV head) counts and
    expected arrivals); every result checked."""
    shapes = [small_workload(60 + i, ctx, Hq, Hkv, 128, "bf16")
              for i, (ctx, Hq, Hkv) in enumerate([([50000], 32, 4), ([20000, 9000, 0], 32, 4),
                                                  ([70000], 16, 2), ([40000, 1], 32, 8)])]
    devs = [upload(w) for w in shapes]
    refs = [reference(w) for w in shapes]
    for i in range(12):
        k = (i * 3) % 4
        say(f"single launch call {i} shape {k}")
        got = decode(devs[k], shapes[k], 512)
        check_close(to_f64(got), refs[k], f"call {i} shape {k}")


def test_setting_off_gives_two_launches():
    w = wl.config(2)
    dev = upload(w)
    with fused_mode(0):
        assert not B.pa_fused_applies(dev["q"], dev["k_cache"], dev["block_tables"], 512)
    assert B.pa_fused_applies(dev["q"], dev["k_cache"], dev["block_tables"], 512)
    with pytest.raises(B.PaError):
        B.pa_set_fused(-1)


def test_noalloc_single_launch_matches_pa_decode():
    """pa_decode_noalloc takes the single launch too (its static scratch holds the
    counters): bitwise equal to pa_decode, two calls in a row."""
    for seed, ctx in ((70, [50000, 3000]), (71, [40000])):
        w = small_workload(seed, ctx, 32, 4, 128, "bf16")
        dev = upload(w)
        assert B.pa_fused_applies(dev["q"], dev["k_cache"], dev["block_tables"], 512)
        say(f"single launch pa_decode_noalloc ctx={ctx}")
        got = torch.empty_like(dev["q"])
        B.pa_decode_noalloc(got, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                            dev["context_lens"], w.scale, 512)
        want = decode(dev, w, 512)
        check_close(to_f64(got), reference(w), "pa_decode_noalloc single launch")
        assert torch.equal(bits(got), bits(want))


def test_graph_replays():
    """A captured single-launch step replayed five times, with eager calls of another
    shape in between: every replay equals the eager result (the counters and flags the
    launch leaves at zero make each replay start clean)."""
    w = small_workload(72, [60000], 32, 4, 128, "bf16")
    other = small_workload(73, [30000, 100], 32, 4, 128, "bf16")
    dev, dev2 = upload(w), upload(other)
    eager = decode(dev, w, 512)
    out = torch.empty_like(dev["q"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream (workspace allocated here)
        B.pa_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                    dev["context_lens"], w.scale, 512, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.pa_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                    dev["context_lens"], w.scale, 512, stream=s)
    ref2 = reference(other)
    for i in range(5):
        say(f"single launch graph replay {i}")
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(eager)), f"replay {i} differs from the eager call"
        check_close(to_f64(decode(dev2, other, 512)), ref2, f"eager call after replay {i}")
