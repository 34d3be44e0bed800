"""pa_prefill's two PV forms on the GPU (see pa_set_prefill_mode).

Mode 0 (default) feeds P and V to the matrix cores as fp16; bf16 V is converted when it
is staged, and a value beyond fp16's range (|v| >= 65536) makes a second launch recompute
the call in mode 1's form (P as a 16-bit high plus low part, V unconverted).  Checked
here against the float64 oracle at the decode tolerance: mode 1 on its own; bf16 V with
values just inside fp16's range (no recompute: the result differs from mode 1's) and
beyond it, in the cached prefix and in the new tokens (recompute: bitwise mode 1's
result); values beyond the range in rows no query sees (cache slots past a prefix: not
read, no recompute); and a captured graph replayed while V changes between the two
cases (every replay correct).  The inputs are the pages' prefill shapes (prefix_prefill
kernel docstring in project_6 optimizations/prefix_prefill_patch.py: GQA, head_dim 128
and 256) at small sizes, N(0, 1) values with a few large ones planted in distinct
head-dim columns, so that no column cancels two large values.
"""
import dataclasses
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


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    with prefill_mode(0):
        yield


def upload(w):
    d = {n: to_device(getattr(w, n), w.dtype) for n in ("q", "k_new", "v_new", "k_cache",
                                                          "v_cache")}
    for n in ("block_tables", "context_lens", "query_start"):
        d[n] = torch.from_numpy(np.ascontiguousarray(getattr(w, n), dtype=np.int32)).cuda()
    return d


def run(w, dev, out=None):
    if out is None:
        out = torch.empty_like(dev["q"])
    B.pa_prefill(out, dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                 dev["block_tables"], dev["context_lens"], dev["query_start"], w.scale)
    torch.cuda.synchronize()
    return out


def reference(w):
    return oracle.prefill_attention(w.q, w.k_new, w.v_new, w.k_cache, w.v_cache,
                                    w.block_tables, w.context_lens, w.query_start, w.scale,
                                    w.dtype)


def check_rows(got, ref, what):
    check_close(got.reshape(1, -1, got.shape[-1]), ref.reshape(1, -1, ref.shape[-1]), what)


def bf16_bits(x):
    return wl.to_storage(np.array([x], dtype=np.float32), "bf16")[0]


def base(seed, D=128, G=4, dtype="bf16"):
    return wl.make_prefill_workload("modes", seed, context_lens=[70, 0, 200],
                                    query_lens=[40, 90, 33], num_q_heads=2 * G,
                                    num_kv_heads=2, head_dim=D, dtype=dtype)


def plant(w, where, value):
    """Copy of w with `value` (bf16) at six (key, head-dim column) places of V: in the
    cached prefix of sequence 2 (where="cache"), in the new tokens (where="new"), or in
    cache slots past sequence 0's 70-token prefix (where="past": read by no query)."""
    vc, vn = w.v_cache.copy(), w.v_new.copy()
    val = bf16_bits(value)
    D = w.head_dim
    for n in range(6):
        col = (37 * n + 5) % D
        if where == "cache":
            key = 31 * n + 3  # < 200
            blk = w.block_tables[2, key // 16]
            vc[blk, n % 2, key % 16, col] = val
        elif where == "new":
            row = int(w.query_start[1]) + 13 * n  # sequence 1's new tokens
            vn[row, n % 2, col] = val
        else:
            key = 70 + n  # slots 70..75 of the block holding key 70 (block 4 of 16 tokens)
            blk = w.block_tables[0, key // 16]
            vc[blk, n % 2, key % 16, col] = val
    return dataclasses.replace(w, v_cache=vc, v_new=vn)


TWO = [(D, dt, sc) for D in (128, 256) for dt in ("bf16", "f16") for sc in (None, 0.3)]


@pytest.mark.parametrize("D,dtype,scale", TWO,
                         ids=[f"D{d}-{t}-scale_{s or 'pages'}" for d, t, s in TWO])
def test_mode1_matches_oracle(D, dtype, scale):
    w = wl.make_prefill_workload("mode1", 3100 + TWO.index((D, dtype, scale)),
                                 context_lens=[0, 17, 130, 64], query_lens=[5, 70, 40, 129],
                                 num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=dtype,
                                 scale=scale)
    say(f"prefill mode 1 D={D} {dtype} scale={w.scale:.4f}")
    dev = upload(w)
    with prefill_mode(1):
        got = run(w, dev)
    check_rows(to_f64(got), reference(w), f"mode 1 D={D} {dtype}")


@pytest.mark.parametrize("D", (128, 256))
@pytest.mark.parametrize("where", ("cache", "new"))
def test_bf16_values_beyond_fp16_are_recomputed(D, where):
    w = plant(base(3200 + D, D), where, 70000.0)
    say(f"prefill bf16 |v| = 70000 in {where}, D={D}")
    dev = upload(w)
    got = run(w, dev)
    check_rows(to_f64(got), reference(w), f"|v| 70000 in {where}")
    with prefill_mode(1):
        two = run(w, dev)
    assert torch.equal(got, two), "the recompute launch must leave mode 1's result"


@pytest.mark.parametrize("value", (65280.0, -65280.0, 1.0e30))
def test_bf16_extremes(value):
    """65280 (the largest bf16 below 65536) fits fp16: no recompute, so the result is
    mode 0's own, not mode 1's.  1e30 does not fit: the recompute gives mode 1's result.
    (Values near fp32's limit are out of reach of both forms: the lazy rescale lets a
    probability reach 2^8 before O is rescaled, and O accumulates in fp32.)"""
    w = plant(base(3300, 128), "cache", value)
    say(f"prefill bf16 v = {value:g}")
    dev = upload(w)
    got = run(w, dev)
    ref = reference(w)
    check_rows(to_f64(got), ref, f"v {value:g}")
    with prefill_mode(1):
        two = run(w, dev)
    if abs(value) < 65536:
        assert not torch.equal(got, two), "one-part result expected (no recompute)"
    else:
        assert torch.equal(got, two), "recompute expected"


def test_values_beyond_fp16_in_unread_slots_change_nothing():
    w = base(3400, 128)
    dev = upload(w)
    want = run(w, dev)
    w2 = plant(w, "past", 1.0e30)
    say("prefill bf16 |v| = 1e30 in cache slots past a prefix")
    got = run(w2, upload(w2))
    assert torch.equal(got, want)


def test_graph_replays_follow_the_values():
    """A captured bf16 prefill replayed while v_new alternates between N(0, 1) values and
    values beyond fp16: every replay matches the oracle for the values it saw."""
    w = base(3500, 128)
    w_big = plant(w, "new", -90000.0)
    dev = upload(w)
    v_small = dev["v_new"].clone()
    v_big = to_device(w_big.v_new, "bf16")
    refs = {"small": reference(w), "big": reference(w_big)}
    out = torch.empty_like(dev["q"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def call():
        B.pa_prefill(out, dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                     dev["block_tables"], dev["context_lens"], dev["query_start"], w.scale,
                     stream=s)

    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for i, kind in enumerate(("small", "big", "small", "big", "big", "small")):
        dev["v_new"].copy_(v_small if kind == "small" else v_big)
        out.fill_(7.0)
        torch.cuda.synchronize()
        say(f"prefill graph replay {i} ({kind} values)")
        g.replay()
        torch.cuda.synchronize()
        check_rows(to_f64(out), refs[kind], f"replay {i} ({kind})")
