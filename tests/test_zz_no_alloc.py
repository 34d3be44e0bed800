"""pa_decode_noalloc (the allocation-free decode entry point) against pa_decode.

Two calls in a row through the C ABI, the second with a smaller input, each compared with
pa_decode (same path rule, same kernels: bitwise equal), and, like pa_decode_ex on a
caller workspace, with the float64 oracle at the fp16/bf16 tolerance.  The static scratch keeps the first call's
contents, which must not leak into the second.  A call whose workspace would exceed the
scratch is refused on the host with PA_ERR_WORKSPACE.
"""
import sys

import pytest

import oracle
from paged_split_kv_pa_amd import binding as B

from helpers import check_close, small_workload, to_f64, upload

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


def _run_both(w, P):
    dev = upload(w)
    ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                  w.scale, w.dtype)
    need = B.pa_workspace_bytes(dev["q"], dev["k_cache"], dev["block_tables"], 0, P)
    assert need <= B.NOALLOC_SCRATCH_BYTES
    got = torch.full_like(dev["q"], 5.0)
    B.pa_decode_noalloc(got, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                        dev["context_lens"], w.scale, P)
    want = torch.empty_like(dev["q"])
    B.pa_decode(want, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                dev["context_lens"], w.scale, P)
    two = torch.empty_like(dev["q"])
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    B.pa_decode_ex(two, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                   dev["context_lens"], w.scale, P, workspace=ws)
    torch.cuda.synchronize()
    check_close(to_f64(got), ref, "pa_decode_noalloc")
    check_close(to_f64(two), ref, "pa_decode_ex")
    # same path and kernels as pa_decode (single launch where it applies): same bits
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), \
        "pa_decode_noalloc and pa_decode differ"


def test_two_calls_second_smaller():
    # 1: several long and short sequences, V2 with a work split (bf16, GQA 8, head_dim 128)
    w1 = small_workload(41, [20000, 3000, 517, 1, 0, 9000], 32, 4, 128, "bf16")
    say("noalloc call 1: 6 sequences up to 20000 tokens, bf16 G8 D128, P=512")
    _run_both(w1, 512)
    # 2: a smaller input (fewer, shorter sequences; fp16, head_dim 256, partition 256)
    w2 = small_workload(42, [1500, 300], 16, 2, 256, "f16", sigma=0.5)
    say("noalloc call 2: 2 sequences up to 1500 tokens, f16 G8 D256, P=256")
    _run_both(w2, 256)


def test_oversized_call_is_refused_on_the_host():
    # S=16, Hq=32, head_dim 256, 65536-token table rows: the V2 workspace would be
    # 16*32*128*256*4 bytes (64 MiB) plus statistics, above the scratch.  Validation
    # happens before any launch, so small tensors with a wide block table suffice.
    S, Hq, Hkv, D, MB = 16, 32, 4, 256, 4096
    q = torch.zeros(S, Hq, D, dtype=torch.float16, device="cuda")
    k = torch.zeros(4, Hkv, 16, D, dtype=torch.float16, device="cuda")
    bt = torch.zeros(S, MB, dtype=torch.int32, device="cuda")
    ctx = torch.ones(S, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    assert B.pa_workspace_bytes(q, k, bt, 0, 512) > B.NOALLOC_SCRATCH_BYTES
    say("noalloc oversized call (host-side refusal)")
    with pytest.raises(B.PaError) as e:
        B.pa_decode_noalloc(out, q, k, k, bt, ctx, 0.0625, 512)
    assert e.value.status == -7 and "static scratch" in str(e.value)
