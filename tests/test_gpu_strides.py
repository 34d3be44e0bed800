"""Strided tensors at the C ABI (GPU): q and out as views into wider buffers (a fused QKV
projection output and a padded output buffer), the block table as a column slice of a
wider table, and K and V interleaved per cache block.

The callers of the decode op hand it views: its query is commonly a slice of the fused
QKV projection (project_6 commit 96f4baf page, V2 plan, integration note on the
_custom_ops.py / paged_attn.py call sites).  Each strided call is checked against the
float64 oracle and bitwise against the same call on dense copies (same kernels, same
launch shape), and the parts of the buffers outside the views must be left untouched.
"""
import sys

import numpy as np
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


def strided_views(dev, D):
    """Views of the dense device tensors in wider buffers (copies of the same values)."""
    q, k, v, bt = dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"]
    S, Hq, _ = q.shape
    NB, Hkv = k.shape[0], k.shape[1]
    # q inside a fused [S, (Hq + 2 Hkv) * D] projection output, the rest junk
    qkv = torch.full((S, (Hq + 2 * Hkv) * D), 3.0e4, dtype=q.dtype, device=q.device)
    qkv[:, :Hq * D] = q.reshape(S, Hq * D)
    qv = qkv[:, :Hq * D].unflatten(1, (Hq, D))
    # out inside [S, Hq + 3, D], starting at head 1
    obuf = torch.full((S, Hq + 3, D), 7.0, dtype=q.dtype, device=q.device)
    ov = obuf[:, 1:Hq + 1]
    # K and V interleaved per block: [NB, 2, Hkv, 16, D]
    kv = torch.empty((NB, 2, Hkv, 16, D), dtype=k.dtype, device=k.device)
    kv[:, 0] = k
    kv[:, 1] = v
    # the table as columns 3 .. 3 + MB of a wider table (4-byte aligned start)
    MB = bt.shape[1]
    wide = torch.full((S, MB + 7), -5, dtype=torch.int32, device=bt.device)
    wide[:, 3:3 + MB] = bt
    return qv, ov, obuf, kv[:, 0], kv[:, 1], wide[:, 3:3 + MB]


CASES = [
    # (name, context lens, Hq, Hkv, D, dtype)
    ("bf16-g8-d128", [3000, 17, 1, 700, 0], 32, 4, 128, "bf16"),
    ("f16-g8-d256", [1200, 513, 64], 16, 2, 256, "f16"),
    ("f32-g4-d128", [900, 5], 4, 1, 128, "f32"),
    ("bf16-g2-d128", [640, 33], 4, 2, 128, "bf16"),
]


@pytest.mark.parametrize("name,ctx,Hq,Hkv,D,dtype", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("path,P", [(B.PA_PATH_AUTO, 512), (B.PA_PATH_V1, 512),
                                    (B.PA_PATH_V2, 512), (B.PA_PATH_V2, 256)],
                         ids=["auto", "v1", "v2-P512", "v2-P256"])
def test_strided_views_match_dense(name, ctx, Hq, Hkv, D, dtype, path, P):
    w = small_workload(31, ctx, Hq, Hkv, D, dtype)
    dev = upload(w)
    ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                  w.scale, w.dtype)
    say(f"strides {name} path={path} P={P}")
    qv, ov, obuf, kv_k, kv_v, btv = strided_views(dev, D)
    nbytes = B.pa_workspace_bytes(dev["q"], dev["k_cache"], dev["block_tables"], 0, P)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    B.pa_decode_ex(ov, qv, kv_k, kv_v, btv, dev["context_lens"], w.scale, P, workspace=ws,
                   path=path)
    dense = torch.empty_like(dev["q"])
    B.pa_decode_ex(dense, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                   dev["context_lens"], w.scale, P, workspace=ws, path=path)
    torch.cuda.synchronize()
    check_close(to_f64(ov), ref, f"strided {name}")
    assert torch.equal(ov.contiguous().view(torch.int16 if dtype != "f32" else torch.int32),
                       dense.view(torch.int16 if dtype != "f32" else torch.int32)), \
        "strided and dense calls differ"
    assert torch.all(obuf[:, 0] == 7.0) and torch.all(obuf[:, Hq + 1:] == 7.0), \
        "out buffer written outside the view"


def test_pa_decode_with_fused_qkv_view():
    """pa_decode (library workspace, automatic path) on the 8K-token shape with q a view
    into the fused QKV output."""
    w = small_workload(32, [8192], 32, 4, 128, "bf16")
    dev = upload(w)
    ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                  w.scale, w.dtype)
    qv, ov, obuf, kv_k, kv_v, btv = strided_views(dev, 128)
    say("strides pa_decode 8192 tokens")
    B.pa_decode(ov, qv, kv_k, kv_v, btv, dev["context_lens"], w.scale, 512)
    torch.cuda.synchronize()
    check_close(to_f64(ov), ref, "pa_decode strided")
