"""Seeded precision sweep of the matrix-core decode path against the float64 oracle.

Inputs are N(0, 1) in the storage type (q, K and V), contexts of 2 to 199 tokens,
the head groups and head dims the matrix-core kernel is built for, and two scales:
the pages' 1/sqrt(head_dim) (project_6 optimizations/prefix_prefill_patch.py
docstring: head_dim 128, 256 less often) and 0.3, which makes the softmax peaky (a
few keys carry most of the weight, the regime where the rounding of the
probabilities matters most).  Each combination runs 10 sequences in one call, on
the automatic path (one partition: V1) and on forced V2 with 64- and 128-token
partitions (several partitions, phase 2, and at 128 tokens the work split into
64-token pieces).  240 (sequence) cases per path, all at the tolerance for
fp16/bf16 KV with fp32 accumulation: |gpu - ref| <= 2e-3 + 1e-2 |ref| element-wise
and a per-(sequence, head) relative L2 error <= 1e-2.
"""
import itertools
import math
import sys

import numpy as np
import pytest

import oracle
from paged_split_kv_pa_amd import binding as B

from helpers import check_close, small_workload, to_f64, upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

COMBOS = list(itertools.product((128, 256), ("bf16", "f16"), (4, 8, 16), ("pages", "0.3")))
NUM_SEQS = 10
HKV = 2


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _case(D, dtype, G, scale_kind):
    seed = 1000 + COMBOS.index((D, dtype, G, scale_kind))
    scale = 1.0 / math.sqrt(D) if scale_kind == "pages" else 0.3
    w = small_workload(seed, None, G * HKV, HKV, D, dtype, scale=scale,
                       context_lens_fn=lambda rng: rng.integers(2, 200, size=NUM_SEQS))
    ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                  w.scale, w.dtype)
    return w, ref


@pytest.mark.parametrize("D,dtype,G,scale_kind", COMBOS,
                         ids=[f"D{d}-{t}-G{g}-scale_{s}" for d, t, g, s in COMBOS])
def test_precision_sweep(D, dtype, G, scale_kind):
    w, ref = _case(D, dtype, G, scale_kind)
    dev = upload(w)
    say(f"precision D={D} {dtype} G={G} scale={w.scale:.4f} ctx={list(map(int, w.context_lens))}")
    runs = [("auto", B.PA_PATH_AUTO, 512), ("v2-P64", B.PA_PATH_V2, 64),
            ("v2-P128", B.PA_PATH_V2, 128)]
    for name, path, P in runs:
        out = torch.empty_like(dev["q"])
        nbytes = B.pa_workspace_bytes(dev["q"], dev["k_cache"], dev["block_tables"], 0, P)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        B.pa_decode_ex(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                       dev["context_lens"], w.scale, P, workspace=ws, path=path)
        torch.cuda.synchronize()
        got = to_f64(out)
        err, rel = check_close(got, ref, f"D={D} {dtype} G={G} scale={w.scale} {name}")
        say(f"  {name}: max_abs_err={err:.3e} row_rel_l2={rel:.3e}")
