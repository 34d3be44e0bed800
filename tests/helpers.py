"""Helpers shared by the GPU tests: device upload of seeded workloads and the
tolerance check against the float64 oracle."""
import contextlib
import numpy as np

from paged_split_kv_pa_amd import workloads as wl

# Tolerance for fp16/bf16 KV with fp32 accumulation: |gpu - ref| <= ATOL + RTOL*|ref|
# element-wise, plus a relative L2 bound per (sequence, head) so that a near-zero output
# cannot pass on the absolute term alone.
ATOL = 2e-3
RTOL = 1e-2
ROW_REL_L2 = 1e-2


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_device(arr, dtype, device="cuda"):
    """Storage array (see workloads) -> device tensor of the matching torch dtype."""
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def upload(w, device="cuda"):
    import torch
    return {
        "q": to_device(w.q, w.dtype, device),
        "k_cache": to_device(w.k_cache, w.dtype, device),
        "v_cache": to_device(w.v_cache, w.dtype, device),
        "block_tables": torch.from_numpy(w.block_tables).to(device),
        "context_lens": torch.from_numpy(w.context_lens).to(device),
    }


def to_f64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check_close(got, ref, what=""):
    """Raise AssertionError with a summary when got (GPU) misses ref (oracle)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} elements outside tolerance; worst at {idx}: "
                             f"got {got[idx]!r} ref {ref[idx]!r}")
    num = np.linalg.norm((got - ref).reshape(-1, ref.shape[-1]), axis=-1)
    den = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=-1)
    rel = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    assert rel.max() <= ROW_REL_L2, f"{what}: row relative L2 error {rel.max():.3e}"
    return float(err.max()), float(rel.max())


def small_workload(seed, ctx, Hq, Hkv, D, dtype, **kw):
    return wl.make_workload("case", seed, context_lens=ctx, num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim=D, dtype=dtype, **kw)


@contextlib.contextmanager
def fused_mode(mode):
    """Run the block with the library's single-launch setting changed, then restore it."""
    from paged_split_kv_pa_amd import binding as B
    old = B.pa_get_fused()
    B.pa_set_fused(mode)
    try:
        yield
    finally:
        B.pa_set_fused(old)


@contextlib.contextmanager
def prefill_mode(mode):
    """Run the block with the library's prefill PV form changed, then restore it."""
    from paged_split_kv_pa_amd import binding as B
    old = B.pa_get_prefill_mode()
    B.pa_set_prefill_mode(mode)
    try:
        yield
    finally:
        B.pa_set_prefill_mode(old)


@contextlib.contextmanager
def work_split(pieces, first_item=0):
    """Run the block with the library's work-split setting changed, then restore it."""
    from paged_split_kv_pa_amd import binding as B
    old = B.pa_get_work_split()
    B.pa_set_work_split(pieces, first_item)
    try:
        yield
    finally:
        B.pa_set_work_split(*old)
