"""Host-side tests of the C ABI (no GPU needed).

The library must load and export every entry point that include/pa_decode.h
declares, and every validation error must be reported before any HIP call,
so bad arguments are forced from the host here.  Fake device pointers are
never dereferenced: each call below fails validation first.
"""
import ctypes
import os
import re

import pytest

from paged_split_kv_pa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa_decode.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(pa_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("pa_decode", "pa_decode_ex", "pa_workspace_bytes", "pa_v2_partition",
              "pa_v2_reduce", "pa_v1", "pa_choose_path", "pa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in pa_decode.h but not exported"
    assert set(declared_functions()) == set(B.SIGNATURES), "binding and header disagree"


def test_version(lib):
    assert "gfx950" in B.pa_version()


def dims(**kw):
    d = dict(num_seqs=2, num_q_heads=32, num_kv_heads=4, head_dim=128, block_size=16,
             num_blocks=64, max_blocks_per_seq=8, dtype=B.PA_BF16)
    d.update(kw)
    return B.PaDims(**d)


FAKE = [ctypes.c_void_p(0x10000 + 0x1000 * i) for i in range(6)]  # aligned, never read


def decode(d, ptrs=None, scale=0.1, P=512, lib=None):
    ptrs = FAKE if ptrs is None else ptrs
    return B.lib().pa_decode(ctypes.byref(d), *ptrs, scale, P, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), -2),
    (dict(num_q_heads=30), -3),
    (dict(num_kv_heads=0), -3),
    (dict(num_seqs=-1), -3),
    (dict(num_blocks=0), -3),
    (dict(max_blocks_per_seq=0), -3),
    (dict(head_dim=64), -6),
    (dict(block_size=32), -6),
    (dict(num_q_heads=24, num_kv_heads=8), -6),   # G = 3
    (dict(num_q_heads=64, num_kv_heads=2), -6),   # G = 32
    (dict(max_blocks_per_seq=1 << 27), -6),
])
def test_dims_validation(kw, status):
    assert decode(dims(**kw)) == status
    assert B.pa_last_error()


@pytest.mark.parametrize("P", [0, -16, 8, 500, 100])
def test_partition_size_validation(P):
    assert decode(dims(), P=P) == -5
    assert "partition_size" in B.pa_last_error()


def test_null_pointers():
    for i in range(6):
        ptrs = list(FAKE)
        ptrs[i] = ctypes.c_void_p(0)
        assert decode(dims(), ptrs) == -1
    assert B.lib().pa_decode(None, *FAKE, 0.1, 512, None) == -1


def test_misaligned_pointer():
    ptrs = list(FAKE)
    ptrs[1] = ctypes.c_void_p(0x10008)
    assert decode(dims(), ptrs) == -4


def test_nonfinite_scale():
    assert decode(dims(), scale=float("inf")) == -3
    assert decode(dims(), scale=float("nan")) == -3


def test_empty_batch_is_a_no_op():
    # S = 0: nothing to do, no pointer is needed and no HIP call is made.
    nul = [ctypes.c_void_p(0)] * 6
    assert decode(dims(num_seqs=0), nul) == 0


def layout(d, hint, P):
    v = (ctypes.c_int64 * 5)()
    assert B.lib().pa_workspace_layout(ctypes.byref(d), hint, P, v) == 0
    return list(v)


def test_workspace_bytes_layout():
    d = dims(num_seqs=3, max_blocks_per_seq=100)  # capacity 1600 tokens
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for hint, P, pmax in ((0, 512, 4), (513, 512, 2), (0, 16, 100)):
        rows = 3 * 32 * pmax
        off_max = a256(rows * 128 * 4)
        off_sum = off_max + a256(rows * 4)
        total = off_sum + a256(rows * 4)
        assert layout(d, hint, P) == [pmax, 0, off_max, off_sum, total]
        assert B.lib().pa_workspace_bytes(ctypes.byref(d), hint, P) == total
    # Invalid: hint above capacity, bad partition size, NULL output.
    assert B.lib().pa_workspace_bytes(ctypes.byref(d), 1601, 512) == 0
    assert B.lib().pa_workspace_bytes(ctypes.byref(d), 0, 24) == 0
    v = (ctypes.c_int64 * 5)()
    assert B.lib().pa_workspace_layout(ctypes.byref(d), 0, 24, v) == -5
    assert B.lib().pa_workspace_layout(ctypes.byref(d), 0, 512, None) == -1


def test_long_context_partition_grid():
    # 100000 tokens at P = 512: 196 partitions (tests/golden/partition_counts.txt).
    d = dims(num_seqs=1, max_blocks_per_seq=6250)
    assert layout(d, 0, 512)[0] == 196


def test_workspace_required_for_v2():
    d = dims()
    lib = B.lib()
    st = lib.pa_decode_ex(ctypes.byref(d), *FAKE, 0.1, 512, None, None, 0, 0, B.PA_PATH_V2)
    assert st == -7
    need = lib.pa_workspace_bytes(ctypes.byref(d), 0, 512)
    st = lib.pa_decode_ex(ctypes.byref(d), *FAKE, 0.1, 512, None, ctypes.c_void_p(0x80000),
                          need - 1, 0, B.PA_PATH_V2)
    assert st == -7
    st = lib.pa_decode_ex(ctypes.byref(d), *FAKE, 0.1, 512, None, None, 0, 0, 5)
    assert st == -3


def test_hint_above_capacity_rejected():
    d = dims(max_blocks_per_seq=8)
    st = B.lib().pa_decode_ex(ctypes.byref(d), *FAKE, 0.1, 512, None, None, 0, 129, B.PA_PATH_V1)
    assert st == -3


def test_v2_phase_entry_points_validate():
    d = dims()
    lib = B.lib()
    assert lib.pa_v2_partition(ctypes.byref(d), *FAKE, 0.1, 512, 0, None, 0, None) == -7
    assert lib.pa_v2_reduce(ctypes.byref(d), FAKE[0], FAKE[5], 512, 0, None, 0, None) == -7
    assert lib.pa_v2_reduce(ctypes.byref(d), None, FAKE[5], 512, 0, ctypes.c_void_p(0x80000),
                            1 << 30, None) == -1
    assert lib.pa_v2_partition(ctypes.byref(d), *FAKE, 0.1, 100, 0, None, 0, None) == -5
    assert lib.pa_v1(ctypes.byref(dims(head_dim=96)), *FAKE, 0.1, 0, None) == -6


def test_too_many_partitions():
    d = dims(max_blocks_per_seq=(8192 * 512) // 16 + 16)
    assert decode(d, P=512) == -6


def test_num_partitions_golden():
    path = os.path.join(ROOT, "tests", "golden", "partition_counts.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    for n, P, _full, _last, total in rows:
        assert B.pa_num_partitions(int(n), int(P)) == int(total)
    assert B.pa_num_partitions(0, 512) == 0
    assert B.pa_num_partitions(-1, 512) == -1
    assert B.pa_num_partitions(10, 0) == -1


def test_path_rules():
    old = B.pa_get_v1_max_context()
    try:
        # Pages' rule (project_6 commit a2a5dd8 page): V1 iff the context bound <= 8192.
        B.pa_set_v1_max_context(8192)
        assert B.pa_get_v1_max_context() == 8192
        assert B.pa_choose_path(dims(max_blocks_per_seq=512)) == B.PA_PATH_V1      # 8192
        assert B.pa_choose_path(dims(max_blocks_per_seq=513)) == B.PA_PATH_V2      # 8208
        assert B.pa_choose_path(dims(max_blocks_per_seq=6250)) == B.PA_PATH_V2
        assert B.pa_choose_path(dims(max_blocks_per_seq=6250), 4000) == B.PA_PATH_V1
        B.pa_set_v1_max_context(0)
        assert B.pa_choose_path(dims(max_blocks_per_seq=1)) == B.PA_PATH_V2
        # Measured MI355X rule (default): V1 iff one partition or S*Hkv >= 256.
        B.pa_set_v1_max_context(-5)
        assert B.pa_get_v1_max_context() == -1
        one = dims(num_seqs=1, num_kv_heads=4, max_blocks_per_seq=512)            # 8192 tokens
        assert B.pa_choose_path(one, 0, 512) == B.PA_PATH_V2
        assert B.pa_choose_path(one, 512, 512) == B.PA_PATH_V1                    # one partition
        assert B.pa_choose_path(one, 513, 512) == B.PA_PATH_V2
        assert B.pa_choose_path(one, 1024, 1024) == B.PA_PATH_V1
        wide = dims(num_seqs=64, num_kv_heads=4, max_blocks_per_seq=6250)         # 256 KV heads
        assert B.pa_choose_path(wide, 0, 512) == B.PA_PATH_V1
        narrow = dims(num_seqs=63, num_kv_heads=4, max_blocks_per_seq=6250)       # 252
        assert B.pa_choose_path(narrow, 0, 512) == B.PA_PATH_V2
    finally:
        B.pa_set_v1_max_context(old)


def test_mfma_variant_knob():
    old = B.pa_get_mfma_variant()
    try:
        for v in (0, 1, 2, -1):
            B.pa_set_mfma_variant(v)
            assert B.pa_get_mfma_variant() == v
        for bad in (3, -2):
            with pytest.raises(B.PaError):
                B.pa_set_mfma_variant(bad)
    finally:
        B.pa_set_mfma_variant(old)


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 128)
    k = torch.zeros(4, 1, 16, 128)
    with pytest.raises(B.PaError):
        B.pa_decode(q.clone(), q, k, k, torch.zeros(1, 4, dtype=torch.int32),
                    torch.ones(1, dtype=torch.int32), 0.1)


def test_workspace_layout_helper_matches_library():
    torch = pytest.importorskip("torch")
    q = torch.zeros(3, 32, 128, dtype=torch.bfloat16)
    k = torch.zeros(64, 4, 16, 128, dtype=torch.bfloat16)
    bt = torch.zeros(3, 100, dtype=torch.int32)
    lay = B.workspace_layout(q, k, bt, 0, 512)
    d = B.dims_of(q, k, bt)
    assert lay["bytes"] == B.lib().pa_workspace_bytes(ctypes.byref(d), 0, 512)
