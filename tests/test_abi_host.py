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

import split_rule

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
    # out, q, k_cache, v_cache: 16 bytes; block_tables, context_lens: 4 bytes
    for i in range(4):
        ptrs = list(FAKE)
        ptrs[i] = ctypes.c_void_p(0x10008)
        assert decode(dims(), ptrs) == -4
    for i in (4, 5):
        ptrs = list(FAKE)
        ptrs[i] = ctypes.c_void_p(0x10002)
        assert decode(dims(), ptrs) == -4


# Strides (elements; dims(): S=2, Hq=32, Hkv=4, D=128, MB=8, bf16).  pa_choose_path
# validates the dims like every decode entry point and makes no HIP call.
@pytest.mark.parametrize("kw,status", [
    (dict(q_stride_dim=2), B.PA_ERR_STRIDE),                 # innermost stride must be 1
    (dict(out_stride_dim=3), B.PA_ERR_STRIDE),
    (dict(out_stride_head=64), B.PA_ERR_STRIDE),             # out heads overlap (D = 128)
    (dict(out_stride_seq=31 * 128), B.PA_ERR_STRIDE),        # out sequences overlap
    (dict(kv_stride_block=4 * 16 * 128 - 8), B.PA_ERR_STRIDE),  # shorter than a block
    (dict(bt_stride_seq=4), B.PA_ERR_STRIDE),                # shorter than a table row
    (dict(q_stride_head=-128), B.PA_ERR_STRIDE),
    (dict(q_stride_head=132), -4),                          # 264-byte rows: misaligned
    (dict(out_stride_seq=32 * 128 + 4), -4),
    (dict(kv_stride_block=4 * 16 * 128 + 4), -4),
    (dict(q_stride_seq=1 << 31), -6),                       # beyond the kernels' 32 bits
])
def test_stride_validation(kw, status):
    assert B.lib().pa_choose_path(ctypes.byref(dims(**kw)), 0, 512) == status
    assert B.pa_last_error()
    assert decode(dims(**kw)) == status


@pytest.mark.parametrize("kw", [
    dict(q_stride_seq=(32 + 8) * 128, q_stride_head=128, q_stride_dim=1),  # fused QKV view
    dict(out_stride_seq=40 * 128, out_stride_head=128),
    dict(q_stride_head=0, q_stride_seq=0, out_stride_dim=1),   # 0 = row-major
    dict(kv_stride_block=2 * 4 * 16 * 128),                     # K and V interleaved per block
    dict(bt_stride_seq=100),                                    # column slice of a wider table
    dict(q_stride_head=64, q_stride_seq=128),                   # overlapping q rows: allowed
])
def test_valid_strides_pass_validation(kw):
    assert B.lib().pa_choose_path(ctypes.byref(dims(**kw)), 0, 512) in (B.PA_PATH_V1,
                                                                       B.PA_PATH_V2)


def test_nonfinite_scale():
    assert decode(dims(), scale=float("inf")) == -3
    assert decode(dims(), scale=float("nan")) == -3


def test_empty_batch_is_a_no_op():
    # S = 0: nothing to do, no pointer is needed and no HIP call is made.
    nul = [ctypes.c_void_p(0)] * 6
    assert decode(dims(num_seqs=0), nul) == 0


def layout(d, hint, P):
    v = (ctypes.c_int64 * B.LAYOUT_FIELDS)()
    assert B.lib().pa_workspace_layout(ctypes.byref(d), hint, P, v) == 0
    return list(v)


def test_workspace_bytes_layout():
    d = dims(num_seqs=3, max_blocks_per_seq=100)  # capacity 1600 tokens, 4 KV heads
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # (hint, P, Pmax, piece slots): pieces are multiples of 64 tokens, at most 16, so
    # P = 512 cuts into up to 8 pieces, 1024 into 16, 64 and 96 not at all; slots =
    # min(1024, items * pieces).
    for hint, P, pmax, slots in ((0, 512, 4, 384), (513, 512, 2, 192), (16, 512, 1, 96),
                                 (0, 16, 100, 0), (0, 96, 17, 0), (64, 64, 1, 0),
                                 (0, 64, 25, 0), (0, 256, 7, 336), (0, 128, 13, 312),
                                 (0, 1024, 2, 384)):
        assert split_rule.piece_slots(3 * 4 * pmax, P) == slots
        rows = 3 * 32 * pmax
        off_max = a256(rows * 128 * 4)
        off_sum = off_max + a256(rows * 4)
        off_pout = off_sum + a256(rows * 4)
        off_pmax = off_pout + a256(slots * 8 * 128 * 4)
        off_psum = off_pmax + a256(slots * 8 * 4)
        total = off_psum + a256(slots * 8 * 4)
        assert layout(d, hint, P) == [pmax, 0, off_max, off_sum, slots, off_pout, off_pmax,
                                      off_psum, total]
        assert B.lib().pa_workspace_bytes(ctypes.byref(d), hint, P) == total
    # Invalid: hint above capacity, bad partition size, NULL output.
    assert B.lib().pa_workspace_bytes(ctypes.byref(d), 1601, 512) == 0
    assert B.lib().pa_workspace_bytes(ctypes.byref(d), 0, 24) == 0
    v = (ctypes.c_int64 * B.LAYOUT_FIELDS)()
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
        # Measured MI355X rule (default): V1 iff the bound is <= 256 tokens or S*Hkv >= 256.
        B.pa_set_v1_max_context(-5)
        assert B.pa_get_v1_max_context() == -1
        one = dims(num_seqs=1, num_kv_heads=4, max_blocks_per_seq=512)            # 8192 tokens
        assert B.pa_choose_path(one, 0, 512) == B.PA_PATH_V2
        assert B.pa_choose_path(one, 256, 512) == B.PA_PATH_V1                    # short
        assert B.pa_choose_path(one, 257, 512) == B.PA_PATH_V2
        assert B.pa_choose_path(one, 512, 512) == B.PA_PATH_V2                    # one partition
        assert B.pa_choose_path(one, 1024, 1024) == B.PA_PATH_V2
        wide = dims(num_seqs=64, num_kv_heads=4, max_blocks_per_seq=6250)         # 256 KV heads
        assert B.pa_choose_path(wide, 0, 512) == B.PA_PATH_V1
        narrow = dims(num_seqs=63, num_kv_heads=4, max_blocks_per_seq=6250)       # 252
        assert B.pa_choose_path(narrow, 0, 512) == B.PA_PATH_V2
    finally:
        B.pa_set_v1_max_context(old)


def test_mfma_variant_knob():
    old = B.pa_get_mfma_variant()
    try:
        for v in (0, 1, 2, 3, -1):
            B.pa_set_mfma_variant(v)
            assert B.pa_get_mfma_variant() == v
        for bad in (4, -2):
            with pytest.raises(B.PaError):
                B.pa_set_mfma_variant(bad)
    finally:
        B.pa_set_mfma_variant(old)


def test_work_split_knob():
    old = B.pa_get_work_split()
    try:
        for pieces, first in ((-1, 0), (0, 0), (1, 3), (2, 0), (4, 7), (8, 1 << 40), (16, 5)):
            B.pa_set_work_split(pieces, first)
            assert B.pa_get_work_split() == (pieces, first)
        for bad in (3, -2, 32, 6):
            with pytest.raises(B.PaError):
                B.pa_set_work_split(bad, 0)
        with pytest.raises(B.PaError):
            B.pa_set_work_split(4, -1)
        assert B.pa_get_work_split() == (16, 5)  # a rejected call changes nothing
    finally:
        B.pa_set_work_split(*old)


def split_plan(d, hint, P):
    v = (ctypes.c_int64 * 4)()
    st = B.lib().pa_split_plan(ctypes.byref(d), hint, P, v)
    return st, list(v)


@pytest.mark.parametrize("S,Hkv,MB,hint,P,pieces,first", [
    (1, 4, 6250, 0, 512, 8, 768),       # long context: cut the 16 tail items
    (1, 4, 6250, 0, 512, 16, 768),      # P = 512 allows at most 8 pieces
    (1, 4, 6250, 0, 512, 8, 0),         # every item: only the last 128 fit 1024 slots
    (1, 4, 6250, 0, 1024, 16, 0),       # P = 1024: 16 pieces of 64 tokens
    (2, 8, 513, 0, 512, 4, 200),        # cut starts inside a (sequence, head) row
    (3, 4, 100, 0, 512, 8, 0),
    (3, 4, 100, 0, 256, 16, 0),         # P = 256 allows at most 4 pieces
    (3, 4, 100, 0, 128, 16, 0),         # P = 128: 2 pieces of 64 tokens
    (3, 4, 100, 0, 64, 2, 0),           # P = 64 cannot be cut
    (3, 4, 100, 0, 96, 4, 0),           # P = 96 is not a multiple of 64
    (3, 4, 100, 0, 16, 2, 0),
    (3, 4, 100, 0, 512, 2, 1000),       # first beyond the items: no cut
    (1, 1, 4, 0, 512, 16, 0),
])
def test_split_plan_fixed_pieces(S, Hkv, MB, hint, P, pieces, first):
    old = B.pa_get_work_split()
    try:
        B.pa_set_work_split(pieces, first)
        d = dims(num_seqs=S, num_q_heads=8 * Hkv, num_kv_heads=Hkv, max_blocks_per_seq=MB)
        st, got = split_plan(d, hint, P)
        assert st == 0, B.pa_last_error()
        pmax = -(-(hint if hint > 0 else MB * 16) // P)
        items = S * Hkv * pmax
        assert got == [items, *split_rule.plan(items, P, pieces, first)]
        assert got[3] <= (1 << 24)
        if got[2] > 1:
            assert (items - got[1]) * got[2] <= layout(d, hint, P)[4]  # fits the slots
        B.pa_set_work_split(0, 0)
        assert split_plan(d, hint, P)[1] == [items, items, 1, items]
    finally:
        B.pa_set_work_split(*old)


def test_split_rule_examples():
    # The automatic rule on 256 compute units.
    assert split_rule.plan(784, 512, -1, ncu=256) == (768, 8, 896)     # 100K tokens, 4 KV heads
    assert split_rule.plan(768, 512, -1, ncu=256) == (768, 1, 768)     # balanced already
    assert split_rule.plan(832, 512, -1, ncu=256) == (768, 4, 1024)    # remainder 64
    assert split_rule.plan(896, 512, -1, ncu=256) == (768, 2, 1024)    # remainder 128
    assert split_rule.plan(960, 512, -1, ncu=256) == (960, 1, 960)     # remainder 192 > 128
    assert split_rule.plan(868, 512, -1, ncu=256) == (768, 8, 1568)    # 100: no multiple
    assert split_rule.plan(64, 512, -1, ncu=256) == (0, 8, 512)        # 8K tokens, 4 KV heads
    assert split_rule.plan(128, 512, -1, ncu=256) == (0, 4, 512)       # 16K tokens
    assert split_rule.plan(200, 512, -1, ncu=256) == (0, 2, 400)
    assert split_rule.plan(2, 512, -1, ncu=256) == (0, 8, 16)
    assert split_rule.plan(64, 64, -1, ncu=256) == (64, 1, 64)         # P = 64: no pieces
    assert split_rule.plan(8192, 512, -1, ncu=256) == (8192, 1, 8192)  # 32 per CU
    assert split_rule.plan(257, 256, -1, ncu=256) == (256, 4, 260)     # P = 256: at most 4


def test_split_plan_automatic_needs_a_device():
    old = B.pa_get_work_split()
    try:
        B.pa_set_work_split(-1, 0)
        st, got = split_plan(dims(num_seqs=1, max_blocks_per_seq=6250), 0, 512)
        assert st in (0, -8)  # -8 (PA_ERR_HIP) where no device is visible
        if st == 0:
            assert got[0] == 784 and got[3] >= 784
    finally:
        B.pa_set_work_split(*old)


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
    assert lay["slots"] == split_rule.piece_slots(3 * 4 * 4, 512) == 384
    assert lay["piece_out"][1] == (384, 8, 128)
    assert lay["piece_sum"][0] + 384 * 8 * 4 <= lay["bytes"]


def test_copy_blocks_validation():
    lib = B.lib()
    K, V, PR = FAKE[0], FAKE[1], FAKE[2]
    assert lib.pa_copy_blocks(None, None, 4096, 10, None, 0, None) == 0  # no pairs: no-op
    for bb in (0, -16, 24, 1 << 31):
        assert lib.pa_copy_blocks(K, V, bb, 10, PR, 1, None) == -3
    assert lib.pa_copy_blocks(K, V, 4096, 0, PR, 1, None) == -3
    assert lib.pa_copy_blocks(K, V, 4096, 10, PR, -1, None) == -3
    assert lib.pa_copy_blocks(None, V, 4096, 10, PR, 1, None) == -1
    assert lib.pa_copy_blocks(K, V, 4096, 10, None, 1, None) == -1
    assert lib.pa_copy_blocks(ctypes.c_void_p(0x10008), V, 4096, 10, PR, 1, None) == -4
    assert lib.pa_copy_blocks(K, ctypes.c_void_p(0x10008), 4096, 10, PR, 1, None) == -4
    assert lib.pa_copy_blocks(K, V, 4096, 10, ctypes.c_void_p(0x10002), 1, None) == -4
    assert "block_pairs" in B.pa_last_error()


def pdims(**kw):
    d = dict(num_seqs=2, num_tokens=100, num_q_heads=32, num_kv_heads=4, head_dim=128,
             block_size=16, num_blocks=64, max_blocks_per_seq=8, dtype=B.PA_BF16,
             max_query_len=0)
    d.update(kw)
    return B.PaPrefillDims(**d)


PF_FAKE = [ctypes.c_void_p(0x20000 + 0x1000 * i) for i in range(9)]


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=9), -2),
    (dict(num_seqs=-1), -3),
    (dict(num_tokens=-1), -3),
    (dict(num_q_heads=30), -3),
    (dict(num_blocks=0), -3),
    (dict(max_query_len=101), -3),
    (dict(dtype=B.PA_F32), -6),
    (dict(head_dim=64), -6),
    (dict(head_dim=192), -6),
    (dict(block_size=32), -6),
    (dict(num_q_heads=96, num_kv_heads=4), -6),   # G = 24
    (dict(num_kv_heads=70000, num_q_heads=70000), -6),
    (dict(max_blocks_per_seq=(1 << 26) - 1, num_tokens=(1 << 30) + 100), -6),  # > 2^31 keys
])
def test_prefill_validation(kw, status):
    st = B.lib().pa_prefill(ctypes.byref(pdims(**kw)), *PF_FAKE, 0.1, None)
    assert st == status, B.pa_last_error()


def test_prefill_pointers_and_empty_calls():
    lib = B.lib()
    assert lib.pa_prefill(None, *PF_FAKE, 0.1, None) == -1
    for i in range(9):
        ptrs = list(PF_FAKE)
        ptrs[i] = ctypes.c_void_p(0)
        assert lib.pa_prefill(ctypes.byref(pdims()), *ptrs, 0.1, None) == -1
    ptrs = list(PF_FAKE)
    ptrs[1] = ctypes.c_void_p(0x20008)  # q misaligned
    assert lib.pa_prefill(ctypes.byref(pdims()), *ptrs, 0.1, None) == -4
    ptrs = list(PF_FAKE)
    ptrs[8] = ctypes.c_void_p(0x20002)  # query_start misaligned
    assert lib.pa_prefill(ctypes.byref(pdims()), *ptrs, 0.1, None) == -4
    assert lib.pa_prefill(ctypes.byref(pdims()), *PF_FAKE, float("nan"), None) == -3
    nul = [ctypes.c_void_p(0)] * 9
    assert lib.pa_prefill(ctypes.byref(pdims(num_tokens=0)), *nul, 0.1, None) == 0
    assert lib.pa_prefill(ctypes.byref(pdims(num_seqs=0)), *nul, 0.1, None) == 0


def test_prefill_mode_knob():
    old = B.pa_get_prefill_mode()
    try:
        for m in (1, 0):
            B.pa_set_prefill_mode(m)
            assert B.pa_get_prefill_mode() == m
        for bad in (-1, 2):
            with pytest.raises(B.PaError):
                B.pa_set_prefill_mode(bad)
        assert B.pa_get_prefill_mode() == 0
    finally:
        B.pa_set_prefill_mode(old)


def test_prefill_split_knob():
    old = B.pa_get_prefill_split()
    try:
        for v in (0, 4, 16, 1 << 20, -1):
            B.pa_set_prefill_split(v)
            assert B.pa_get_prefill_split() == v
        for bad in (-2, 1, 2, 3, (1 << 20) + 1):
            with pytest.raises(B.PaError):
                B.pa_set_prefill_split(bad)
        assert B.pa_get_prefill_split() == -1
    finally:
        B.pa_set_prefill_split(old)


def test_prefill_workspace_bytes_without_a_device():
    """Calls that cannot take the planned schedule need no workspace, and that is decided
    without the device; calls that can need the compute-unit count (PA_ERR_HIP here if no
    device is visible)."""
    lib = B.lib()
    old_split, old_mode = B.pa_get_prefill_split(), B.pa_get_prefill_mode()
    try:
        small = pdims(max_blocks_per_seq=8, num_tokens=64)  # <= 16 tiles per row block
        assert lib.pa_prefill_workspace_bytes(ctypes.byref(small)) == 0
        big = pdims(max_blocks_per_seq=4096, num_tokens=4096)
        r = lib.pa_prefill_workspace_bytes(ctypes.byref(big))
        assert r == -8 or r > 320 * 1024
        B.pa_set_prefill_split(0)
        assert lib.pa_prefill_workspace_bytes(ctypes.byref(big)) == 0
        B.pa_set_prefill_split(-1)
        B.pa_set_prefill_mode(1)
        assert lib.pa_prefill_workspace_bytes(ctypes.byref(big)) == 0
        assert lib.pa_prefill_workspace_bytes(None) == -1
        assert lib.pa_prefill_workspace_bytes(ctypes.byref(pdims(head_dim=64))) == -6
    finally:
        B.pa_set_prefill_split(old_split)
        B.pa_set_prefill_mode(old_mode)


def test_prefill_ex_validation_without_a_device():
    lib = B.lib()
    nul = [ctypes.c_void_p(0)] * 9
    # empty calls need nothing
    assert lib.pa_prefill_ex(ctypes.byref(pdims(num_seqs=0)), *nul, 0.1, None, 0, None) == 0
    assert lib.pa_prefill_ex(None, *PF_FAKE, 0.1, None, 0, None) == -1
    assert lib.pa_prefill_ex(ctypes.byref(pdims()), *PF_FAKE, float("inf"), None, 0, None) == -3
