"""Thin Python binding of libpa_decode.so (the C ABI in include/pa_decode.h).

Argument marshalling only: torch tensors are turned into device pointers and
a ``pa_dims_t``; every step of the computation runs in the library's HIP
kernels.  The functions keep the C names.  There is no fallback: if the
library is missing or a call fails, a ``PaError`` is raised.

Tensors (all on the same CUDA/HIP device):
  q, out           [S, Hq, D]        float32 / float16 / bfloat16; any sequence and head
                                     strides (e.g. views into a fused QKV buffer), head-dim
                                     stride 1
  k_cache, v_cache [NB, Hkv, 16, D]  same dtype as q; each block [Hkv, 16, D] dense, any
                                     (common) block stride
  block_tables     [S, MB]           int32; any row stride, entries contiguous
  context_lens     [S]               int32, contiguous
The strides travel in pa_dims_t; the library validates them (PA_ERR_STRIDE, PA_ERR_ALIGN).
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libpa_decode.so")

PA_OK = 0
STATUS_NAMES = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_DTYPE", -3: "PA_ERR_SHAPE",
                -4: "PA_ERR_ALIGN", -5: "PA_ERR_PARTITION", -6: "PA_ERR_UNSUPPORTED",
                -7: "PA_ERR_WORKSPACE", -8: "PA_ERR_HIP", -9: "PA_ERR_INTERNAL",
                -10: "PA_ERR_STRIDE"}
PA_ERR_STRIDE = -10
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_PATH_AUTO, PA_PATH_V1, PA_PATH_V2 = 0, 1, 2


class PaError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


class PaDims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("q_stride_seq", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
                ("q_stride_dim", ctypes.c_int64), ("out_stride_seq", ctypes.c_int64),
                ("out_stride_head", ctypes.c_int64), ("out_stride_dim", ctypes.c_int64),
                ("kv_stride_block", ctypes.c_int64), ("bt_stride_seq", ctypes.c_int64)]


class PaPrefillDims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("max_query_len", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_DIMS = ctypes.POINTER(PaDims)

# name -> (restype, argtypes); mirrors include/pa_decode.h
SIGNATURES = {
    "pa_decode": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I32, _P]),
    "pa_decode_noalloc": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I32, _P]),
    "pa_workspace_bytes": (_SZ, [_DIMS, _I64, _I32]),
    "pa_workspace_layout": (_I32, [_DIMS, _I64, _I32, ctypes.POINTER(_I64)]),
    "pa_decode_ex": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I32, _P, _P, _SZ,
                            _I64, _I32]),
    "pa_decode_profiled": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I32, _P, _P,
                                  _SZ, _I64, _I32, _P, _P]),
    "pa_v2_partition": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I32, _I64, _P,
                               _SZ, _P]),
    "pa_v2_reduce": (_I32, [_DIMS, _P, _P, _I32, _I64, _P, _SZ, _P]),
    "pa_v1": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I64, _P]),
    "pa_choose_path": (_I32, [_DIMS, _I64, _I32]),
    "pa_set_v1_max_context": (None, [_I64]),
    "pa_get_v1_max_context": (_I64, []),
    "pa_num_partitions": (_I64, [_I64, _I32]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_release": (None, []),
    "pa_version": (ctypes.c_char_p, []),
    "pa_set_mfma_variant": (_I32, [_I32]),
    "pa_get_mfma_variant": (_I32, []),
    "pa_set_fused": (_I32, [_I32]),
    "pa_get_fused": (_I32, []),
    "pa_set_prefill_mode": (_I32, [_I32]),
    "pa_get_prefill_mode": (_I32, []),
    "pa_set_prefill_split": (_I32, [_I32]),
    "pa_get_prefill_split": (_I32, []),
    "pa_fused_applies": (_I32, [_DIMS, _I32]),
    "pa_set_work_split": (_I32, [_I32, _I64]),
    "pa_get_work_split": (_I32, [ctypes.POINTER(_I64)]),
    "pa_split_plan": (_I32, [_DIMS, _I64, _I32, ctypes.POINTER(_I64)]),
    "pa_copy_blocks": (_I32, [_P, _P, _I64, _I64, _P, _I64, _P]),
    "pa_copy_blocks_profiled": (_I32, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _P]),
    "pa_prefill": (_I32, [ctypes.POINTER(PaPrefillDims), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                          ctypes.c_float, _P]),
    "pa_prefill_profiled": (_I32, [ctypes.POINTER(PaPrefillDims), _P, _P, _P, _P, _P, _P, _P,
                                   _P, _P, ctypes.c_float, _P, _P, _P]),
    "pa_prefill_ex": (_I32, [ctypes.POINTER(PaPrefillDims), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                             ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "pa_prefill_workspace_bytes": (_I64, [ctypes.POINTER(PaPrefillDims)]),
}

LAYOUT_FIELDS = 9

_lib_handle = None


def lib():
    """Load libpa_decode.so once; raise if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise PaError(-9, f"HIP library not built: {LIB_PATH} is missing "
                              "(run `python -m paged_split_kv_pa_amd.build`)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = h
    return _lib_handle


def _check(status):
    if status != PA_OK:
        raise PaError(status, pa_last_error())


def _dtype_code(t):
    import torch
    codes = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
    if t.dtype not in codes:
        raise PaError(-2, f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def dims_of(q, k_cache, block_tables, out=None, v_cache=None):
    """pa_dims_t from tensor shapes and strides (q [S,Hq,D], k_cache [NB,Hkv,bs,D], table
    [S,MB]; out and v_cache, when given, for their strides)."""
    if q.dim() != 3 or k_cache.dim() != 4 or block_tables.dim() != 2:
        raise PaError(-3, "q must be 3-D, k_cache 4-D and block_tables 2-D")
    S, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    if Dk != D:
        raise PaError(-3, f"head_dim of q ({D}) and k_cache ({Dk}) differ")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t is not None and tuple(t.stride()[1:]) != (bs * D, D, 1) and t.numel() > 0:
            raise PaError(PA_ERR_STRIDE, f"{name}: every block must be a dense [Hkv, 16, D] "
                                         f"array (strides {tuple(t.stride())})")
    if v_cache is not None and v_cache.stride(0) != k_cache.stride(0):
        raise PaError(PA_ERR_STRIDE, "k_cache and v_cache must have the same block stride")
    if block_tables.stride(1) != 1 and block_tables.shape[1] > 1:
        raise PaError(PA_ERR_STRIDE, "block_tables rows must be contiguous")
    d = PaDims(S, Hq, Hkv, D, bs, NB, block_tables.shape[1], _dtype_code(q))

    def st(t, i):  # the stride of a size-1 dimension is never used: 0 (the default)
        return 0 if t.shape[i] == 1 else t.stride(i)
    d.q_stride_seq, d.q_stride_head, d.q_stride_dim = st(q, 0), st(q, 1), q.stride(2)
    if out is not None:
        d.out_stride_seq, d.out_stride_head, d.out_stride_dim = st(out, 0), st(out, 1), \
            out.stride(2)
    d.kv_stride_block = st(k_cache, 0)
    d.bt_stride_seq = st(block_tables, 0)
    return d


def _ptr(t, name, dtype=None, strided=False):
    """Device address of t; strided tensors are described to the library by their
    strides (pa_dims_t), others must be contiguous."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise PaError(-1, f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise PaError(-1, f"{name} must be a device tensor")
    if not strided and not t.is_contiguous():
        raise PaError(-3, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PaError(-2, f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _tensors(out, q, k_cache, v_cache, block_tables, context_lens):
    import torch
    for name, t in (("out", out), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != q.dtype:
            raise PaError(-2, f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    if tuple(out.shape) != tuple(q.shape):
        raise PaError(-3, "out must have the shape of q")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise PaError(-3, "v_cache must have the shape of k_cache")
    if context_lens.dim() != 1 or context_lens.shape[0] != q.shape[0] or \
            block_tables.shape[0] != q.shape[0]:
        raise PaError(-3, "block_tables and context_lens need one row per sequence")
    return (_ptr(out, "out", strided=True), _ptr(q, "q", strided=True),
            _ptr(k_cache, "k_cache", strided=True), _ptr(v_cache, "v_cache", strided=True),
            _ptr(block_tables, "block_tables", torch.int32, strided=True),
            _ptr(context_lens, "context_lens", torch.int32))


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, partition_size=512,
              stream=None):
    """One decode step; path by context bound; library-owned workspace."""
    d = dims_of(q, k_cache, block_tables, out, v_cache)
    ptrs = _tensors(out, q, k_cache, v_cache, block_tables, context_lens)
    _check(lib().pa_decode(ctypes.byref(d), *ptrs, float(scale), int(partition_size),
                           _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # PA_NOALLOC_SCRATCH_BYTES


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      partition_size=512, stream=None):
    """pa_decode with the library's static scratch as the V2 workspace: no allocation."""
    d = dims_of(q, k_cache, block_tables, out, v_cache)
    ptrs = _tensors(out, q, k_cache, v_cache, block_tables, context_lens)
    _check(lib().pa_decode_noalloc(ctypes.byref(d), *ptrs, float(scale), int(partition_size),
                                   _stream(stream)))
    return out


def pa_workspace_bytes(q, k_cache, block_tables, max_context_len=0, partition_size=512):
    d = dims_of(q, k_cache, block_tables)
    n = lib().pa_workspace_bytes(ctypes.byref(d), int(max_context_len), int(partition_size))
    if n == 0 and d.num_seqs > 0:
        raise PaError(-3, pa_last_error())
    return n


def _ws(workspace):
    if workspace is None:
        return ctypes.c_void_p(0), 0
    return _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()


def pa_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                 partition_size=512, stream=None, workspace=None, max_context_len=0,
                 path=PA_PATH_AUTO):
    d = dims_of(q, k_cache, block_tables, out, v_cache)
    ptrs = _tensors(out, q, k_cache, v_cache, block_tables, context_lens)
    wp, wb = _ws(workspace)
    _check(lib().pa_decode_ex(ctypes.byref(d), *ptrs, float(scale), int(partition_size),
                              _stream(stream), wp, wb, int(max_context_len), int(path)))
    return out


def pa_decode_profiled(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       partition_size=512, stream=None, workspace=None, max_context_len=0,
                       path=PA_PATH_AUTO, start_event=None, stop_event=None):
    """pa_decode_ex plus runtime timestamps (hipEvent_t handles) of the attention kernel."""
    d = dims_of(q, k_cache, block_tables, out, v_cache)
    ptrs = _tensors(out, q, k_cache, v_cache, block_tables, context_lens)
    wp, wb = _ws(workspace)
    _check(lib().pa_decode_profiled(ctypes.byref(d), *ptrs, float(scale), int(partition_size),
                                    _stream(stream), wp, wb, int(max_context_len), int(path),
                                    start_event, stop_event))
    return out


def pa_v2_partition(out, q, k_cache, v_cache, block_tables, context_lens, scale, workspace,
                    partition_size=512, max_context_len=0, stream=None):
    d = dims_of(q, k_cache, block_tables, out, v_cache)
    ptrs = _tensors(out, q, k_cache, v_cache, block_tables, context_lens)
    wp, wb = _ws(workspace)
    _check(lib().pa_v2_partition(ctypes.byref(d), *ptrs, float(scale), int(partition_size),
                                 int(max_context_len), wp, wb, _stream(stream)))
    return out


def pa_v2_reduce(out, q, k_cache, block_tables, context_lens, workspace, partition_size=512,
                 max_context_len=0, stream=None):
    import torch
    d = dims_of(q, k_cache, block_tables, out)
    wp, wb = _ws(workspace)
    _check(lib().pa_v2_reduce(ctypes.byref(d), _ptr(out, "out", strided=True),
                              _ptr(context_lens, "context_lens", torch.int32),
                              int(partition_size), int(max_context_len), wp, wb,
                              _stream(stream)))
    return out


def pa_v1(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len=0,
          stream=None):
    d = dims_of(q, k_cache, block_tables, out, v_cache)
    ptrs = _tensors(out, q, k_cache, v_cache, block_tables, context_lens)
    _check(lib().pa_v1(ctypes.byref(d), *ptrs, float(scale), int(max_context_len),
                       _stream(stream)))
    return out


def pa_choose_path(dims, max_context_len=0, partition_size=512):
    r = lib().pa_choose_path(ctypes.byref(dims), int(max_context_len), int(partition_size))
    if r < 0:
        raise PaError(r, pa_last_error())
    return r


def pa_set_v1_max_context(tokens):
    lib().pa_set_v1_max_context(int(tokens))


def pa_get_v1_max_context():
    return int(lib().pa_get_v1_max_context())


def pa_num_partitions(n, partition_size):
    return int(lib().pa_num_partitions(int(n), int(partition_size)))


def pa_last_error():
    msg = lib().pa_last_error()
    return msg.decode() if msg else ""


def pa_release():
    lib().pa_release()


def pa_version():
    return lib().pa_version().decode()


def pa_set_mfma_variant(variant):
    _check(lib().pa_set_mfma_variant(int(variant)))


def pa_get_mfma_variant():
    return int(lib().pa_get_mfma_variant())


def pa_set_fused(mode):
    """Single-launch V2 for library-managed workspaces: 1 where it applies, 0 never
    (the default)."""
    _check(lib().pa_set_fused(int(mode)))


def pa_get_fused():
    return int(lib().pa_get_fused())


def pa_set_prefill_mode(mode):
    """0: P and V as fp16 in prefill's PV products (bf16 recomputed in the two-part form
    when V does not fit fp16); 1: P as a 16-bit high plus low part (process-wide)."""
    _check(lib().pa_set_prefill_mode(int(mode)))


def pa_get_prefill_mode():
    return int(lib().pa_get_prefill_mode())


def pa_set_prefill_split(chunk_tiles):
    """Prefill load balance: -1 automatic chunks (default), 0 none, k >= 4 chunks of at
    most k 64-key tiles (process-wide)."""
    _check(lib().pa_set_prefill_split(int(chunk_tiles)))


def pa_get_prefill_split():
    return int(lib().pa_get_prefill_split())


def pa_fused_applies(q, k_cache, block_tables, partition_size=512):
    """True if pa_decode would run V2 as a single launch for these shapes."""
    d = dims_of(q, k_cache, block_tables)
    r = lib().pa_fused_applies(ctypes.byref(d), int(partition_size))
    if r < 0:
        raise PaError(r, pa_last_error())
    return bool(r)


def pa_set_work_split(pieces, first_item=0):
    """-1 automatic, 0/1 off, 2/4/8/16 pieces for every item from first_item on."""
    _check(lib().pa_set_work_split(int(pieces), int(first_item)))


def pa_get_work_split():
    """(pieces, first_item) of the current work-split setting."""
    f = ctypes.c_int64()
    return int(lib().pa_get_work_split(ctypes.byref(f))), int(f.value)


def split_plan(q, k_cache, block_tables, max_context_len=0, partition_size=512):
    """Work split a V2 call would use: dict items, first, pieces, workgroups."""
    d = dims_of(q, k_cache, block_tables)
    v = (ctypes.c_int64 * 4)()
    _check(lib().pa_split_plan(ctypes.byref(d), int(max_context_len), int(partition_size), v))
    return dict(zip(("items", "first", "pieces", "workgroups"), list(v)))


def pa_copy_blocks(k_cache, v_cache, block_pairs, stream=None):
    """Copy blocks src -> dst of both pools (v_cache may be None) for the (src, dst)
    int32 rows of ``block_pairs`` [n, 2]; all device tensors."""
    for t in (k_cache, v_cache, block_pairs):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise PaError(-1, "pa_copy_blocks takes contiguous device tensors")
    if v_cache is not None and (v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype):
        raise PaError(-3, "v_cache must match k_cache in shape and dtype")
    if block_pairs.dtype.itemsize != 4 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise PaError(-3, "block_pairs must be an int32 tensor [n, 2]")
    block_bytes = k_cache[0].numel() * k_cache.element_size()
    _check(lib().pa_copy_blocks(ctypes.c_void_p(k_cache.data_ptr()),
                                ctypes.c_void_p(v_cache.data_ptr() if v_cache is not None else 0),
                                int(block_bytes), int(k_cache.shape[0]),
                                ctypes.c_void_p(block_pairs.data_ptr()), int(block_pairs.shape[0]),
                                _stream(stream)))


def prefill_dims_of(q, k_new, k_cache, block_tables, context_lens, max_query_len=0):
    """pa_prefill_dims_t from tensor shapes: q [T,Hq,D], k_new [T,Hkv,D], k_cache
    [NB,Hkv,bs,D], block_tables [S,MB], context_lens [S]."""
    if q.dim() != 3 or k_new.dim() != 3 or k_cache.dim() != 4 or block_tables.dim() != 2:
        raise PaError(-3, "q / k_new must be 3-D, k_cache 4-D and block_tables 2-D")
    T, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    if Dk != D or tuple(k_new.shape) != (T, Hkv, D):
        raise PaError(-3, "k_new must be [T, Hkv, D] matching q and k_cache")
    return PaPrefillDims(context_lens.shape[0], T, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                         _dtype_code(q), int(max_query_len))


def pa_prefill_workspace_bytes(q, k_new, k_cache, block_tables, context_lens, max_query_len=0):
    """Bytes of the workspace pa_prefill_ex needs for these tensors (0: none)."""
    d = prefill_dims_of(q, k_new, k_cache, block_tables, context_lens, max_query_len)
    r = int(lib().pa_prefill_workspace_bytes(ctypes.byref(d)))
    if r < 0:
        _check(r)
    return r


def pa_prefill(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, query_start,
               scale, max_query_len=0, stream=None, start_event=None, stop_event=None,
               workspace=None):
    """Paged prefix-prefill attention (include/pa_decode.h, pa_prefill); all device tensors.
    With `workspace` (a uint8 device tensor, see pa_prefill_workspace_bytes) the call goes
    through pa_prefill_ex."""
    d = prefill_dims_of(q, k_new, k_cache, block_tables, context_lens, max_query_len)
    for name, t in (("out", out), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        if t.dtype != q.dtype:
            raise PaError(-2, f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    if tuple(out.shape) != tuple(q.shape) or tuple(v_new.shape) != tuple(k_new.shape) or \
            tuple(v_cache.shape) != tuple(k_cache.shape):
        raise PaError(-3, "out / v_new / v_cache shapes must match q / k_new / k_cache")
    if query_start.dim() != 1 or query_start.shape[0] != context_lens.shape[0] + 1 or \
            block_tables.shape[0] != context_lens.shape[0]:
        raise PaError(-3, "query_start needs S+1 entries, block_tables one row per sequence")
    import torch
    ptrs = (_ptr(out, "out"), _ptr(q, "q"), _ptr(k_new, "k_new"), _ptr(v_new, "v_new"),
            _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
            _ptr(block_tables, "block_tables", torch.int32),
            _ptr(context_lens, "context_lens", torch.int32),
            _ptr(query_start, "query_start", torch.int32))
    if workspace is not None:
        if start_event is not None or stop_event is not None:
            raise PaError(-9, "timestamps are taken with the library's workspace only")
        _check(lib().pa_prefill_ex(ctypes.byref(d), *ptrs, float(scale),
                                   ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                   _stream(stream)))
    elif start_event is None and stop_event is None:
        _check(lib().pa_prefill(ctypes.byref(d), *ptrs, float(scale), _stream(stream)))
    else:
        _check(lib().pa_prefill_profiled(ctypes.byref(d), *ptrs, float(scale), _stream(stream),
                                         start_event, stop_event))
    return out


def workspace_layout(q, k_cache, block_tables, max_context_len=0, partition_size=512):
    """Section offsets of a V2 workspace, as the library computes them.

    Returns a dict: pmax, bytes, slots, and for tmp_out / max_logits / exp_sums /
    piece_out / piece_max / piece_sum a (byte offset, shape) pair; all are fp32,
    tmp_out [S, Hq, pmax, D], the statistics [S, Hq, pmax], piece_out
    [slots, G, D] and the piece statistics [slots, G].
    """
    d = dims_of(q, k_cache, block_tables)
    v = (ctypes.c_int64 * LAYOUT_FIELDS)()
    _check(lib().pa_workspace_layout(ctypes.byref(d), int(max_context_len),
                                     int(partition_size), v))
    pmax, o_tmp, o_max, o_sum, slots, o_pout, o_pmax, o_psum, nbytes = list(v)
    S, Hq, D = d.num_seqs, d.num_q_heads, d.head_dim
    G = Hq // d.num_kv_heads
    return {"pmax": pmax, "bytes": nbytes, "slots": slots,
            "tmp_out": (o_tmp, (S, Hq, pmax, D)),
            "max_logits": (o_max, (S, Hq, pmax)), "exp_sums": (o_sum, (S, Hq, pmax)),
            "piece_out": (o_pout, (slots, G, D)), "piece_max": (o_pmax, (slots, G)),
            "piece_sum": (o_psum, (slots, G))}
