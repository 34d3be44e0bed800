"""Exact upcast of stored values to float64 (oracle; test infrastructure only).

The decode problem is stated on fp16/bf16 (and, for the tiny case, fp32) KV
caches with fp32 accumulation (project_6 optimizations/prefix_prefill_patch.py,
docstring: the attention dtype is fp16/bf16).  The oracle works in float64, so
every stored value must first be turned into the float64 it represents,
exactly.  All three formats embed exactly in float64.

Storage conventions (shared with the input generators, which only *produce*
these arrays):

* ``"f32"``  -- ``numpy.float32`` array.
* ``"f16"``  -- ``numpy.float16`` array (IEEE binary16).
* ``"bf16"`` -- ``numpy.uint16`` array holding bfloat16 bit patterns: the top
  16 bits of the IEEE binary32 value.
"""

import numpy as np

STORAGE_DTYPES = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def upcast(arr, dtype):
    """Return the float64 values that ``arr`` (stored as ``dtype``) represents.

    bfloat16 is the upper half of a binary32 word, so the value is recovered by
    placing the 16 stored bits in the high half of a 32-bit word and reading
    that word as binary32; the widening to float64 is then exact.
    """
    a = np.asarray(arr)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError(f"f32 storage must be float32, got {a.dtype}")
        return a.astype(np.float64)
    if dtype == "f16":
        if a.dtype != np.float16:
            raise TypeError(f"f16 storage must be float16, got {a.dtype}")
        return a.astype(np.float64)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError(f"bf16 storage must be uint16 bit patterns, got {a.dtype}")
        word = a.astype(np.uint32) << np.uint32(16)
        return word.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")
