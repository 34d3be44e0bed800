"""Paged split-KV decode attention for AMD Instinct MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``paged_split_kv_pa_amd/lib/libpa_decode.so``, declared in
``include/pa_decode.h``).  ``paged_split_kv_pa_amd.binding`` marshals torch
tensors into that ABI; nothing in this package computes attention in Python.
``paged_split_kv_pa_amd.workloads`` draws the seeded synthetic inputs.
"""

__all__ = ["binding", "workloads"]
