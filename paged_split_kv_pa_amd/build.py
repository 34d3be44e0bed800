"""Build libpa_decode.so (the HIP kernels + C ABI) in-tree for gfx950.

Usage: ``python -m paged_split_kv_pa_amd.build`` or ``build()`` from Python.
The library is written to ``paged_split_kv_pa_amd/lib/libpa_decode.so``; the
object files of each translation unit are compiled in parallel.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libpa_decode.so"
SOURCES = ["pa_api.hip", "pa_kernels.hip", "pa_copy.hip", "pa_prefill.hip"]
ARCH = "gfx950"

# hipcc flags.  Packed fp32 instructions are disabled for every HIP source.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source flags.  The prefill kernel keeps its 128 output accumulators per lane in
# VGPRs (the softmax rescales them with VALU instructions); in the default AGPR form the
# compiler copied them between the register files on every K/V tile.
# The decode kernels take their latency-critical arguments as leading scalars (see
# PA_ATTN_LEAD_PARAMS and PA_REDUCE_LEAD_PARAMS in pa_kernels.hip); the hardware preloads
# those into registers.  Their accumulators stay in VGPRs too: at head_dim 256 (over 256
# registers per lane) the AGPR form moved ~240 values between the register files per KV
# block; at head_dim 128 the code is the same either way.
SOURCE_FLAGS = {"pa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "pa_kernels.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=12",
                                   "-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 target feature; that warning is harmless.
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose=False, extra_flags=()):
    """Compile every HIP source for gfx950 and link the shared library. Returns its path."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    out = os.path.join(LIBDIR, LIBNAME)
    tmp = out + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
