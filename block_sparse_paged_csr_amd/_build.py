"""Compile the HIP library ``libsa.so`` in-tree for gfx950.

``python -m block_sparse_paged_csr_amd._build`` (or ``build()``) always
recompiles. The loader never compiles: it only opens the built library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libsa.so")
SOURCES = ["sa_api.hip", "sa_index.hip", "sa_forward.hip", "sa_forward_wave.hip",
           "sa_forward_small.hip", "sa_forward_mfma.hip", "sa_combine.hip"]

# Packed fp32 VALU forms are kept out of the generated code; the compiler
# only warns on the host pass that it does not know the feature.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument"]
# Per-file flags. The MFMA kernels keep their matrix accumulators in ordinary
# VGPRs: the chunked kernel rescales its output accumulators between chunks,
# which in accumulation registers would cost a copy each way (the other
# kernels of that file compile to the same code either way).
FILE_FLAGS = {"sa_forward_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source to an object (in parallel, each with its own
    flags), then link the shared library."""
    import tempfile
    names = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="sa_build_") as odir:
        procs, objs = [], []
        for name in names:
            obj = os.path.join(odir, name + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(name, []), *extra_flags, "-c",
                   os.path.join(CSRC, name), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                 text=True)))
            objs.append(obj)
        failed = []
        for name, p in procs:
            out, _ = p.communicate()
            if p.returncode != 0:
                sys.stderr.write(out)
                failed.append(name)
        if failed:
            raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
