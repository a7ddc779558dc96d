"""Build libdash_attn.so in-tree with hipcc for gfx950.

    python -m scheduling_persistent_attn_amd.build

Compiles each source to an object in parallel, then links one shared library
next to this file.  Always recompiles (it is the "does it build" check).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdash_attn.so")
SOURCES = ["bwd.hip", "bwd_wide.hip", "fwd.hip", "api.cpp", "sim.cpp"]
HOST_ONLY = {"sim.cpp"}  # plain C++, no HIP
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=" + ARCH,
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast",
    "-munsafe-fp-atomics",
    "-Wno-unused-command-line-argument",
]

# per-source additions: the backward kernel keeps its matrix-product
# accumulators in the vector registers (the softmax reads S and dP and the
# dQ partial sum is loaded straight into its accumulator), and pins the
# operands it holds for a whole KV tile to the accumulation registers itself
EXTRA = {"bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "bwd_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        if src in HOST_ONLY:
            cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-c", os.path.join(CSRC, src), "-o", obj]
        else:
            cmd = [cc] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
