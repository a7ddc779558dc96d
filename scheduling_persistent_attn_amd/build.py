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
SOURCES = ["bwd.hip", "bwd_wide.hip", "bwd_wide64.hip", "fwd.hip", "api.cpp", "sim.cpp", "table.cpp"]
HOST_ONLY = {"sim.cpp", "table.cpp"}  # plain C++, no HIP
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
         "bwd_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "bwd_wide64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# The debug build with the per-task trace (DASH_TASK_TRACE): the sources that
# read the flag are compiled again with it and linked into a second library.
TRACE_LIB = os.path.join(HERE, "libdash_attn_trace.so")
TRACED = ("bwd.hip", "bwd_wide.hip", "bwd_wide64.hip", "api.cpp")


def build(verbose=False):
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(job):
        src, traced = job
        obj = os.path.join(objdir, src + (".trace.o" if traced else ".o"))
        flags = ["-DDASH_TASK_TRACE=1"] if traced else []
        if src in HOST_ONLY:
            cmd = ["g++", "-O2", "-std=c++17", "-fPIC"] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        else:
            cmd = [cc] + COMMON + EXTRA.get(src, []) + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
        return obj

    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in TRACED]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = dict(zip(jobs, ex.map(compile_one, jobs)))
    for lib, traced in ((LIB, False), (TRACE_LIB, True)):
        parts = [objs[(src, traced and src in TRACED)] for src in SOURCES]
        tmp = lib + ".tmp"
        cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + parts
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
