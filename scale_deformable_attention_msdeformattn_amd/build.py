"""Build libmsda.so (the HIP/gfx950 library behind include/msda.h) in-tree.

Compiles every ``csrc/*.hip`` with hipcc for gfx950 and links one shared
library next to this file. Runs on a machine without a GPU (hipcc
cross-compiles). Packed-FP32 instructions are disabled for device code.
"""
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmsda.so")
ARCH = os.environ.get("MSDA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument",
    # device code: no packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        procs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), src))
            objs.append(obj)
        for p, src in procs:
            _, err = p.communicate()
            err = "\n".join(ln for ln in err.splitlines()
                            if "packed-fp32-ops' is not a recognized feature" not in ln)
            if p.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
