"""Build liboscar.so (HIP, gfx950) in-tree with hipcc.

    python -m long_context_decode_oscar_amd.build
    python -m long_context_decode_oscar_amd.build --phase-stamps   # profiling variant

Every source is compiled with packed-fp32 instruction selection disabled
(``-target-feature -packed-fp32-ops``) and the objects are linked into one
shared library next to this file.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liboscar.so")
SOURCES = ["oscar_api.hip", "decode.hip", "write.hip", "calib.hip"]
ARCH = os.environ.get("OSCAR_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        # kernel arguments preloaded into scalar registers at wave launch (the
        # code object carries the fallback loads for firmware without it)
        "-mllvm", "-amdgpu-kernarg-preload-count=16",
        f"-I{os.path.join(HERE, '..', 'include')}",
    ]


STAMPS_LIB = os.path.join(HERE, "liboscar_stamps.so")


def build(verbose: bool = False, phase_stamps: bool = False) -> str:
    """Compiles every source and links liboscar.so.  phase_stamps=True builds
    the profiling variant liboscar_stamps.so instead, whose plain decode
    records a per-wave phase timeline (bench.py --phase-stamps reads it)."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build", "stamps" if phase_stamps else "")
    os.makedirs(objdir, exist_ok=True)
    extra = ["-DOSCAR_PHASE_STAMPS=1"] if phase_stamps else []

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = STAMPS_LIB if phase_stamps else LIB
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_stamps="--phase-stamps" in sys.argv))
