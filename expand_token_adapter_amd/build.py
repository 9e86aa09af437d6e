"""Build the HIP library liblora_batch.so for gfx950 with hipcc (in-tree).

Every source is compiled to its own object (in parallel), then the objects are
linked into one shared library.  No relocatable device code: each object
carries the device code of its own kernels.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblora_batch.so")
SOURCES = ["segments.hip", "forward.hip", "fused.hip", "backward.hip", "optimizer.hip", "noalloc.hip", "abi.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed-fp32 instructions stay off in every build of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building liblora_batch.so: " + " ".join(cmd[-3:]))
    return res


def build(verbose: bool = False, out: str = LIB, defines=(), jobs: int = 0) -> str:
    """Compile every source into liblora_batch.so next to this file (or `out`,
    with extra -D tuning `defines`); return its path."""
    defs = ["-D" + d for d in defines]
    inc = ["-I", INCLUDE, "-I", CSRC]
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="lora_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc()] + HIPCC_FLAGS + defs + inc + ["-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = out + ".tmp%d" % os.getpid()
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
