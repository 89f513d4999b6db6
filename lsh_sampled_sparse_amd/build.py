"""Compile libmagicpig.so (HIP, gfx950) in-tree with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmagicpig.so")
SOURCES = ["api.hip", "index_build.hip", "decode.hip", "tables.hip", "probe.hip", "noalloc.hip"]
ARCH = os.environ.get("MP_OFFLOAD_ARCH", "gfx950")

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         # keep hipcc from forming packed-fp32 VALU ops on its own
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics"]


def _compile(src, verbose):
    obj = os.path.join(CSRC, "_build", os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(CSRC, "_build"), exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", OUT + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
