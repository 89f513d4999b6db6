"""Compile the fp64 oracle into oracle/liboracle.so (plain C, gcc, no fast-math).

Test infrastructure only: building the checker is not using it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


# Host sanitizers of the checked build: AddressSanitizer (bounds, use after
# free, leaks) and UndefinedBehaviorSanitizer, every report fatal.
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    """Compile oracle.c to `out` (default oracle/liboracle.so).  With
    `sanitize` the library is built under SANITIZE_FLAGS; a process loading it
    must have the sanitizer runtimes preloaded (sanitized_env)."""
    out = out or OUT
    opt = SANITIZE_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-D_GNU_SOURCE", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def sanitized_env(lib_path: str, base: dict | None = None) -> dict:
    """Environment of a Python process that loads the sanitized oracle at
    lib_path: gcc's ASan and UBSan runtimes preloaded, leak checks off (the
    interpreter itself keeps memory to the end), every report fatal."""
    env = dict(os.environ if base is None else base)
    rt = [subprocess.run(["gcc", f"-print-file-name={n}"], check=True, capture_output=True,
                         text=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    env["LD_PRELOAD"] = ":".join(rt)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    env["MP_ORACLE_LIB"] = lib_path
    return env


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
