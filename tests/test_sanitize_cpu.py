"""Host code under sanitizers (CPU only, no GPU).

* The library's C-ABI source (argument validation, handle registry, workspace
  and scratch layouts, launch sequences) compiled with g++ under
  AddressSanitizer + UndefinedBehaviorSanitizer, and separately under
  ThreadSanitizer, with stand-in launchers that touch every byte the kernels
  would read or write (tests/sanitize/abi_host_check.cpp).
* The oracle (oracle/oracle.c) compiled under AddressSanitizer +
  UndefinedBehaviorSanitizer, running the oracle pin tests in a child
  interpreter with the sanitizer runtimes preloaded.

Each sanitizer run also gets one planted mistake (in a copy of the source, on
the CPU) to show that it is seen.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECK_SRC = os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp")
ROCM_INC = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(
    shutil.which("g++") is None or shutil.which("gcc") is None
    or not os.path.isdir(os.path.join(ROCM_INC, "hip")),
    reason="needs gcc/g++ and the HIP headers")

ASAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
TSAN = ["-fsanitize=thread"]


def _build_check(src, out, flags):
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *flags,
           "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INC, "-w", src, "-o", out, "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def _tree_copy(tmp_path, api_edit=None):
    """The check and the sources it includes, under tmp_path (api.hip edited
    by api_edit(text) when given)."""
    for rel in ("tests/sanitize/abi_host_check.cpp", "lsh_sampled_sparse_amd/csrc/api.hip",
                "lsh_sampled_sparse_amd/csrc/mp_internal.h", "include/magicpig.h",
                "include/magicpig_bench.h", "include/magicpig_testing.h"):
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        text = open(os.path.join(ROOT, rel)).read()
        if api_edit is not None and rel.endswith("api.hip"):
            text = api_edit(text)
        dst.write_text(text)
    return str(tmp_path / "tests/sanitize/abi_host_check.cpp")


def test_abi_host_path_asan_ubsan(tmp_path):
    exe = _build_check(CHECK_SRC, str(tmp_path / "abi_asan"), ASAN)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    rc, out = _run([exe, "all"], env=env)
    print(out[-4000:])
    assert rc == 0 and "ALL OK" in out


def test_abi_host_path_tsan(tmp_path):
    exe = _build_check(CHECK_SRC, str(tmp_path / "abi_tsan"), TSAN)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    rc, out = _run([exe, "threads"], env=env)
    print(out[-4000:])
    assert rc == 0 and "ALL OK" in out and "WARNING: ThreadSanitizer" not in out


@pytest.mark.parametrize("name,old,new,report", [
    # the chunk partials laid out one float short per head
    ("scratch_region_short", "off + BHq * lay.n_chunks * int64_t(kD + 2) * 4",
     "off + BHq * lay.n_chunks * int64_t(kD + 1) * 4", "heap-buffer-overflow"),
    # destroy forgets to free the handle
    ("handle_leak", "if (idx && unregister_handle(idx)) delete idx;",
     "if (idx) unregister_handle(idx);", "LeakSanitizer"),
])
def test_abi_check_sees_planted_mistakes(tmp_path, name, old, new, report):
    def edit(text):
        assert old in text, f"planted edit {name} no longer applies"
        return text.replace(old, new)
    src = _tree_copy(tmp_path, edit)
    exe = _build_check(src, str(tmp_path / "abi_mut"), ASAN)
    rc, out = _run([exe, "all"], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert rc != 0 and report in out, out[-3000:]


def _sanitized_oracle(tmp_path, src=None):
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    lib = str(tmp_path / "liboracle_san.so")
    if src is None:
        ob.build(sanitize=True, out=lib)
    else:
        cmd = ["gcc", *ob.SANITIZE_FLAGS, "-std=c11", "-D_GNU_SOURCE", "-fno-fast-math",
               "-ffp-contract=off", "-fPIC", "-shared", "-o", lib, src, "-lm"]
        subprocess.run(cmd, check=True)
    return lib, ob.sanitized_env(lib)


def test_oracle_pins_asan_ubsan(tmp_path):
    lib, env = _sanitized_oracle(tmp_path)
    rc, out = _run([sys.executable, "-c",
                    "import oracle, ctypes; oracle.lib(); print(oracle._LIB_PATH)"],
                   env=dict(env, PYTHONPATH=ROOT), timeout=120)
    assert rc == 0 and out.strip().endswith(lib), out
    rc, out = _run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests",
                    "test_oracle_pins.py"), "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"],
                   env=env, timeout=600)
    print(out[-3000:])
    assert rc == 0, out[-3000:]


def test_oracle_sanitizer_sees_a_planted_overrun(tmp_path):
    """orc_mean made to read one key past the end: the sanitized oracle stops
    the child with a heap-buffer-overflow report."""
    text = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    old = "void orc_mean(const double *keys, int64_t n, int d, double *mu)\n{"
    assert old in text
    text = text.replace(old, old + "\n    volatile double past = keys[n * d]; (void)past;")
    src = tmp_path / "oracle_mut.c"
    src.write_text(text)
    lib, env = _sanitized_oracle(tmp_path, str(src))
    code = ("import numpy as np, oracle\n"
            "k = np.ones((5, 128))\n"
            "print(oracle.mean(k)[:2])\n")
    rc, out = _run([sys.executable, "-c", code], env=dict(env, PYTHONPATH=ROOT), timeout=120)
    assert rc != 0 and "heap-buffer-overflow" in out, out[-3000:]
