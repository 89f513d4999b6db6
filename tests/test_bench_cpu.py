"""Host-side checks of bench.py's plumbing: the source hash that guards the
stored counter traffic ignores comments and whitespace but not code, the
stored records are well formed, and a multi-GPU request is refused."""

import importlib.util
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_text_drops_comments_and_whitespace_only():
    b = _bench()
    src = "int a = 1; // one\n/* block\n comment */ int  b =\n 2;\n"
    assert b.code_text(src) == "int a = 1; int b = 2;"
    # a comment edit keeps the text, a code edit changes it
    assert b.code_text(src.replace("// one", "// the first")) == b.code_text(src)
    assert b.code_text(src.replace("2;", "3;")) != b.code_text(src)


def test_stored_traffic_records_are_well_formed():
    b = _bench()
    assert set(b.MEASURED_TRAFFIC) == set(b.KERNEL_SOURCES)
    for kernel, m in b.MEASURED_TRAFFIC.items():
        assert re.fullmatch(r"[0-9a-f]{64}", m["sources_sha256"]), kernel
        # the scales are stored to 4 decimals; the bytes used them unrounded
        again = m["fetch_kib"] * 1024 * m["fetch_scale"] + m["write_kib"] * 1024 * m["write_scale"]
        assert abs(m["bytes_per_launch"] - again) <= 1e-4 * again, kernel
        for name in b.KERNEL_SOURCES[kernel]:
            assert os.path.exists(os.path.join(b.CSRC, name)), name


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
