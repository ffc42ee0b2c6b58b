"""The oracle and the library's host-side checks under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no GPU). The oracle is rebuilt with the
sanitizers and driven in a child process that preloads their runtimes; any report aborts
the child and fails the test."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN = _runtime("libasan.so")
UBSAN = _runtime("libubsan.so")

DRIVER = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, ROOT)
    from oracle import topk as otk
    from workloads import gen
    g = np.random.default_rng(5)
    for dtype in (gen.BF16, gen.FP32):
        for fam in ("normal", "ties", "specials", "constant", "tiny", "ascending"):
            for rows, n in ((1, 1), (3, 7), (5, 1000), (2, 70001)):
                x = gen.rows_family(fam, dtype, 9, rows, n)
                for k in sorted({1, min(n, 5), n}):
                    v, i = otk.topk(x, k)
                    assert (i >= 0).all() and (i < n).all()
                    lens = g.integers(-2, n + 3, size=rows)
                    otk.topk_ragged(x, lens, k)
        x = gen.rows_family("normal", dtype, 10, 1, 1 << 21)  # one long row: the chunked path
        otk.topk(x, 4096)
        otk.topk(x, 37, indices=False)
        otk.topk(x, 37, values=False, threads=3)
    print("sanitized oracle runs clean")
""").replace("ROOT", repr(ROOT))


@pytest.mark.skipif(ASAN is None or UBSAN is None, reason="gcc sanitizer runtimes not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_topk_san.so")
    subprocess.check_call(["g++", "-O1", "-g", "-std=c++17", "-shared", "-fPIC", "-pthread",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle_topk.cpp"), "-o", lib])
    env = dict(os.environ, DS_ORACLE_LIB=lib, LD_PRELOAD=f"{ASAN}:{UBSAN}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-c", DRIVER], env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "sanitized oracle runs clean" in res.stdout
