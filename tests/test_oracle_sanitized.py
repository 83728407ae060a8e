"""The oracle's C under AddressSanitizer and UndefinedBehaviorSanitizer (CPU tier).

``oracle/oracle.c`` is built a second time, with ``-fsanitize=address,undefined``,
into a temporary directory, and a child process drives every exported function
through ctypes with ``libasan`` preloaded: the three activations on ragged shapes
(single rows, single columns, a prime width), zero tokens, the partials sum for
k = 1..5, the plain product, and each rejected argument.  Results are checked
against NumPy float64 on the same inputs; any sanitizer report fails the test.
The library under test is the sanitized copy, never the one the other tests load.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ORACLE_C = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None,
                                reason="gcc with AddressSanitizer is not available")

CHILD = textwrap.dedent(r"""
    import ctypes, sys
    import numpy as np
    lib = ctypes.CDLL(sys.argv[1])
    dp = ctypes.POINTER(ctypes.c_double)
    lib.orc_shard_forward.argtypes = [dp, ctypes.c_int64, ctypes.c_int64, dp, ctypes.c_int64, dp,
                                      ctypes.c_int64, ctypes.c_int, dp]
    lib.orc_partials_sum.argtypes = [ctypes.POINTER(dp), ctypes.c_int32, ctypes.c_int64, dp]
    lib.orc_matmul.argtypes = [dp, ctypes.c_int64, ctypes.c_int64, dp, ctypes.c_int64, dp]
    P = lambda a: a.ctypes.data_as(dp)
    rng = np.random.default_rng(5)
    acts = {0: lambda s, F: np.tanh(s), 1: lambda s, F: s[:, :F] / (1 + np.exp(-s[:, :F])) * s[:, F:],
            2: lambda s, F: s}
    for M, d, F, N in [(1, 1, 1, 1), (3, 5, 2, 7), (17, 31, 13, 1), (2, 64, 37, 33), (0, 4, 4, 4)]:
        for act, f in acts.items():
            X = rng.standard_normal((M, d))
            A = rng.standard_normal((d, 2 * F if act == 1 else F)) * 0.3
            B = rng.standard_normal((F, N))
            out = np.full((M, N), np.nan)
            assert lib.orc_shard_forward(P(X), M, d, P(A), F, P(B), N, act, P(out)) == 0
            if M:
                ref = f(X @ A, F) @ B
                assert np.allclose(out, ref, rtol=1e-12, atol=1e-12), (M, d, F, N, act)
    for k in range(1, 6):
        parts = [rng.standard_normal(1001) for _ in range(k)]
        arr = (dp * k)(*[P(p) for p in parts])
        z = np.zeros(1001)
        assert lib.orc_partials_sum(arr, k, 1001, P(z)) == 0
        assert np.allclose(z, np.sum(parts, axis=0), rtol=1e-13, atol=1e-13)
    X = rng.standard_normal((9, 11)); W = rng.standard_normal((11, 6)); Y = np.zeros((9, 6))
    assert lib.orc_matmul(P(X), 9, 11, P(W), 6, P(Y)) == 0 and np.allclose(Y, X @ W, rtol=1e-13)
    # rejected arguments: nothing is read or written
    one = np.zeros((1, 1))
    assert lib.orc_shard_forward(P(one), -1, 1, P(one), 1, P(one), 1, 0, P(one)) != 0
    assert lib.orc_shard_forward(P(one), 1, 0, P(one), 1, P(one), 1, 0, P(one)) != 0
    assert lib.orc_shard_forward(P(one), 1, 1, P(one), 1, P(one), 1, 7, P(one)) != 0
    assert lib.orc_shard_forward(None, 1, 1, P(one), 1, P(one), 1, 0, P(one)) != 0
    assert lib.orc_partials_sum(None, 1, 1, P(one)) != 0
    assert lib.orc_partials_sum((dp * 1)(P(one)), 0, 1, P(one)) != 0
    assert lib.orc_matmul(P(one), 1, 0, P(one), 1, P(one)) != 0
    print("sanitized oracle ok")
""")


def test_oracle_under_address_and_undefined_behavior_sanitizers(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-Wall",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", so, ORACLE_C, "-lm"], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, "-c", CHILD, so], capture_output=True, text=True, env=env,
                       timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert "sanitized oracle ok" in r.stdout
