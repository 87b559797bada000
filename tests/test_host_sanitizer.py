"""The host-side argument checks and the workspace layout under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/host_checks.cpp compiles the library's HIP-free check headers (layout.hpp for the
product-key forward, checks.hpp for the Engram lookup, the bag backward and the Memory
Attention values) with g++ and both sanitizers, with every finding fatal.  It is fed the
argument cases the ABI tests name plus a seeded sweep of extreme values (zero, negative,
INT32/INT64 limits, powers of two around every bound, NaN and infinite epsilons); the run
must end cleanly, and every verdict must equal the shipped library's for the same arguments
(through its C ABI, before any device call), so the sanitized code is the code that ships.
"""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
I32 = [-(1 << 31), -1, 0, 1, 2, 3, 7, 8, 16, 31, 32, 33, 63, 64, 65, 96, 128, 255, 256, 257, 512, 513, 514, 1024,
       2048, 4096, 46340, 46341, (1 << 24) - 1, 1 << 24, (1 << 31) - 1]
I64 = I32 + [(1 << 25), (1 << 26), (1 << 31), (1 << 32), (1 << 38), (1 << 62), (1 << 63) - 1, -(1 << 63)]
EPS = ["0", "1e-6", "0.5", "1", "1.5", "-1e-6", "nan", "inf", "-inf"]


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("host_checks") / "host_checks")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "sparse_key_value_amd", "csrc"),
                    os.path.join(ROOT, "tests", "host_checks.cpp"), "-o", exe], check=True, capture_output=True)

    def run(lines):
        r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=300,
                           env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0"})
        assert r.returncode == 0 and "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-3000:]
        out = r.stdout.splitlines()
        assert len(out) == len(lines)
        return out
    return run


@pytest.fixture(scope="module")
def P():
    import sparse_key_value_amd as P
    return P


def _pkm_cases(rng, n):
    base = [2048, 4, 512, 4096, 32, 2048, 1, 1, 1, "1e-6", 16384]
    cases = [base[:], [1024, 4, 96, 1024, 64, 1024, 1, 1, 0, "1e-6", 8192], [256, 1, 128, 256, 32, 256, 0, 0, 0, "0", 512]]
    # the ABI tests' invalid configs, one field changed each
    for i, v in [(6, 7), (0, 0), (0, 1020), (1, 0), (2, 511), (3, 0), (3, 46341), (4, 0), (4, 65), (5, 12), (7, 2),
                 (10, 0), (10, 1 << 25), (2, 514)]:
        c = base[:]
        c[i] = v
        cases.append(c)
    for _ in range(n):
        c = base[:]
        for i in rng.choice(11, size=int(rng.integers(1, 4)), replace=False):
            c[i] = str(rng.choice(EPS)) if i == 9 else int(rng.choice(I64 if i == 10 else I32))
        cases.append(c)
    return [" ".join(["pkm"] + [str(x) for x in c]) for c in cases]


def _config(P, c):
    f = c.split()[1:]
    return P.pkm_config(*(int(x) for x in f[:9]), float(f[9]), int(f[10]))


def test_pkm_config_checks_and_layout_under_sanitizers(harness, P):
    rng = np.random.default_rng(0)
    cases = _pkm_cases(rng, 3000)
    out = harness(cases)
    kinds = {"ok": 0, "einval": 0, "eunsupported": 0}
    lib = P._lib._lib
    for c, v in zip(cases, out):
        kinds[v.split()[0]] += 1
        size = lib.pkm_workspace_size(ctypes.byref(_config(P, c)))
        if v.startswith("ok "):
            assert size == int(v.split()[1]), (c, v, size)
        else:
            code, why = v.split(" ", 1)
            assert size == 0 and P.pkm_last_error().endswith(why), (c, v, P.pkm_last_error())
            assert P.pkm_last_error().startswith("unsupported" if code == "eunsupported" else "invalid"), (c, v)
    assert min(kinds.values()) > 0, kinds


def test_engram_bag_and_ma_checks_under_sanitizers(harness, P):
    rng = np.random.default_rng(1)
    lib = P._lib._lib
    lines = []
    for _ in range(1500):
        e = [2, 2, 8, 128, 2097143, 128000, 1, 0, "1e-6", 16384, 4096]
        for i in rng.choice(11, size=int(rng.integers(1, 3)), replace=False):
            e[i] = str(rng.choice(EPS)) if i == 8 else int(rng.choice(I64 if i in (4, 9, 10) else I32))
        lines.append("engram " + " ".join(str(x) for x in e))
    for _ in range(800):
        b = [16384, 128, 16777216]
        for i in rng.choice(3, size=int(rng.integers(1, 3)), replace=False):
            b[i] = int(rng.choice(I32 if i == 1 else I64))
        lines.append("bag " + " ".join(str(x) for x in b))
    for _ in range(800):
        m = [32000, 2048, 32, "1e-6", 1]
        for i in rng.choice(5, size=int(rng.integers(1, 3)), replace=False):
            m[i] = str(rng.choice(EPS)) if i == 3 else int(rng.choice(I64 if i == 0 else I32))
        lines.append("mafold " + " ".join(str(x) for x in m))
    for _ in range(800):
        m = [32000, 2048, 1, 16384]
        for i in rng.choice(4, size=int(rng.integers(1, 3)), replace=False):
            m[i] = int(rng.choice(I64 if i in (0, 3) else I32))
        lines.append("mavalues " + " ".join(str(x) for x in m))
    out = harness(lines)
    assert {v.split()[0] for v in out} == {"ok", "einval"}
    reasons = {}
    for c, v in zip(lines, out):
        if v != "ok":
            reasons.setdefault(c.split()[0], set()).add(v.split(" ", 1)[1])
    assert set(reasons) == {"engram", "bag", "mafold", "mavalues"}
    dummy = ctypes.c_void_p(256)
    for c, v in zip(lines, out):
        f = c.split()
        kind, a = f[0], f[1:]
        if kind == "engram":
            cfg = P.engram_config(int(a[0]), int(a[1]), int(a[2]), int(a[3]), int(a[4]), int(a[5]), int(a[6]), int(a[7]),
                                  float(a[8]))
            # ids and mult given, rows NULL: the checks run, then a valid call stops at rows
            rc = lib.engram_hash(ctypes.byref(cfg), dummy, int(a[9]), int(a[10]), None, dummy, None, None)
        elif kind == "bag":
            rc = lib.pkm_bag_backward_workspace_size(int(a[0]), int(a[1]), int(a[2]))
            rc = -1 if rc == 0 else 0
        elif kind == "mafold":
            rc = lib.ma_fold_table(None, int(a[0]), int(a[1]), int(a[2]), None, ctypes.c_float(float(a[3])), int(a[4]),
                                   None, None)
        else:
            rc = lib.ma_values(None, int(a[0]), int(a[1]), int(a[2]), None, int(a[3]), None, None, None)
        msg = P.pkm_last_error()
        if v == "ok":
            # a valid call succeeds or stops past the checks (at a NULL data pointer, or at the
            # device, which a CPU run does not have), with a message that is no check's reason
            assert rc == P.PKM_OK or not any(msg.endswith(w) for w in reasons[kind]), (c, msg)
        else:
            why = v.split(" ", 1)[1]
            assert rc != P.PKM_OK and msg.endswith(why), (c, v, msg)
