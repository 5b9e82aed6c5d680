"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C ABI (``csrc/fa_api.cpp``: argument checks, size products, dispatch,
  workspace pointer derivation) is built with g++ together with stand-in
  launchers (``tests/sanitize/abi_stubs.cpp``) and driven over valid and
  invalid arguments by ``tests/sanitize/abi_driver.cpp``.
* The FP64 oracle (``oracle/oracle.c``) is built with gcc and the whole pin
  battery of ``tests/oracle_pins.py`` runs against that build, with the
  sanitizer runtimes preloaded into the Python process.
* A copy of the oracle with a planted out-of-bounds read shows that the
  sanitizer is live in that process.

Only host compilers are used here; no device code is built with a sanitizer.
"""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_flashattention_amd", "csrc")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="host compilers not available")


def _runtime_preload():
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                           text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            pytest.skip(f"{name} not found")
        libs.append(p)
    return ":".join(libs)


def _sanitized_env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime_preload()
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return env


def _build_oracle(src, out):
    subprocess.run(["gcc", *SAN, "-std=c11", "-shared", "-fPIC", "-pthread", src, "-o", out, "-lm"],
                   check=True, capture_output=True, text=True)


def test_c_abi_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(ROOT, "tests", "sanitize"),
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(ROOT, "tests", "sanitize", "abi_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "hip_runtime_api.h" in r.stderr:
        pytest.skip("HIP runtime headers not available")
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_oracle_pin_battery_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    _build_oracle(os.path.join(ROOT, "oracle", "oracle.c"), lib)
    r = subprocess.run([sys.executable, "-m", "tests.oracle_pins", lib], cwd=ROOT,
                       capture_output=True, text=True, timeout=600, env=_sanitized_env())
    assert r.returncode == 0, r.stderr[-4000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert json.loads(r.stdout.strip().splitlines()[-1]) == []


def test_sanitizer_is_live_in_the_battery(tmp_path):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    planted = src.replace("acc += qi[c] * kj[c];", "acc += qi[c] * kj[c + d];")
    assert planted != src
    path = tmp_path / "oracle_oob.c"
    path.write_text(planted)
    lib = str(tmp_path / "liboracle_oob.so")
    _build_oracle(str(path), lib)
    r = subprocess.run([sys.executable, "-m", "tests.oracle_pins", lib], cwd=ROOT,
                       capture_output=True, text=True, timeout=600, env=_sanitized_env())
    assert r.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in r.stderr
