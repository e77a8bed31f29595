"""Address and undefined-behaviour sanitizers on the CPU side.

Two programs under tests/sanitize/ are built with -fsanitize=address,undefined
(host code only) and run here, without a GPU:

* the C oracle (oracle/kda_oracle.c) with a driver that runs small problems of
  every decay mode and dtype, thread counts and column ranges;
* the ABI layer's host side (kda_api.cpp: argument checks, the launch plan,
  workspace sizes, status strings, timing records) with a driver that makes
  only calls the host checks reject, empty problems and size queries; it is
  linked with the kernels' ordinary objects, which no call reaches.

Any sanitizer report ends the program with a non-zero status.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "linear_attention_sequence_kda_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
SAN = "-fsanitize=address,undefined"


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p


def test_oracle_under_asan_ubsan():
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", SAN, "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-pthread", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "kda_oracle.c"),
          "-o", exe, "-lm"])
    p = _run([exe], env=ENV)
    assert "ok" in p.stdout
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr


def test_abi_host_checks_under_asan_ubsan():
    from linear_attention_sequence_kda_amd import build as kbuild
    hipcc = kbuild.hipcc()
    os.makedirs(OUT, exist_ok=True)
    objdir = os.path.join(ROOT, "_build", "obj")
    kernels = [os.path.join(objdir, os.path.splitext(s)[0] + ".o")
               for s in kbuild.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kernels):
        kbuild.build()
    api = os.path.join(OUT, "kda_api_san.o")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    # host-only instrumentation: the sanitizer flags apply to the host pass
    _run([hipcc, f"--offload-arch={kbuild.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xarch_host", SAN, "-Xarch_host", "-fno-sanitize-recover=all",
          "-Xarch_host", "-fno-omit-frame-pointer"] + inc +
         ["-c", os.path.join(CSRC, "kda_api.cpp"), "-o", api])
    drv = os.path.join(OUT, "abi_driver.o")
    _run([hipcc, "-O1", "-g", "-x", "c", "-Xarch_host", SAN, "-Xarch_host",
          "-fno-sanitize-recover=all"] + inc + ["-c", os.path.join(HERE, "abi_driver.c"), "-o", drv])
    exe = os.path.join(OUT, "abi_driver")
    _run([hipcc, f"--offload-arch={kbuild.ARCH}", "-Xarch_host", SAN, drv, api] + kernels +
         kbuild.link_flags() + ["-o", exe])
    p = _run([exe], env=ENV)
    assert "ok" in p.stdout
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr
