"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host-side code (no GPU).

* The oracle (plain C) is built with gcc -fsanitize=address,undefined and run by
  tests/sanitize/oracle_driver.c over every exported function, both build methods, both
  modes, the head variants, the sampling driver and the planted faults.
* The library's host code (validation, workspace and attention planning, argument
  rejection, the load policy) is compiled by hipcc with the sanitizers on the host side only
  (device code is never built with them) and run by tests/sanitize/abi_driver.c through
  calls that all return before anything reaches a device.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all) and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "draft_tree_construction_rank_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", *SAN, "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "dtree_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"), timeout=600)
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_library_host_code_under_asan_ubsan(tmp_path):
    srcs = ["abi", "build_kernels", "build_resident", "verify_kernels", "attn_kernels"]
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    procs = []
    for s in srcs:
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
               "-c", os.path.join(CSRC, s + ".hip"), "-o", str(tmp_path / (s + ".o"))]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    for cmd, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, "%s\n%s" % (" ".join(cmd), err[-4000:])
    lib = str(tmp_path / "libdtree_san.so")
    _run([CLANG + "++", "-shared", "-fPIC", "-fsanitize=address,undefined",
          *[str(tmp_path / (s + ".o")) for s in srcs], "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    exe = str(tmp_path / "abi_driver")
    _run([CLANG, "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"),
          os.path.join(HERE, "abi_driver.c"), lib, "-Wl,-rpath," + str(tmp_path), "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "abi driver: ok" in r.stdout
