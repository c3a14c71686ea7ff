"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer of the fp64
oracle and of the library's host-side validation (the race-detection /
sanitizer item of the test strategy, host code only: GPU sanitizers are not
available for the device code).

- oracle/helm_oracle.c with tests/sanitize/oracle_driver.c (gcc): every
  oracle entry point on tiny inputs, both storage types, valid and invalid
  arguments, leak detection on.
- cross_model_kv_helm_amd/csrc/api.hip recompiled with the sanitizers on its
  host code only, linked with the other objects of the last build into a
  separate library, driven by tests/sanitize/host_checks.cpp (clang, the
  same sanitizer runtime): status names, the arch gate, workspace sizes
  (including overflowing shapes), the mapper and paged-table checks and
  transfers refused before any enqueue.  No GPU is involved.

A sanitizer report or a wrong return value fails the test.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = {"UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, env_extra=None, cwd=None):
    env = dict(os.environ, **SAN_ENV, **(env_extra or {}))
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=cwd, timeout=300)
    out = p.stdout + p.stderr
    assert p.returncode == 0, f"{' '.join(cmd[:3])} ... exited {p.returncode}:\n{out[-4000:]}"
    return out


def _clean(out):
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "helm_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          "-o", exe, "-lm"])
    out = _run([exe], {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1"})
    _clean(out)
    assert "all calls as expected" in out


def test_library_host_validation_under_sanitizers(tmp_path):
    objs = [o for o in glob.glob(os.path.join(ROOT, "cross_model_kv_helm_amd", "_build", "*.hip.o"))
            if not o.endswith("api.hip.o")]
    if not os.path.exists(HIPCC) or not os.path.exists(CLANGXX) or len(objs) < 5:
        pytest.skip("needs hipcc, clang++ and the objects of a library build (run __graft_entry__.build())")
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libhelmkv_san.so")
    exe = str(tmp_path / "host_checks")
    inc = os.path.join(ROOT, "include")
    # the sanitizers apply to the host pass only (each flag after -Xarch_host)
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-inline-asm", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", inc, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(ROOT, "cross_model_kv_helm_amd", "csrc", "api.hip"), "-o", api_o])
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api_o, *objs, "-o", lib])
    _run([CLANGXX, "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-I", inc,
          os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), lib, "-Wl,-rpath," + str(tmp_path), "-o", exe])
    # leak detection off: the HIP runtime keeps allocations until exit
    out = _run([exe], {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"})
    _clean(out)
    assert "all calls as expected" in out
