"""The host layer and the oracle under AddressSanitizer + UndefinedBehaviorSanitizer.

Two instrumented builds, each exercised in a subprocess of its own (the
clang and gcc sanitizer runtimes cannot share a process):

* the C-ABI library with its host code (argument validation, workspace
  layout, ``ssd_api.cpp``) compiled with ``-fsanitize=address,undefined``
  and linked with the already-built kernel objects; ``test_abi_host.py``
  runs against it (no GPU: the validators never dereference a pointer);
* the C oracle (``oracle/*.c``) built by gcc with the same sanitizers; the
  oracle pin tests run against it.

A report from either sanitizer aborts the subprocess, which fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_04_amd", "csrc")
OBJ = os.path.join(ROOT, "selective_state_space_04_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KERNEL_OBJS = ["ssd_kernels.o", "ssd_walk.o", "ssd_backward.o", "ssd_epilogue.o", "ssd_scan.o", "ssd_noalloc.o"]
SAN_OPTS = "detect_leaks=0:halt_on_error=1:abort_on_error=1"


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    if r.returncode != 0:
        pytest.fail(f"{' '.join(cmd[:4])} ... failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}")
    return r


def _clang_runtime(name):
    p = subprocess.run(["/opt/rocm/llvm/bin/clang", f"-print-file-name={name}"], capture_output=True,
                       text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_layer_under_sanitizers(tmp_path):
    if not all(os.path.exists(os.path.join(OBJ, o)) for o in KERNEL_OBJS):
        pytest.skip("kernel objects not built (run __graft_entry__.build())")
    asan = _clang_runtime("libclang_rt.asan-x86_64.so")
    if asan is None:
        pytest.skip("clang AddressSanitizer runtime not found")
    api = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libssd_san.so")
    # host code only (--offload-host-only); each sanitizer flag applies to the
    # host compilation alone
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-x", "hip",
          "--offload-host-only", *san, "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "ssd_api.cpp"), "-o", api])
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *[os.path.join(OBJ, o) for o in KERNEL_OBJS], api,
          *san, "-shared-libsan", "-o", lib])
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS=SAN_OPTS, UBSAN_OPTIONS="print_stacktrace=1",
               SSD_TEST_SANITIZED_LIB=lib)
    r = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
              os.path.join(ROOT, "tests", "test_abi_host.py")], env=env)
    assert " passed" in r.stdout, r.stdout[-2000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libssd_oracle_san.so")
    src = [os.path.join(ROOT, "oracle", f) for f in ("ssd_recurrence.c", "ssd_backward.c", "selective_scan.c")]
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-std=c11", *src, "-o", lib, "-lm"])
    libs = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
            for n in ("libasan.so", "libubsan.so")]
    env = dict(os.environ, LD_PRELOAD=":".join(libs), ASAN_OPTIONS=SAN_OPTS,
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", SSD_TEST_SANITIZED_ORACLE=lib,
               OMP_NUM_THREADS="4")
    pins = [os.path.join(ROOT, "tests", f) for f in
            ("test_oracle_pins.py", "test_oracle_backward_pins.py", "test_oracle_scan_pins.py")]
    r = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *pins], env=env)
    assert " passed" in r.stdout, r.stdout[-2000:]
