"""Address and undefined-behaviour sanitizer builds of the host-side code (CPU only).

* The CPU oracle (oracle/qt_oracle.c) with gcc -fsanitize=address,undefined, driven
  through full, Talker-only and predictor-only frames of a tiny model in bf16 and
  INT8 modes (tests/sanitize/oracle_driver.c), leak detection on.
* The library's host code (configuration checks, buffer sizing, weight-table
  validation and its error paths, the scheduler's grouping rule) with the same
  sanitizers on the host side of a hipcc build, driven without a GPU
  (tests/sanitize/abi_driver.cpp).  The device code is built as usual.
A sanitizer report makes the driver exit non-zero."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "streaming_tts_decode_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{cmd[0]} failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "qt_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=ENV)
    assert "oracle driver ok" in r.stdout


def test_library_host_code_under_asan_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "abi_asan")
    srcs = [os.path.join(CSRC, f) for f in ("qt_abi.cpp", "qt_sched.cpp", "qt_kernels.hip",
                                             "qt_gemm.hip", "qt_pred.hip")]
    host_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", f]
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san + srcs +
         [os.path.join(HERE, "abi_driver.cpp"), "-o", exe])
    r = _run([exe], env=ENV)
    assert "abi driver ok" in r.stdout
