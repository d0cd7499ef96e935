"""CPU tests under AddressSanitizer + UndefinedBehaviorSanitizer (host code only).

Two separately built, instrumented copies run the CPU tests that exercise them, each in a child
process with its sanitizer runtime preloaded (the Python interpreter itself is not instrumented):

* the fp64 oracle (oracle/oracle.c, gcc, ASan + UBSan) under its pins;
* the C-ABI host side of the library (csrc/fd_api.cpp, clang host pass only: argument checks,
  plans, workspace sizes, the scratch bookkeeping), linked with the normally built device
  objects, under the ABI tests.

UBSan findings abort (no recovery), ASan reports abort by default; leak checking is off (the
interpreter's own allocations are not ours).  Nothing here touches a GPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_attention_06_amd")
BUILD = os.path.join(PKG, "_build")


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan_runtime():
    for base in ("/opt/rocm/lib/llvm/lib/clang", "/opt/rocm/llvm/lib/clang"):
        if not os.path.isdir(base):
            continue
        for ver in sorted(os.listdir(base), reverse=True):
            p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(p):
                return p
    return None


def _run_child(env_extra, args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               **env_extra)
    # first prove the runtime is live in the child, then run the tests
    probe = subprocess.run([sys.executable, "-c", "import ctypes; ctypes.CDLL(None).__asan_init"],
                           env=env, capture_output=True, text=True, cwd=ROOT)
    assert probe.returncode == 0, f"sanitizer runtime not active in the child: {probe.stderr[-500:]}"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *args],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan and shutil.which("gcc")):
        pytest.skip("gcc sanitizer runtimes not available")
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-lpthread"], check=True)
    out = _run_child({"LD_PRELOAD": f"{asan}:{ubsan}", "ORACLE_LIB": lib},
                     ["tests/test_oracle_pins.py", "tests/test_oracle_window_pins.py",
                      "tests/test_oracle_append_pins.py"])
    assert "passed" in out


def test_abi_host_side_under_asan_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    objs = [os.path.join(BUILD, f + ".o") for f in ("fd_kernels.hip", "fd_wide.hip", "fd_direct.hip", "fd_append.hip",
                                                  "fd_check.hip")]
    if not rt or not os.path.exists(hipcc) or not all(os.path.exists(o) for o in objs):
        pytest.skip("clang ASan runtime, hipcc or the built device objects not available")
    api_o = str(tmp_path / "fd_api.o")
    lib = str(tmp_path / "libfd_asan.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
                    *san, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                    "-c", os.path.join(PKG, "csrc", "fd_api.cpp"), "-o", api_o],
                   check=True, capture_output=True)
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api_o, *objs,
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"],
                   check=True, capture_output=True)
    out = _run_child({"LD_PRELOAD": rt, "FD_LIB": lib}, ["tests/test_abi.py"])
    assert "passed" in out
