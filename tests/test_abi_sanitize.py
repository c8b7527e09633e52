"""Sanitizer build of the C ABI's host code (no GPU): csrc/sma_api.hip is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer on its host
pass only (-Xarch_host; the device code is built as usual), linked with the
driver tests/sanitize/abi_driver.cpp against the library's kernels, and run.
The driver calls every entry point with arguments the validation rejects
and runs the workspace-size arithmetic at the extreme sizes it accepts; any
memory error or undefined behaviour aborts it, and each rejection must
return its documented status and message."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_mla_attention_index_amd")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not present")
def test_abi_layer_under_asan_and_ubsan():
    if not os.path.exists(os.path.join(PKG, "libsma.so")):
        pytest.skip("libsma.so not built")
    os.makedirs(OUT, exist_ok=True)
    obj = os.path.join(OUT, "sma_api_sanitized.o")
    exe = os.path.join(OUT, "abi_driver")
    inc = os.path.join(ROOT, "include")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument", *san, "-I", inc, "-c",
                    os.path.join(PKG, "csrc", "sma_api.hip"), "-o", obj], check=True, capture_output=True)
    # the driver is host C++ only
    host_san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    subprocess.run([CLANGXX, "-O1", "-g", "-std=c++17", *host_san, "-I", inc,
                    os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), obj, "-L", PKG, "-lsma",
                    "-L", "/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "abi_driver ok" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
    shutil.rmtree(OUT, ignore_errors=True)
