"""The library's host code (group planner, table and workspace layouts,
argument checks of every entry point) under AddressSanitizer and
UndefinedBehaviorSanitizer: tlc.hip is compiled with both on its host
code, linked with tests/sanitize/host_checks.cpp, and run on the CPU.  The
C++ program plans ragged groups (1 to 3000 tensors, sizes from 1 to 2^32-1 and
around tile, chunk and span boundaries) into exactly sized buffers, checks
the plans against the documented layout, and calls every entry point with
arguments that must be refused before any launch.  No GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.timeout(300)
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not installed")
    obj = tmp_path / "tlc_san.o"
    drv = tmp_path / "host_checks.o"
    exe = tmp_path / "host_checks"
    common = ["-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include")]
    # device code as in the product build; the sanitizers on the host code only
    subprocess.run([HIPCC, "--offload-arch=gfx950", *common, "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer", "-c", "-x", "hip",
                    os.path.join(ROOT, "gradient_compression_distributed_lc_amd", "csrc", "tlc.hip"),
                    "-o", str(obj)], check=True, capture_output=True)
    host_flags = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run([CLANG, *common, *host_flags, "-fno-omit-frame-pointer", "-c",
                    os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), "-o", str(drv)],
                   check=True, capture_output=True)
    subprocess.run([CLANG, *host_flags, str(drv), str(obj), "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
