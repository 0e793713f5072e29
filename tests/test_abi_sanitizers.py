"""The C ABI's host code (parameter validation, the plan's schedule
construction, the error paths) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: the library is rebuilt with the
sanitizers on its host code only (the device code is built as usual and
never runs here), the plain-C caller tests/c_abi/swattn_c_demo.c is built
with them too, and its `validate` mode must pass without a report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
# host code only: each sanitizer flag goes to the host compilation
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_validation_paths_are_clean_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libswattn.so"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN.split(),
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "sliding_window_attention_banded_amd", "csrc"),
                    os.path.join(ROOT, "sliding_window_attention_banded_amd", "csrc", "swattn.hip"),
                    "-o", str(lib)], check=True, capture_output=True, timeout=600)
    exe = tmp_path / "swattn_c_demo"
    subprocess.run([CLANG, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "swattn_c_demo.c"), "-o", str(exe),
                    "-L", str(tmp_path), "-lswattn", "-Wl,-rpath," + str(tmp_path),
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")],
                   check=True, capture_output=True, timeout=300)
    env = dict(os.environ)
    # the HIP runtime itself is not instrumented; its allocations are not ours
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([str(exe), "validate"], capture_output=True, text=True, timeout=120, env=env)
    report = res.stdout + res.stderr
    assert res.returncode == 0, report
    assert "validate: ok" in res.stdout
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
