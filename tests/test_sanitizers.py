"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):

- the oracle (oracle/razer_oracle.c), driven over every entry point, block
  size, scale format and mode, with zero, subnormal and non-finite tensors and
  rejected arguments (oracle/sanitize_driver.c);
- the C ABI's host-side argument checks (csrc/rz_api.cpp), linked against stub
  launchers, over rejected and accepted arguments of every entry point
  (csrc/host_check.cpp).

Each build stops at the first report (-fno-sanitize-recover=all), so a clean
exit status means no report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, tmp_path, what):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path)
    assert r.returncode == 0, f"{what} failed:\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc missing")
    exe = str(tmp_path / "rzo_san")
    _run(["gcc", "-std=c11", "-ffp-contract=off", "-Wall", *SAN, "-o", exe,
          os.path.join(ROOT, "oracle", "razer_oracle.c"), os.path.join(ROOT, "oracle", "sanitize_driver.c"),
          "-lm"], tmp_path, "oracle sanitizer build")
    r = _run([exe], tmp_path, "oracle under sanitizers")
    assert "sanitize_driver: ok" in r.stdout


def test_abi_checks_are_clean_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang missing")
    exe = str(tmp_path / "rz_hostcheck")
    csrc = os.path.join(ROOT, "nvfp4_razer_w4a16_amd", "csrc")
    # host-only C++ build (no offload): the checks in rz_api.cpp with stub launchers
    _run([CLANG, "-x", "c++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN, "-o", exe,
          os.path.join(csrc, "rz_api.cpp"), os.path.join(csrc, "host_check.cpp"),
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], tmp_path, "ABI sanitizer build")
    r = _run([exe], tmp_path, "ABI checks under sanitizers")
    assert "host_check: ok" in r.stdout
