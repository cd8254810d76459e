"""Sanitizer builds of the host code (no GPU needed).

* The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
  (errors fatal) runs the whole pin suite (tests/test_oracle_pins.py) through
  LCSI_ORACLE_LIB.
* The library's host code (csrc/api.hip: argument validation, workspace
  sizing, the F/S loop) built with host-only ASan + UBSan runs the C-ABI
  tests (tests/test_abi.py) through LCSI_LIB; its device code is the normal
  build's.
Both runs must end cleanly with no sanitizer report."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_sparse_idx_amd")


def _runtime(pattern):
    hits = sorted(glob.glob(pattern))
    return hits[-1] if hits else None


def _run_pytest(test_file, env_extra, preload):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", test_file, "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-4000:]
    return out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's libasan.so is not installed")
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-fPIC", "-shared", "-std=c11", "-D_GNU_SOURCE", "-Wall",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-o", lib, os.path.join(ROOT, "oracle", "lcsi_oracle.c"), "-lm", "-lpthread"], check=True)
    out = _run_pytest("tests/test_oracle_pins.py", {"LCSI_ORACLE_LIB": lib}, asan)
    assert "passed" in out


def test_abi_validation_under_host_asan_and_ubsan(tmp_path):
    rt = _runtime("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if rt is None or shutil.which("hipcc") is None:
        pytest.skip("hipcc or clang's ASan runtime is not installed")
    objs = [os.path.join(PKG, "_build", f"{s}.o") for s in ("score", "select", "attn", "overlap")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("build the library first (python -m long_context_sparse_idx_amd.build)")
    obj = str(tmp_path / "api_asan.o")
    lib = str(tmp_path / "liblcsi_asan.so")
    # sanitizers on the host pass only (device code is never instrumented)
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", obj], check=True, capture_output=True)
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, obj, *objs], check=True,
                   capture_output=True)
    out = _run_pytest("tests/test_abi.py", {"LCSI_LIB": lib}, rt)
    assert "passed" in out
