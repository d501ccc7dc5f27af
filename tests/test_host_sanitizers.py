"""The C ABI's host code (argument validation, device queries, default unit
counts, workspace carving, the measurement hook) built with AddressSanitizer
and UndefinedBehaviorSanitizer and run on the CPU against a fake device and
fake kernel launchers (tests/sanitize/abi_host_check.cpp). No GPU."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _compile(src, obj):
    # host-only compilation: the sanitizers instrument host code only
    cmd = [HIPCC, "--offload-host-only", "-x", "hip", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "mla_decode_attention_amd", "csrc"),
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm toolchain")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    api = str(tmp_path / "api.o")
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "abi_host_check")
    _compile(os.path.join(ROOT, "mla_decode_attention_amd", "csrc", "mla_api.hip"), api)
    _compile(os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp"), drv)
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", api, drv, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
