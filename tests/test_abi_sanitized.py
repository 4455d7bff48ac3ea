"""The C-ABI front end (sage_abi.hip: validation, workspace arithmetic,
aliasing checks, status strings) built with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code, the kernel launchers replaced by
stubs that report no device (tests/sanitized/stub_launch.cpp), running the host
ABI tests on the CPU. The GPU code is not sanitised (GPU sanitisers are not
used here); only the front end's host code is."""
import glob
import os
import shutil
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_attention_channel_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

pytestmark = [
    pytest.mark.skipif(not os.path.exists(HIPCC) or not ASAN_RT, reason="hipcc or the ASan runtime is missing"),
    pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-only test (stub launchers, fake addresses)"),
]


def test_host_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libsage_sanitized.so"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-Werror",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libasan",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-shared", "-o", str(lib),
           os.path.join(CSRC, "sage_abi.hip"), os.path.join(ROOT, "tests", "sanitized", "stub_launch.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, LD_PRELOAD=ASAN_RT[-1], ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1", SAGE_LIB_PATH=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0 and "Sanitizer" not in r.stdout + r.stderr, (r.stdout[-4000:] + r.stderr[-4000:])
