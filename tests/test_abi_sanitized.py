"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled with the sanitizers on the host side only
(device code is built as usual and never run), linked with the C driver
tests/abi_sanitize_main.c, and run on the CPU: every entry point's
validation paths plus a seeded sweep of extreme sizes.  Any sanitizer report
(out-of-bounds access, leak, signed overflow, invalid shift, ...) aborts the
run and fails the test.
"""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "speculative_verify_isd_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANG),
                    reason="ROCm toolchain not available")
@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")),
                    reason="a preloaded library would precede the sanitizer runtime")
def test_abi_host_paths_are_sanitizer_clean(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    common = ["-O1", "-g", "-fno-omit-frame-pointer", "-I", INC]

    def compile_one(f):
        obj = str(tmp_path / (f + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fPIC", *common,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN,
               "-c", os.path.join(CSRC, f), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True)
        return obj

    with ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(compile_one, srcs))
    main_o = str(tmp_path / "main.o")
    subprocess.run([CLANG, *common, "-fsanitize=address,undefined", "-c",
                    os.path.join(HERE, "abi_sanitize_main.c"), "-o", main_o], check=True)
    exe = str(tmp_path / "abi_san")
    subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, main_o, *objs, "-o", exe], check=True,
                   capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout, r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "failures 0" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
