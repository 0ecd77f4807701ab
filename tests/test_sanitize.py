"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code (CPU
only): the ABI layer (abi.cpp + plan.cpp, with the kernel launchers replaced
by host stubs from tests/sanitize/launch_stubs.cpp) and the fp64 oracle
(oracle/attn_oracle.c), driven through their argument checks, dispatch paths
and small problems in a child process with the ASan runtime preloaded. Any
report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_rope_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-O1", "-g"]


def _asan_runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(shutil.which("g++") is None or _asan_runtime() is None,
                    reason="needs g++ with the ASan runtime")
def test_host_code_under_sanitizers(tmp_path):
    abi = tmp_path / "libabi_san.so"
    subprocess.run(["g++", "-std=c++17", "-shared", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", os.path.join(CSRC, "abi.cpp"),
                    os.path.join(CSRC, "plan.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(abi)],
                   check=True)
    orc = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-shared", "-fPIC", "-fopenmp", *SAN,
                    os.path.join(ROOT, "oracle", "attn_oracle.c"), "-lm", "-o", str(orc)],
                   check=True)
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ATTN_ORACLE_LIB=str(orc),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "drive.py"),
                        str(abi)], env=env, capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert "abi paths ok" in r.stdout and "oracle paths ok" in r.stdout
