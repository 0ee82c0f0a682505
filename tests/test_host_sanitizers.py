"""The host validation layer under AddressSanitizer and UndefinedBehaviorSanitizer.

csrc/host.cpp (every argument check of the C ABI, the host-only history
selection, keep counts and byte counts) is compiled with g++
-fsanitize=address,undefined -fno-sanitize-recover=all. Its device launchers
are replaced by stubs that fail (tests/host_sanitize/launch_stubs.cpp), so
the library needs no GPU, and a case that reached a launch would show as
SA_E_HIP instead of its expected status. tests/test_abi_cpu.py then runs
against that library in a child process with the ASan runtime preloaded: an
out-of-bounds access, a use after free or undefined behaviour in any check
aborts the child and fails this test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _runtime(name):
    gxx = shutil.which("g++")
    if gxx is None:
        return None
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_checks_clean_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("g++ with libasan, or the HIP runtime library, is not installed")
    lib = tmp_path / "libsegattn.so"
    build = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer",
             os.path.join(ROOT, "diffusion_transformer_attention_segment_amd", "csrc", "host.cpp"),
             os.path.join(ROOT, "tests", "host_sanitize", "launch_stubs.cpp"),
             "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
             "-o", str(lib)]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, LD_PRELOAD=asan, SEGATTN_LIBRARY=str(lib),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",   # the interpreter's own leaks
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi_cpu.py"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
