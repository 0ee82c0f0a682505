"""Build the HIP library (libsegattn.so) for gfx950 with hipcc, in-tree.

    python -m diffusion_transformer_attention_segment_amd.build

Compiles every source under csrc/ to an object in _build/ (at the repository
root) and links them into diffusion_transformer_attention_segment_amd/libsegattn.so.
A debug build of the same library, libsegattn_debug.so, differs only in its host
code (host.cpp with SA_DEBUG_CHECKS): device index lists are checked before
every launch that reads them, and attention outputs start as NaN canaries.
libsegattn_probe.so holds the MFMA throughput probes the bench reports
(csrc/mfma_probe.hip); it is not part of the segment-attention ABI.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsegattn.so")
DEBUG_LIB = os.path.join(PKG, "libsegattn_debug.so")
PROBE_LIB = os.path.join(PKG, "libsegattn_probe.so")
ARCH = "gfx950"

SOURCES = ["host.cpp", "kv_append.hip", "attention_bf16.hip", "attention_fp8.hip", "attention_combine.hip",
           "gather.hip", "sparse_select.hip", "camera.hip"]

# Packed-fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(exe):
        exe = shutil.which("hipcc")
    if not exe:
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return exe


def _compile(job):
    src, defines = job
    tag = "_debug" if defines else ""
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    lang = ["-x", "hip"]
    cmd = ([hipcc()] + COMMON + DEVICE_FLAGS + defines + lang +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj, out


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    assert SOURCES[0] == "host.cpp"   # the debug library swaps the first object
    jobs = ([(src, []) for src in SOURCES] + [("host.cpp", ["-DSA_DEBUG_CHECKS"])] +
            [("mfma_probe.hip", [])])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(_compile, jobs))
    for _, out in results:
        if verbose and out.strip():
            print(out)
    objs = [obj for obj, _ in results]
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link([objs[n]] + objs[1:n], DEBUG_LIB)
    _link([objs[n + 1]], PROBE_LIB)
    if verbose:
        print("built", LIB, DEBUG_LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
