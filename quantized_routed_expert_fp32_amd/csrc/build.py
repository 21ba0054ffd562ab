"""Builds libmoe.so (HIP kernels for gfx950 + host C ABI) in-tree.

    python -m quantized_routed_expert_fp32_amd.csrc.build   (or build())

build_host_sanitized() builds _build/libmoe_hostsan.so: the host sources
(packer, layout arithmetic, C ABI validation) with AddressSanitizer and
UndefinedBehaviorSanitizer and the device entry points replaced by refusals
(host_stubs.cpp), for running the host tests sanitised without a GPU.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
OUT = os.path.join(PKG, "libmoe.so")
CEIL_OUT = os.path.join(PKG, "libmoe_ceilings.so")   # bench.py's MFMA ceiling probe
BUILD = os.path.join(PKG, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["route.hip", "decode.hip", "grouped.hip", "noalloc.hip"]
CXX_SOURCES = ["pack.cpp", "api.cpp"]
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
               "-munsafe-fp-atomics", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
             f"-I{ROCM}/include"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    jobs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        jobs.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(HERE, s), "-o", o])
    for s in CXX_SOURCES:
        o = os.path.join(BUILD, s.replace(".cpp", ".o"))
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(HERE, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(_run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = OUT + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
          f"-L{ROCM}/lib", "-lamdhip64", "-lpthread"])
    os.replace(tmp, OUT)
    # the benchmark's measured MFMA ceiling: a library of its own
    tmp = CEIL_OUT + ".tmp"
    _run([hipcc, *HIPCC_FLAGS, "-shared", "-o", tmp, os.path.join(HERE, "ceilings.hip"),
          f"-L{ROCM}/lib", "-lamdhip64"])
    os.replace(tmp, CEIL_OUT)
    if verbose:
        print("built", OUT)
    return OUT


SAN_OUT = os.path.join(BUILD, "libmoe_hostsan.so")
SAN_FLAGS = ["-O1", "-g", "-fPIC", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_host_sanitized(verbose=False):
    """The host-only sanitizer flavour (g++ only, no GPU code)."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    for s in CXX_SOURCES + ["host_stubs.cpp"]:
        o = os.path.join(BUILD, "san_" + s.replace(".cpp", ".o"))
        objs.append(o)
        jobs.append(["g++", *SAN_FLAGS, "-c", os.path.join(HERE, s), "-o", o])
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(_run, jobs))
    tmp = SAN_OUT + ".tmp"
    _run(["g++", "-shared", "-fsanitize=address,undefined", "-o", tmp, *objs, f"-L{ROCM}/lib", "-lamdhip64",
          "-lpthread"])
    os.replace(tmp, SAN_OUT)
    if verbose:
        print("built", SAN_OUT)
    return SAN_OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
