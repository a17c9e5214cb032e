"""Build the gfx950 HIP library ``liblora_gemv.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblora_gemv.so")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "segments.hip", "kernels.hip", "batch_former.cpp", "status.cpp"]
# the host-only calls (lora_form_batch, lora_status_string), built apart with
# the host compiler under AddressSanitizer and UndefinedBehaviorSanitizer
HOST_SOURCES = ["batch_former.cpp", "status.cpp"]
HOST_SAN_LIB = os.path.join(HERE, "liblora_host_san.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
# the benchmark's read-ceiling kernel: a library of its own, outside the C ABI
READ_CEILING_SRC = "read_ceiling.hip"
READ_CEILING_LIB = os.path.join(HERE, "libread_ceiling.so")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-munsafe-fp-atomics",
    # packed fp32 (v_pk_*_f32) stays off: plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build_host_sanitized(verbose: bool = False) -> str:
    """The host-only calls as liblora_host_san.so: g++ with ASan + UBSan (no
    GPU code; loaded instead of liblora_gemv.so for them when LORA_SANITIZE=1)."""
    tmp = HOST_SAN_LIB + ".tmp"
    cmd = [os.environ.get("CXX", "g++"), "-std=c++17", "-fPIC", "-shared", "-Wall", *SANITIZE_FLAGS,
           "-I", INCLUDE, *[os.path.join(CSRC, f) for f in HOST_SOURCES], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("g++ failed on the sanitizer build of the host code")
    os.replace(tmp, HOST_SAN_LIB)
    if verbose:
        print(f"built {HOST_SAN_LIB}")
    return HOST_SAN_LIB


def _build_read_ceiling() -> None:
    tmp = READ_CEILING_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", os.path.join(CSRC, READ_CEILING_SRC), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {READ_CEILING_SRC}")
    os.replace(tmp, READ_CEILING_LIB)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link liblora_gemv.so, and the
    benchmark's libread_ceiling.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + 1) as ex:
        side = ex.submit(_build_read_ceiling)
        objs = list(ex.map(_compile, SOURCES))
        side.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_host_sanitized(verbose=True)
    else:
        build(verbose=True)
