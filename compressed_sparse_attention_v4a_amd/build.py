"""Build libv4a.so in-tree with hipcc for gfx950.

    python -m compressed_sparse_attention_v4a_amd.build

Objects go to _build/ at the repository root; the shared library is written
next to this file.  Every HIP source is compiled with packed-FP32 instruction
selection disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libv4a.so")
ARCH = os.environ.get("V4A_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for a checking build of the
# host code (argument validation, layouts, the C ABI); device code is compiled as usual.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(build_dir, src + ".o")
    cmd = [HIPCC] + COMMON + list(extra)
    if src.endswith(".hip"):
        cmd += ["-x", "hip"] + DEVICE
    else:
        cmd += DEVICE
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile every source and link the library.  sanitize=True builds the host code with
    ASan and UBSan (a checking build for the host tests, written to `out`)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    extra = HOST_SANITIZE if sanitize else []
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + extra + objs + [
        "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
