"""Build liblsh.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m lsh_sparse_attention_hash_amd.build

Each .hip source is compiled to an object in csrc/_build/ (in parallel), then
linked into lsh_sparse_attention_hash_amd/liblsh.so.
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "liblsh.so")
SOURCES = ["api.hip", "hash.hip", "sort.hip", "attend.hip", "combine.hip", "local.hip", "gemm.hip",
           "layer.hip"]
ARCH = "gfx950"
# Packed fp32 instructions are kept out of the generated code on purpose.
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


DIGEST = LIB + ".digest"
HEADERS = ["lsh_device.h", "lsh_launch.h"]


def source_digest() -> str:
    """Digest of everything the library is built from: the kernel and host
    sources, the internal headers, include/lsh.h and the compiler flags."""
    # include directories as paths relative to the repository, so that a copy
    # of the tree elsewhere (another machine) computes the same digest
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    flags = [os.path.relpath(f, root) if f in (INCLUDE, CSRC) else f for f in HIPFLAGS]
    h = hashlib.sha256(" ".join(flags).encode())
    paths = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [os.path.join(INCLUDE, "lsh.h")]
    for path in paths:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def is_current() -> bool:
    """liblsh.so exists and was built from the sources now in the tree."""
    try:
        with open(DIGEST) as f:
            return os.path.exists(LIB) and f.read().strip() == source_digest()
    except OSError:
        return False


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build liblsh.so")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    digest = source_digest()
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(DIGEST, "w") as f:
        f.write(digest + "\n")
    if verbose:
        print(f"built {LIB} (sources {digest})")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
