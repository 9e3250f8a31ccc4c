"""Memory and undefined-behaviour checks of the code that runs on the CPU.

* The oracle (oracle/lsh_oracle.c) is built with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer (halting on the first report) and the oracle pin
  tests run against that build in a child process.
* liblsh is rebuilt with clang's AddressSanitizer and UndefinedBehaviorSanitizer
  on its host side (argument validation, workspace sizing, launch set-up; the
  gfx950 device code is compiled as usual, without them) and the C-ABI host
  tests run against it in a child process.  Nothing is launched: those tests
  exercise every entry point's host path.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lsh_sparse_attention_hash_amd", "csrc")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]


def _run_child(tests, env, timeout=900):
    env = dict(os.environ, **env, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *tests]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    return out


def _gcc_asan():
    gcc = shutil.which("gcc")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip() if gcc else ""
    if not gcc or not os.path.isabs(asan):
        pytest.skip("gcc with libasan is not available")
    return gcc, asan


def _build_oracle(gcc, src, lib):
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                    "-ffp-contract=off", *SAN_FLAGS, src, "-o", lib, "-lm"], check=True)


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    gcc, asan = _gcc_asan()
    lib = str(tmp_path / "liblsh_oracle_san.so")
    _build_oracle(gcc, os.path.join(ROOT, "oracle", "lsh_oracle.c"), lib)
    _run_child(["tests/test_oracle_pins.py"], {"LSH_ORACLE_LIB": lib, "LD_PRELOAD": asan})


def test_the_sanitized_run_reports_a_planted_overflow(tmp_path):
    """The set-up above is live: a private copy of the oracle whose sort
    writes one key past its buffer is stopped by AddressSanitizer."""
    gcc, asan = _gcc_asan()
    src = open(os.path.join(ROOT, "oracle", "lsh_oracle.c")).read()
    bad = src.replace("for (int i = 0; i < len; ++i) { keys[i].bucket = bk[i];",
                      "for (int i = 0; i <= len; ++i) { keys[i].bucket = bk[i];", 1)
    assert bad != src
    path = tmp_path / "lsh_oracle_overflow.c"
    path.write_text(bad)
    lib = str(tmp_path / "liblsh_oracle_overflow.so")
    _build_oracle(gcc, str(path), lib)
    code = ("import numpy as np, sys; sys.path.insert(0, %r); from oracle import oracle; "
            "oracle.sort(np.zeros((1, 1, 1, 4096), np.int32))" % ROOT)
    env = dict(os.environ, LSH_ORACLE_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0",
               OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in r.stderr


def _clang_asan_runtime():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        return None, None
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path):
        # clang's resource directory: lib/linux under `-print-resource-dir`
        res = subprocess.run([hipcc, "-print-resource-dir"], capture_output=True,
                             text=True).stdout.strip()
        path = os.path.join(res, "lib", "linux", "libclang_rt.asan-x86_64.so")
    return hipcc, (path if os.path.exists(path) else None)


def test_library_host_side_under_address_and_undefined_sanitizers(tmp_path):
    hipcc, asan = _clang_asan_runtime()
    if not asan:
        pytest.skip("hipcc with clang's AddressSanitizer runtime is not available")
    sys.path.insert(0, ROOT)
    from lsh_sparse_attention_hash_amd import build as lib_build
    host_flags = []
    for f in SAN_FLAGS:
        host_flags += ["-Xarch_host", f]

    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        cmd = [hipcc, "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={lib_build.ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_flags,
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(lib_build.SOURCES)) as ex:
        objs = list(ex.map(compile_one, lib_build.SOURCES))
    lib = str(tmp_path / "liblsh_host_san.so")
    r = subprocess.run([hipcc, f"--offload-arch={lib_build.ARCH}", "-shared", "-fPIC", *objs,
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    _run_child(["tests/test_abi_host.py"], {"LSH_LIBRARY": lib, "LD_PRELOAD": asan})
