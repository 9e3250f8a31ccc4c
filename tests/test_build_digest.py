"""The library's source digest (recorded beside liblsh.so; tests, the smoke
check and the benchmark rebuild when it no longer matches the tree) must not
depend on where the tree is checked out: a copy of the repository on another
machine has to see the library built here as current."""
import os
import shutil
import subprocess
import sys

from lsh_sparse_attention_hash_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_digest_does_not_depend_on_the_checkout_path(tmp_path):
    copy = tmp_path / "elsewhere" / "repo"
    shutil.copytree(os.path.join(ROOT, "include"), copy / "include")
    shutil.copytree(os.path.join(ROOT, "lsh_sparse_attention_hash_amd"),
                    copy / "lsh_sparse_attention_hash_amd",
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    out = subprocess.run(
        [sys.executable, "-c",
         "from lsh_sparse_attention_hash_amd import build; print(build.source_digest())"],
        cwd=copy, capture_output=True, text=True, check=True).stdout.strip()
    assert out == lib_build.source_digest()
