"""The boundary from plain C: include/dsv4.h compiles as C99 (gcc, -Wall
-Werror) and a C program linked against libdsv4.so runs its host-only calls
and argument checks (tests/c_abi/abi_check.c; no GPU is touched)."""
import os
import shutil
import subprocess

import pytest

import sparse_indexed_attention_amd as dsv4

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_c99_and_library_links_from_c(tmp_path):
    lib_dir = os.path.dirname(dsv4.LIB_PATH)
    assert os.path.exists(dsv4.LIB_PATH)
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi", "abi_check.c"),
           "-L", lib_dir, "-ldsv4", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: ok" in r.stdout
