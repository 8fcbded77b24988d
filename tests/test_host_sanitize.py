"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libdsv4.so is compiled as the in-tree build compiles it, with
the host half instrumented (`-Xarch_host` before each sanitizer flag, so the
device code is untouched), into a library in a temporary folder.  Two plain C
programs linked against it then run:

  * tests/c_abi/abi_check.c, the host-only calls and argument checks;
  * tests/c_abi/host_sanitize_check.c, a seeded sweep of every entry point
    over boundary and extreme arguments (up to INT64_MAX, NULL and misaligned
    pointers, arbitrary cache structs), which checks return codes, error
    messages and untouched caller structs, and that each entry point both
    passes all of its checks and is refused at least once.

No GPU is used: the test runs only where none is visible, so every launch the
sweep reaches fails with DSV4_ERR_HIP before any device work.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from sparse_indexed_attention_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang"
# host half only: -Xarch_host right before each sanitizer flag
SAN = ("-Xarch_host -fsanitize=address,undefined "
       "-Xarch_host -fno-sanitize-recover=undefined "
       "-Xarch_host -fno-omit-frame-pointer").split()

pytestmark = [
    pytest.mark.skipif(os.path.exists("/dev/kfd"),
                       reason="needs a machine without a visible GPU (the sweep reaches launches)"),
    pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not available"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}{r.stderr}"


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san"))
    jobs = []
    for name in B.DEVICE_SOURCES:
        jobs.append([B.hipcc(), *B.COMMON, "-g", "-x", "hip", *B.DEVICE_FLAGS, *SAN, "-c",
                     os.path.join(B.CSRC, name), "-o", os.path.join(out, name + ".o")])
    for name in B.HOST_SOURCES:
        jobs.append([B.hipcc(), *B.COMMON, "-g", "-D__HIP_PLATFORM_AMD__", *SAN, "-c",
                     os.path.join(B.CSRC, name), "-o", os.path.join(out, name + ".o")])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(_run, jobs))
    _run([B.hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host",
          "-fsanitize=address,undefined", "-o", os.path.join(out, "libdsv4.so")]
         + [j[-1] for j in jobs])
    return out


def _build_and_run(lib_dir, source, exe_name):
    exe = os.path.join(lib_dir, exe_name)
    _run([CLANG, "-std=c99", "-Wall", "-Wextra", "-Werror", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), source, "-L", lib_dir, "-ldsv4",
          f"-Wl,-rpath,{lib_dir}", "-o", exe])
    env = dict(os.environ)
    # the HIP runtime's own start-up allocations are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_check_under_sanitizers(sanitized_lib):
    r = _build_and_run(sanitized_lib, os.path.join(HERE, "c_abi", "abi_check.c"), "abi_check")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: ok" in r.stdout


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_extreme_argument_sweep_under_sanitizers(sanitized_lib):
    r = _build_and_run(sanitized_lib, os.path.join(HERE, "c_abi", "host_sanitize_check.c"),
                       "host_sanitize_check")
    if r.returncode == 77:
        pytest.skip(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host_sanitize_check: ok" in r.stdout
