"""Build libdsv4.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m sparse_indexed_attention_amd.build

Each HIP source is compiled to an object for --offload-arch=gfx950, then
linked into ``sparse_indexed_attention_amd/libdsv4.so`` next to this file;
the benchmark's ceiling probes go into ``libdsv4_probe.so`` beside it.
Packed-fp32 instruction selection is disabled for every device compile.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsv4.so")
# ceiling probes for the benchmark (MFMA loop, copy), a library of their own
PROBE_LIB = os.path.join(HERE, "libdsv4_probe.so")
PROBE_SOURCES = ["peak_probe.hip"]

DEVICE_SOURCES = ["compress.hip", "indexer_score.hip", "topk.hip", "sparse_attn.hip",
                  "attn_h64.hip", "noalloc.hip"]
HOST_SOURCES = ["dsv4_api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}"]
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdsv4.so)")


def _compile(args):
    src, obj, device = args
    cmd = [hipcc(), *COMMON]
    cmd += (["-x", "hip", *DEVICE_FLAGS] if device else ["-D__HIP_PLATFORM_AMD__"])
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for name in DEVICE_SOURCES:
        jobs.append((os.path.join(CSRC, name), os.path.join(OBJ, name + ".o"), True))
    for name in HOST_SOURCES:
        jobs.append((os.path.join(CSRC, name), os.path.join(OBJ, name + ".o"), False))
    probe_jobs = [(os.path.join(CSRC, n), os.path.join(OBJ, n + ".o"), True) for n in PROBE_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs) + len(probe_jobs))) as ex:
        for out in ex.map(_compile, jobs + probe_jobs):
            if verbose and out.strip():
                print(out)
    for lib, objs in ((LIB, [j[1] for j in jobs]), (PROBE_LIB, [j[1] for j in probe_jobs])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
