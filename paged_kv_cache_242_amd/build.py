"""Build libpa.so (the gfx950 HIP kernels behind the C ABI of include/pa.h) in-tree.

    python -m paged_kv_cache_242_amd.build        # or: python paged_kv_cache_242_amd/build.py

Each .hip source under csrc/ is compiled with hipcc for gfx950 in parallel, then linked into
paged_kv_cache_242_amd/libpa.so.  Packed fp32 VALU instructions are switched off for all device
code (-packed-fp32-ops).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa)")


def flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


# Per-source extras.  Without NaN semantics fmax needs no operand canonicalisation (fewer VALU per
# score in the prefill kernel).  NaN in the inputs still propagates: a GPU test puts a NaN in one
# visible cached K or V row and checks that exactly the output rows that see it come out NaN.
EXTRA_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [cc] + flags() + EXTRA_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only feature flag; that warning is harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if pr.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {', '.join(os.path.basename(f) for f in failed)}")
    tmp = OUT + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # hipcc's host pass can drop a kernel's launch stub without an error (e.g. when a device
    # builtin gets an argument type the host target rejects); the library would then fail only
    # when loaded.  Refuse to install such a library.
    nm = subprocess.run(["nm", "-C", "--undefined-only", tmp], check=True, capture_output=True, text=True)
    missing = [l.strip() for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs missing from the host code:\n  " + "\n  ".join(missing))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
