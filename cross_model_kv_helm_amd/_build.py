"""Builds libhelmkv.so (the HIP library behind include/helm_kv.h) for gfx950.

All HIP sources are compiled with hipcc for gfx950 only, with packed-fp32
instruction selection disabled, and linked into one shared library next to
this file.  Nothing here imports torch.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhelmkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -Wno-inline-asm: the buffer->LDS copies set m0 themselves in inline assembly
# and name it as clobbered, which clang reports (once per inlined copy) as a
# reserved register in the clobber list.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-inline-asm",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(os.path.dirname(HERE), "include")]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 4) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the packed-fp32 feature flag; that note is harmless.
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    if p.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise subprocess.CalledProcessError(p.returncode, f"hipcc {src}")
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
