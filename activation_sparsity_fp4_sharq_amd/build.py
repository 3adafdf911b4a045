"""Build libsharq.so (the HIP kernels and the C ABI of include/sharq.h) for gfx950.

Every source is compiled by hipcc for gfx950 only, with floating-point contraction
off (the NVFP4 steps are defined as separately rounded fp32 operations) and packed
fp32 instructions disabled.  The library lands next to this file, in-tree.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsharq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs, procs = [], []
    for src in sources():
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


def _drain(procs):
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops' is not a recognized feature" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif text.strip():
            print(text, file=sys.stderr)
    procs.clear()
    if failed:
        for src, text in failed:
            print(f"--- {src}\n{text}", file=sys.stderr)
        raise RuntimeError("hipcc failed for: " + ", ".join(s for s, _ in failed))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
