"""Build libhad.so (host C++ + gfx950 HIP kernels) in place.

Usage: python -m hybrid_attention_decode_amd.build [--jobs N] [--verbose]

Every .cpp under csrc/host and every .hip under csrc/kernels is compiled
with hipcc for gfx950 and linked into hybrid_attention_decode_amd/libhad.so.
The build always recompiles (it is also the "does it build" check).
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libhad.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(CSRC, "host"),
          "-Wall", "-Wno-unused-function"]
# Packed fp32 instructions are disabled for all device code.
HIP_FLAGS = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def sources():
    out = []
    for sub, ext in (("host", ".cpp"), ("kernels", ".hip")):
        d = os.path.join(CSRC, sub)
        for f in sorted(os.listdir(d)):
            if f.endswith(ext):
                out.append(os.path.join(d, f))
    return out


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.relpath(src, CSRC).replace(os.sep, "_") + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += HIP_FLAGS
    cmd += ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the device-only target feature: harmless
    msg = "\n".join(l for l in msg.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    return src, obj, r.returncode, msg


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, os.cpu_count() or 4)
    objs = []
    failed = []
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, obj, rc, msg in ex.map(lambda s: _compile(s, verbose), srcs):
            if msg:
                print(msg, file=sys.stderr, flush=True)
            if rc != 0:
                failed.append(src)
            objs.append(obj)
    if failed:
        raise RuntimeError("compilation failed: " + ", ".join(os.path.relpath(f, ROOT) for f in failed))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
