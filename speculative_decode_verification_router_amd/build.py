"""Builds libmoeverify.so (all HIP sources under csrc/) for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libmoeverify.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU ops stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device target feature; that line is noise
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every csrc/*.hip and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, *extra_flags, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB_PATH + ".tmp"
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB_PATH)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
