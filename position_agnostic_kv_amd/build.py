"""Build the lazyattn shared library for gfx950 with hipcc (in-tree).

``python -m position_agnostic_kv_amd.build`` compiles every ``csrc/*.hip`` (with
hipcc) and ``csrc/*.cpp`` (host-only code, with the host compiler) into ``_build/``
and links ``position_agnostic_kv_amd/liblazyattn.so``.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblazyattn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
    # packed FP32 instructions stay off in every device build
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


HOST_CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def host_sources():
    """Plain C++ host code (the cache manager), built with the host compiler."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".cpp"))


def build(verbose=False, jobs=None):
    """Compile and link; returns the library path.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    hsrcs = host_sources()
    hobjs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".host.o") for s in hsrcs]
    jobs = jobs or min(len(srcs) + len(hsrcs), os.cpu_count() or 4, 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [HIPCC, *FLAGS, "-c", s, "-o", o]) for s, o in zip(srcs, objs)]
        futs += [ex.submit(_run, [HOST_CXX, *HOST_FLAGS, "-c", s, "-o", o]) for s, o in zip(hsrcs, hobjs)]
        for f in futs:
            out = f.result()
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *hobjs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
