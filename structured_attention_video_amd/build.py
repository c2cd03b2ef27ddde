"""Build libmonarch_attn.so in place with hipcc for gfx950.

Usage: python -m structured_attention_video_amd.build [--jobs N] [--hostsan]
Every call recompiles from source. Object files go to csrc/_build/ (the
host-sanitizer build: csrc/_build_hostsan/).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmonarch_attn.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Kernel sources only: no NaN-quieting around min/max (IEEE mode off). The
# C-ABI source keeps strict IEEE semantics for its argument checks.
KERNEL_FLAGS = ["-mno-amdgpu-ieee", "-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, obj: str, dflags=()) -> None:
    extra = KERNEL_FLAGS if os.path.basename(src).startswith("kernel_") else []
    cmd = [hipcc(), *FLAGS, *extra, *dflags, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(x for x in r.stderr.splitlines() if "packed-fp32-ops" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(jobs: int = 8, verbose: bool = True, out: str = OUT, defines=()) -> str:
    bdir = os.path.join(CSRC, "_build" + ("_" + "_".join(d.replace("=", "") for d in defines) if defines else ""))
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(bdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    dflags = [f"-D{d}" for d in defines]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda s_o: _compile(*s_o, dflags), zip(srcs, objs)))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


# Host-sanitizer build of the C-ABI layer (argument checks, plan arithmetic,
# workspace layout): its host code is built with AddressSanitizer and
# UndefinedBehaviorSanitizer (device code as usual), the kernels are linked
# unchanged. The library leaves the sanitizer runtime unresolved: load it into
# a process that preloads the clang ASan runtime (sanitizer_runtime()).
ABI_SOURCE = os.path.join(CSRC, "monarch_attn.hip")
SAN_DIR = os.path.join(CSRC, "_build_hostsan")
SAN_OUT = os.path.join(SAN_DIR, "libmonarch_attn_hostsan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize=vptr", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime that matches hipcc's host compiler."""
    base = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang")
    if not os.path.isdir(base):
        base = "/opt/rocm/llvm/lib/clang"
    for ver in sorted(os.listdir(base), reverse=True):
        cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise RuntimeError("clang ASan runtime not found")


def build_hostsan(jobs: int = 8, verbose: bool = True) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(SAN_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def one(s_o):
        s, o = s_o
        _compile(s, o, SAN_FLAGS if s == ABI_SOURCE else ())

    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(one, zip(srcs, objs)))
    tmp = SAN_OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, SAN_OUT)
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--out", default=OUT, help="output library path")
    ap.add_argument("-D", dest="defines", action="append", default=[], help="extra preprocessor define")
    ap.add_argument("--hostsan", action="store_true", help="build the host-sanitizer library instead")
    a = ap.parse_args()
    if a.hostsan:
        build_hostsan(a.jobs)
    else:
        build(a.jobs, out=a.out, defines=a.defines)
