"""Build libdory.so (HIP for gfx950) in-tree: `python -m looped_ngpt_amd.build`.

Every source is compiled with hipcc for gfx950 only; packed-fp32 ops are
disabled for device code. Objects go to looped_ngpt_amd/_build/, the shared
library to looped_ngpt_amd/libdory.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdory.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _stale(src: str) -> bool:
    """The object is missing or older than its source or any header."""
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    heads = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    heads += [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    return any(os.path.getmtime(f) > t for f in [src, *heads])


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compiles every source (incremental: only those whose object is stale)
    and links libdory.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    todo = [s for s in srcs if _stale(s)] if incremental else srcs
    with cf.ThreadPoolExecutor(max_workers=max(1, min(8, len(todo)))) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    tmp = LIB + ".tmp"
    # --no-undefined: a symbol that a source failed to emit is a build error,
    # not a load-time one
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build(incremental="-i" in sys.argv[1:])
