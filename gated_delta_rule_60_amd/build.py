"""Build step for libkda.so: the gfx950 HIP kernels and the C ABI.

Run ``python -m gated_delta_rule_60_amd.build`` (or ``__graft_entry__.build()``).
The library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_CSRC = os.path.join(_HERE, "csrc")

SOURCES = ["kda_api.cpp", "kda_prefill.hip", "kda_segment.hip", "kda_decode.hip", "kda_backward.hip",
           "kda_bwd_chunk.hip", "kda_noalloc.hip", "kda_anymap.hip"]
ARCH = "gfx950"


def library_path() -> str:
    return os.path.join(_HERE, "libkda.so")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, obj: str, verbose: bool) -> None:
    is_hip = src.endswith(".hip")
    cmd = [hipcc(), "-c", "-O3", "-std=c++17", "-fPIC", "-Wall",
           f"--offload-arch={ARCH}",
           # hand-off of packed fp32 ops to the compiler is disabled on purpose
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(_ROOT, "include"), "-I", _CSRC]
    if is_hip:
        cmd += ["-x", "hip"]
    cmd += [src, "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build_library(verbose: bool = False, jobs: int = 3) -> str:
    """Compile every source for gfx950 and link libkda.so (always rebuilds)."""
    from concurrent.futures import ThreadPoolExecutor

    bdir = os.path.join(_ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    t0 = time.time()
    objs = []
    work = []
    for s in SOURCES:
        src = os.path.join(_CSRC, s)
        obj = os.path.join(bdir, s + ".o")
        objs.append(obj)
        work.append((src, obj))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda w: _compile(w[0], w[1], verbose), work))
    out = library_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} in {time.time() - t0:.1f}s", file=sys.stderr)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
