"""Build the HIP library libpa.so for gfx950 with hipcc (in-tree)."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa.so")

SOURCES = ["pa_api.hip", "pa_store.hip", "pa_rope.hip", "pa_decode.hip", "pa_prefill.hip",
           "pa_prefix.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the prefill work-list claim is one atomic from one lane; without the
    # wave-level atomic rewrite its result is awaited only where it is used
    # (the next item), not right after the claim
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    return res.returncode, msgs


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source into libpa.so; returns its path.  Always recompiles.

    Each source becomes an object of its own (in parallel, they share no device
    code), then one link makes the library."""
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [hipcc(), *compile_flags, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
                           "-c", os.path.join(CSRC, s), "-o", obj]))
    if verbose:
        for _, cmd in jobs:
            print(" ".join(cmd), flush=True)
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as pool:
        results = list(pool.map(lambda j: _run(j[1]), jobs))
    failed = False
    for (obj, _), (rc, msgs) in zip(jobs, results):
        if rc != 0:
            failed = True
            sys.stderr.write("\n".join(msgs) + "\n")
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, msgs = _run(link)
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc link failed ({rc})")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
