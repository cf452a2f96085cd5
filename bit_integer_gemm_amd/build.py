"""Build libqoq.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_integer_gemm_amd.build

Flags: gfx950 only; -O3; no fast-math; no floating-point contraction (the
quantizers' fp32 products and divisions must round exactly like IEEE single
operations); correctly rounded fp32 division; packed-fp32 instructions
disabled in device code.

Each source is compiled to an object of its own (in parallel, under
`_build/`), then the objects are linked into the shared library; no kernel
calls a device function of another source, so no relocatable device code is
needed.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqoq.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")
SOURCES = ["abi.hip", "pack.hip", "act_quant.hip", "gemm.hip", "gemm_ksplit.hip", "gemm_wide.hip", "gemm_stream.hip", "variants.hip",
           "kv4.hip", "measure.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def _stale(obj: str, src: str) -> bool:
    """An object older than its source or than any header it may include."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [src] + [os.path.join(d, f) for d in (CSRC, INCLUDE) for f in os.listdir(d)
                    if f.endswith((".h", ".hpp"))]
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose: bool = False, jobs: int | None = None, force: bool = True) -> str:
    """Compile and link libqoq.so. force=False recompiles only the objects
    older than their source or a header (for quick rebuilds while editing)."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    objs, cmds = [], []
    for s in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o")
        src = os.path.join(CSRC, s)
        objs.append(obj)
        if force or _stale(obj, src):
            cmds.append([cc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
    jobs = jobs or min(max(1, len(cmds)), max(1, (os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    failed = [r for r in results if r.returncode != 0]
    for r in results:
        if r.returncode != 0 or (verbose and r.stderr.strip()):
            sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed compiling libqoq sources")
    tmp = LIB + ".tmp"
    res = _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp],
               verbose)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libqoq.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, force="--changed" not in sys.argv))
