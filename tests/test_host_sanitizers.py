"""libqoq's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library sources are compiled with both sanitizers on their host side
(device code is compiled as usual; each source to an object of its own, in
parallel, reused while it is newer than its sources) and linked with
tests/sanitize/host_checks.cpp, which calls
every C-ABI entry point with invalid arguments, sweeps the size queries over
ordinary and extreme shapes, and runs the valid calls' host path up to the
launch (which fails without a GPU). Any out-of-bounds access, signed
overflow or other undefined behaviour in the host code stops the program.
Runs only where no GPU is visible.
"""
import os
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_integer_gemm_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="host-only build: the checks' fake pointers must never reach a GPU")
@pytest.mark.timeout(900)
def test_host_code_under_asan_and_ubsan():
    from concurrent.futures import ThreadPoolExecutor

    from bit_integer_gemm_amd import build as b
    hipcc = b.hipcc()
    os.makedirs(OUT, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = [os.path.join(CSRC, s) for s in b.SOURCES]
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"))
    objs, jobs = [], []
    for src in srcs:
        obj = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        if b._stale(obj, src):
            jobs.append([hipcc, *flags, *lang, "-c", src, "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, min(len(jobs), os.cpu_count() or 1))) as ex:
        results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), jobs))
    for r in results:
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    exe = os.path.join(OUT, "host_checks")
    res = subprocess.run([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                          "-Xarch_host", "-fsanitize=undefined", *objs, "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout[-4000:] + run.stderr[-4000:]
    assert run.stdout.strip().startswith("ok"), run.stdout
