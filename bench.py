"""Benchmark of the QoQ W4A8 GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads decode,...]

One step = the run-time hot path over the decode-shaped workload: for every
batch size M in {1, 8, 32, 64} (K = N = 4096, group 128), per-token INT8
quantization of the fp16 activations followed by the W4A8 GEMM with its
fused fp16 epilogue, as one qoq_w4a8_linear call (a single fused kernel for
M <= 8, the quantizer and the GEMM for larger M). The weights are quantized and packed once before timing
(they are static in serving); that offline step is timed separately under
"pack". Each GEMM launch reads a different copy of the packed weights and
the copies together exceed 512 MiB, twice the 256 MiB last-level cache, so
every GEMM streams its weights from HBM.

Timing: each step is captured once per weight copy set into a HIP graph; K
graph launches are timed with events on the capture stream. While the host
enqueues, a spin kernel keeps the GPU busy, so launch overhead on the host
never shows up as idle GPU time inside the timed region. Per-kernel
durations of the GEMM kernels (the dominant kernels: the fused kernel for
M <= 8, the GEMM for larger M) are taken the same way: one event pair around
many back-to-back launches, divided by their number.

The other workloads (Llama-3-8B layers at M=256, the M=4096 prefill GEMM,
Qwen1.5-72B layers at M=64 and M=1024) are timed GEMM by GEMM and listed
under "shapes" with their roofline fractions.

Prints ONE JSON line. Only one GPU is used: --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5033.2        # dense INT8 MFMA: 256 CU x 8192 ops/clk x 2.4 GHz
ROTATE_BYTES = 512 << 20       # weight copies per shape: twice the last-level cache
METRIC = "W4A8 GEMM TOPS + % roofline (HBM at M≤64, INT8 MFMA at M≥1024)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a8_gemm_traffic_decode_step.json")
CSRC_DIR = os.path.join(ROOT, "bit_integer_gemm_amd", "csrc")
# the sources whose kernels the decode step launches (the counters are only
# valid for the kernels they were taken on)
GEMM_SOURCES = ("gemm.hip", "gemm_ksplit.hip", "gemm_wide.hip", "gemm_stream.hip",
                "act_quant.hip", "kernel_common.hpp", "qoq_internal.hpp")


def gemm_sources_sha256():
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        h.update(open(os.path.join(CSRC_DIR, name), "rb").read())
    return h.hexdigest()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workloads", default="decode,llama3_8b,prefill,qwen15_72b",
                   help="comma list; the decode step is always the headline")
    p.add_argument("--shape-iters", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the W8A8 / W4A4 / W4A16 comparison GEMMs")
    p.add_argument("--no-kv4", action="store_true",
                   help="skip the KV4 decode-attention workloads")
    p.add_argument("--kv4-workloads", default=",".join(KV4_WORKLOADS),
                   help="comma list of KV4 decode-attention workloads")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
class Blocker:
    """A spin kernel that keeps the GPU busy while the host enqueues."""

    def __init__(self, torch):
        self.torch = torch
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cycles = 2_000_000
        torch.cuda._sleep(cycles)  # warm
        a.record()
        torch.cuda._sleep(cycles)
        b.record()
        torch.cuda.synchronize()
        self.s_per_cycle = a.elapsed_time(b) * 1e-3 / cycles

    def run(self, enqueue, guess_s):
        """Run `enqueue` behind a spin of about 2 x guess_s; returns the host
        enqueue time and whether the spin outlasted it."""
        torch = self.torch
        for _ in range(4):
            torch.cuda.synchronize()
            spin = max(1e-3, 2.0 * guess_s)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            torch.cuda._sleep(int(spin / self.s_per_cycle))
            b.record()
            t0 = time.perf_counter()
            res = enqueue()
            host = time.perf_counter() - t0
            torch.cuda.synchronize()
            if host < a.elapsed_time(b) * 1e-3:
                return res, host, True
            guess_s = 2 * host
        return res, host, False


def event_pairs(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def per_launch_times(torch, blocker, fns, iters):
    """Mean duration of each callable: one event pair around `iters`
    back-to-back launches (enqueued behind the spin kernel), divided by
    `iters`. Each entry of `fns` is a callable or a list of callables used
    round robin (e.g. one per rotated weight copy)."""
    out = []
    for fn in fns:
        seq = fn if isinstance(fn, (list, tuple)) else [fn]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def enqueue():
            a.record()
            for it in range(iters):
                seq[it % len(seq)]()
            b.record()

        blocker.run(enqueue, 30e-6 * iters)
        out.append(a.elapsed_time(b) * 1e-3 / iters)
    return out


# ---------------------------------------------------------------------------
def to_half_device(torch, X, dev):
    return torch.from_numpy(X.view(np.uint16)).view(torch.float16).to(dev)


def rotated_copies(pw, min_bytes=ROTATE_BYTES, max_copies=512, multiple=1):
    n = int(min(max_copies, max(2, -(-min_bytes // pw.packed.numel()))))
    n = -(-n // multiple) * multiple
    return [pw.packed] + [pw.packed.clone() for _ in range(n - 1)]


class GemmCall:
    """A prepared qoq_w4a8_gemm call (pointers resolved once)."""

    def __init__(self, qoq, torch, x8, s_x, packed, s1, N, y, ws):
        M, K = s_x.shape[0], x8.shape[1] * 16
        self.f = qoq.lib().qoq_w4a8_gemm
        wsb = qoq.qoq_gemm_workspace_bytes(M, N, K)
        wsp = None
        if wsb:
            buf = ws.get(wsb)
            wsp, wsb = buf.data_ptr(), buf.numel()
        self.args = (x8.data_ptr(), s_x.data_ptr(), M, K, packed.data_ptr(), s1.data_ptr(), N,
                     128, y.data_ptr(), None, wsp, wsb)
        self.torch = torch

    def __call__(self):
        st = self.f(*self.args, self.torch.cuda.current_stream().cuda_stream)
        if st:
            raise RuntimeError(f"qoq_w4a8_gemm failed with status {st}")


class ActCall:
    def __init__(self, qoq, torch, x, x8, s_x):
        M, K = x.shape
        self.f = qoq.lib().qoq_quantize_act
        self.args = (x.data_ptr(), M, K, x8.data_ptr(), s_x.data_ptr())
        self.torch = torch

    def __call__(self):
        st = self.f(*self.args, self.torch.cuda.current_stream().cuda_stream)
        if st:
            raise RuntimeError(f"qoq_quantize_act failed with status {st}")


class LinearCall:
    """A prepared qoq_w4a8_linear call (activation quantization + GEMM)."""

    def __init__(self, qoq, torch, x, packed, s1, N, y, ws):
        M, K = x.shape
        self.f = qoq.lib().qoq_w4a8_linear
        wsb = qoq.qoq_linear_workspace_bytes(M, N, K)
        wsp = None
        if wsb:
            buf = ws.get(wsb)
            wsp, wsb = buf.data_ptr(), buf.numel()
        self.args = (x.data_ptr(), M, K, packed.data_ptr(), s1.data_ptr(), N, 128, y.data_ptr(),
                     None, wsp, wsb)
        self.torch = torch

    def __call__(self):
        st = self.f(*self.args, self.torch.cuda.current_stream().cuda_stream)
        if st:
            raise RuntimeError(f"qoq_w4a8_linear failed with status {st}")


def fused_bytes(M, K, N, group=wl.GROUP):
    """HBM bytes the fused kernel must move: the weights as for the GEMM,
    the fp16 activations (no INT8 copy, no token scales) and the output."""
    return N * K // 2 + (N * K // group) * 3 // 2 + 2 * N + 2 * M * K + 2 * M * N


def traffic_record():
    """HBM bytes per decode GEMM launch from the committed rocprofv3 counter
    runs, if they were taken on the current GEMM sources (SHA-256 over
    GEMM_SOURCES); else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("gemm_sources_sha256") != gemm_sources_sha256():
        return None
    return rec


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the GEMM would shard by output columns, or by K with an exact INT32 sum); "
              "rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_integer_gemm_amd as qoq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    work = [w for w in args.workloads.split(",") if w and w != "decode"]
    blocker = Blocker(torch)

    # ---------------- headline step: decode workload ----------------
    dw = wl.WORKLOADS["decode"]
    shape = dw.shapes[0]
    K, N = shape.K, shape.N
    W, _, _ = wl.make_case(dw, shape, 1)
    Wd = torch.from_numpy(W).to(dev)
    pw = qoq.pack_weights(Wd)
    torch.cuda.synchronize()
    pack_t = per_launch_times(torch, blocker, [lambda: qoq.pack_weights(Wd)], 5)[0]
    n_m = len(dw.Ms)
    copies = rotated_copies(pw, multiple=n_m)
    ws = qoq.Workspace(dev)
    per_m = []
    for M in dw.Ms:
        _, Xm, _ = wl.make_case(dw, shape, M)
        c = dict(M=M, x=to_half_device(torch, Xm, dev),
                 x8=qoq.empty_act(M, K, dev),
                 s_x=torch.empty(M, dtype=torch.float32, device=dev),
                 y=torch.empty((M, N), dtype=torch.float16, device=dev),
                 fused=qoq.qoq_linear_path(M, N, K) == 1)
        c["act"] = ActCall(qoq, torch, c["x"], c["x8"], c["s_x"])
        per_m.append(c)
    # step j uses copies [n_m*j, n_m*j + n_m); each M is one qoq_w4a8_linear
    # call: a single fused launch for M <= 8, quantizer + GEMM otherwise
    n_phase = len(copies) // n_m
    phases = []
    for j in range(n_phase):
        phases.append([LinearCall(qoq, torch, c["x"], copies[n_m * j + i], pw.s1, N, c["y"], ws)
                       for i, c in enumerate(per_m)])

    def eager_step(j):
        for lin in phases[j % n_phase]:
            lin()

    # capture the steps into HIP graphs on torch's capture stream: one graph
    # of all K timed steps when K <= 64 (each replay of a graph costs about
    # 2 us of its own, which a model's decode step, hundreds of kernels in one
    # graph, spreads much thinner than a 6-kernel step could), else graphs of
    # G = gcd(K, phases) consecutive steps; replaying K/G graphs times exactly
    # K steps, and the untimed warm-up rounds up to whole graphs
    G = args.steps if args.steps <= 64 else math.gcd(args.steps, n_phase)
    for j in range(n_phase):
        eager_step(j)
    torch.cuda.synchronize()
    graphs = []
    for g0 in range(0, n_phase if G < args.steps else 1, G):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(g0, g0 + G):
                eager_step(j)
        graphs.append(g)
    torch.cuda.synchronize()

    for i in range(-(-args.warmup // G)):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed_graph_steps():
        start.record()
        for i in range(args.steps // G):
            graphs[i % len(graphs)].replay()
        end.record()

    _, host_s, covered = blocker.run(timed_graph_steps, 30e-6 * args.steps)
    step_s = start.elapsed_time(end) * 1e-3 / args.steps
    sclk_after = gpu_sclk_mhz()

    def timed_eager_steps():
        start.record()
        for i in range(args.steps):
            eager_step(i)
        end.record()

    blocker.run(timed_eager_steps, 8 * 40e-6 * args.steps)
    eager_step_s = start.elapsed_time(end) * 1e-3 / args.steps

    ops_step = sum(wl.algorithmic_ops(c["M"], K, N) for c in per_m)
    value_tops = ops_step / step_s / 1e12

    # per-launch durations of the dominant kernel, rotating over the weight
    # copies like the step does: the fused kernel for M <= 8, the GEMM
    # kernel (on the quantizer's output) for larger M; and the quantizer
    iters = max(128, n_phase)
    kern = []
    for i, c in enumerate(per_m):
        if c["fused"]:
            kern.append([phases[j][i] for j in range(n_phase)])
        else:
            c["act"]()
            kern.append([GemmCall(qoq, torch, c["x8"], c["s_x"], copies[n_m * j + i], pw.s1, N,
                                  c["y"], ws) for j in range(n_phase)])
    kern_t = per_launch_times(torch, blocker, kern, iters)
    # the plain GEMM kernel on the quantizer's output, also for the fused M
    # (the two-call path of the same step), for comparison
    for c in per_m:
        c["act"]()
    gemm_only_t = per_launch_times(
        torch, blocker, [[GemmCall(qoq, torch, c["x8"], c["s_x"], copies[n_m * j + i], pw.s1, N,
                                   c["y"], ws) for j in range(n_phase)]
                         for i, c in enumerate(per_m)], iters)
    gemm_only_achieved = (sum(wl.algorithmic_bytes(c["M"], K, N) for c in per_m) /
                          sum(gemm_only_t) / 1e9)
    unfused = [c for c in per_m if not c["fused"]]
    act_t = dict(zip([c["M"] for c in unfused],
                     per_launch_times(torch, blocker, [c["act"] for c in unfused], iters)))
    lin_t = per_launch_times(torch, blocker, [[phases[j][i] for j in range(n_phase)]
                                              for i in range(n_m)], iters)
    kern_bytes = [fused_bytes(c["M"], K, N) if c["fused"] else wl.algorithmic_bytes(c["M"], K, N)
                  for c in per_m]
    achieved = sum(kern_bytes) / sum(kern_t) / 1e9
    shapes_out = []
    for c, t, tl, b, tg in zip(per_m, kern_t, lin_t, kern_bytes, gemm_only_t):
        ops = wl.algorithmic_ops(c["M"], K, N)
        rec = dict(workload="decode", shape="square", M=c["M"], K=K, N=N,
                   path="fused" if c["fused"] else "two-call",
                   gemm_us=round(t * 1e6, 3))
        if not c["fused"]:
            rec["act_quant_us"] = round(act_t[c["M"]] * 1e6, 3)
        else:
            rec["gemm_only_us"] = round(tg * 1e6, 3)
        rec.update(linear_us=round(tl * 1e6, 3), tops=round(ops / t / 1e12, 3),
                   gbs=round(b / t / 1e9, 1), hbm_frac=round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                   mfma_frac=round(ops / t / 1e12 / INT8_PEAK_TOPS, 4))
        shapes_out.append(rec)

    # streaming-copy reference (a plain elementwise kernel: read N bytes, write
    # N bytes) of the decode weight size and of 1 GiB; its counters calibrate
    # the HBM-traffic counters of the GEMM. The decode-size copy rotates over
    # >= 512 MiB of buffers like the GEMM, so it reads HBM, not the cache.
    copy_ref = {}
    for label, nbytes in (("decode_weights", pw.packed.numel()), ("1GiB", 1 << 30)):
        n = max(1, -(-ROTATE_BYTES // nbytes))
        bufs = [(torch.empty(nbytes, dtype=torch.uint8, device=dev),
                 torch.empty(nbytes, dtype=torch.uint8, device=dev)) for _ in range(n)]
        calls = [(lambda a=a, b=b: torch.bitwise_not(a, out=b)) for a, b in bufs]
        t = per_launch_times(torch, blocker, [calls], max(20, n))[0]
        copy_ref[label] = {"bytes": nbytes, "us": round(t * 1e6, 3),
                           "gbs": round(2 * nbytes / t / 1e9, 1)}
        del bufs, calls
    # streaming-read reference of the decode weight size: the library's plain
    # read kernel (16-byte loads, 4 in flight per thread), same rotation, at
    # several grid sizes; the fastest is the achievable single-launch rate
    nbytes = pw.packed.numel()
    n = max(1, -(-ROTATE_BYTES // nbytes))
    rbufs = [torch.zeros(nbytes, dtype=torch.uint8, device=dev) for _ in range(n)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    by_grid = {}
    for wgs in (256, 512, 1024, 2048):
        def rd(a, wgs=wgs):
            st = qoq.qoq_stream_read(a.data_ptr(), nbytes, wgs, sink.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
            if st:
                raise RuntimeError(f"qoq_stream_read failed with status {st}")
        t = per_launch_times(torch, blocker, [[(lambda a=a: rd(a)) for a in rbufs]], max(20, n))[0]
        by_grid[wgs] = round(t * 1e6, 3)
    best = min(by_grid.values())
    read_ref = {"decode_weights": {"bytes": nbytes, "us": best,
                                   "gbs": round(nbytes / (best * 1e-6) / 1e9, 1),
                                   "us_by_workgroups": by_grid}}
    del rbufs

    # ---------------- other workloads, GEMM by GEMM ----------------
    del copies, phases, graphs
    torch.cuda.empty_cache()
    for key in work:
        w = wl.WORKLOADS[key]
        for shp in w.shapes:
            Wk, _, _ = wl.make_case(w, shp, 1)
            pwk = qoq.pack_weights(torch.from_numpy(Wk).to(dev))
            del Wk
            ck = rotated_copies(pwk)
            for M in w.Ms:
                _, Xk, _ = wl.make_case(w, shp, M)
                xk8, sk = qoq.quantize_act(to_half_device(torch, Xk, dev))
                yk = torch.empty((M, shp.N), dtype=torch.float16, device=dev)
                calls = [GemmCall(qoq, torch, xk8, sk, cp, pwk.s1, shp.N, yk, ws) for cp in ck]
                for cl in calls[:3]:
                    cl()
                t = per_launch_times(torch, blocker, [calls], max(args.shape_iters, len(calls)))[0]
                ops = wl.algorithmic_ops(M, shp.K, shp.N)
                b = wl.algorithmic_bytes(M, shp.K, shp.N)
                t_floor = max(b / (HBM_PEAK_GBS * 1e9), ops / (INT8_PEAK_TOPS * 1e12))
                shapes_out.append(dict(workload=key, shape=shp.name, M=M, K=shp.K, N=shp.N,
                                       gemm_us=round(t * 1e6, 3), tops=round(ops / t / 1e12, 3),
                                       gbs=round(b / t / 1e9, 1),
                                       hbm_frac=round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                                       mfma_frac=round(ops / t / 1e12 / INT8_PEAK_TOPS, 4),
                                       roofline_frac=round(t_floor / t, 4)))
            del ck, pwk
            torch.cuda.empty_cache()

    variants = None if args.no_variants else variant_comparison(torch, qoq, blocker, dev, ws,
                                                                args.shape_iters)
    kv4 = None if args.no_kv4 else kv4_attention_bench(torch, qoq, blocker, dev, ws,
                                                       args.shape_iters,
                                                       args.kv4_workloads.split(","))
    cpu = None if args.no_cpu_baseline else cpu_baseline(dw, shape, args.cpu_seconds)
    traffic = traffic_record()

    out = {
        "metric": METRIC,
        "value": round(value_tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode-shaped W4A8 GEMM step: per-token INT8 activation "
                               "quantization + W4A8 GEMM for M in {1,8,32,64}, K=N=4096, "
                               "group 128, weights HBM-resident (rotated copies); one "
                               "qoq_w4a8_linear call per M (fused kernel for M<=8)",
                   "M": list(dw.Ms), "K": K, "N": N, "group": 128,
                   "weight_copies": n_phase * n_m},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "kernel": "W4A8 GEMM kernels of the step (fused quantize+GEMM for "
                               "M=1,8; GEMM for M=32,64): sum of algorithmic bytes / sum of "
                               "mean event-timed launch durations"},
        "gemm_only_roofline": {"achieved": round(gemm_only_achieved, 1),
                               "frac": round(gemm_only_achieved / HBM_PEAK_GBS, 4),
                               "kernel": "the GEMM kernel alone on quantized input, M=1,8,32,64 "
                                         "(two-call path)"},
        "cpu_baseline": cpu,
        "step_eager_ms": round(eager_step_s * 1e3, 6),
        "steps_per_graph": G,
        "host_enqueue_covered": covered,
        "pack": {"N": N, "K": K, "us": round(pack_t * 1e6, 1),
                 "weights_per_s": round(N * K / pack_t, 1),
                 "fp32_read_gbs": round(N * K * 4 / pack_t / 1e9, 1)},
        "copy_reference": copy_ref,
        "read_reference": read_ref,
        "shapes": shapes_out,
        "variants": variants,
        "kv4_attention": kv4,
        "host_cores": len(os.sched_getaffinity(0)),
        "device": torch.cuda.get_device_name(dev),
        "platform": {**platform_info(), "sclk_mhz_after_timed_steps": sclk_after},
    }
    print(json.dumps(out), flush=True)


KV4_WORKLOADS = ("llama3_8b_attn", "qwen15_72b_attn", "llama3_8b_long")


def kv4_attention_bench(torch, qoq, blocker, dev, ws, iters, keys=KV4_WORKLOADS):
    """Decode attention over the 4-bit KV cache (SmoothAttention-scaled
    queries), one call per workload: algorithmic bytes (4-bit codes with an
    fp16 scale and a 4-bit zero per cached vector, queries, outputs) over the
    mean launch time, against the HBM peak. The caches rotate over copies
    totalling >= 512 MiB so every call reads from HBM."""
    out = []
    for key in keys:
        w = wl.ATTN_WORKLOADS[key]
        q, k, v, lens = wl.make_attention_case(w)
        C = int(-(-int(lens.max()) // 32) * 32)
        kd = torch.from_numpy(k.view(np.uint16)).view(torch.float16).to(dev)
        vd = torch.from_numpy(v.view(np.uint16)).view(torch.float16).to(dev)
        del k, v
        lam = qoq.kv4_smooth_factors(kd[:4].reshape(-1, w.H_kv, w.D))
        cache = qoq.kv4_alloc_cache(w.B, w.H_kv, C, dev)
        zeros = torch.zeros(w.B, dtype=torch.int32, device=dev)
        qoq.kv4_append(kd, vd, lam, zeros, cache, C)
        cache16 = qoq.kv16_alloc_cache(w.B, w.H_kv, C, dev)
        qoq.kv16_append(kd, vd, zeros, cache16, C)
        del kd, vd
        n_copies = int(min(64, max(2, -(-ROTATE_BYTES // cache.numel()))))
        caches = [cache] + [cache.clone() for _ in range(n_copies - 1)]
        qd = torch.from_numpy(q.view(np.uint16)).view(torch.float16).to(dev)
        lens_d = torch.from_numpy(lens).to(dev)
        o = torch.empty_like(qd)
        max_len = int(lens.max())
        L = qoq.lib()
        wsb = int(L.qoq_kv4_attention_workspace_bytes(w.B, w.H, w.H_kv, w.D, max_len))
        wsp = None
        if wsb:
            buf = ws.get(wsb)
            wsp, wsb = buf.data_ptr(), buf.numel()
        st = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
        calls = [lambda c=c: L.qoq_kv4_decode_attention(qd.data_ptr(), w.B, w.H, w.H_kv, w.D,
                                                        lam.data_ptr(), c.data_ptr(), C,
                                                        lens_d.data_ptr(), max_len, o.data_ptr(),
                                                        wsp, wsb, st()) for c in caches]
        for cl in calls[:2]:
            rc = cl()
            if rc:
                raise RuntimeError(f"kv4 attention: {qoq.qoq_status_string(rc)}")
        t = per_launch_times(torch, blocker, [calls], max(iters, len(calls)))[0]
        # the same attention on an fp16 cache (what the 4-bit cache is set against)
        n16 = int(min(64, max(2, -(-ROTATE_BYTES // cache16.numel()))))
        caches16 = [cache16] + [cache16.clone() for _ in range(n16 - 1)]
        calls16 = [lambda c=c: L.qoq_kv16_decode_attention(qd.data_ptr(), w.B, w.H, w.H_kv, w.D,
                                                           c.data_ptr(), C, lens_d.data_ptr(),
                                                           max_len, o.data_ptr(), wsp, wsb, st())
                   for c in caches16]
        for cl in calls16[:2]:
            rc = cl()
            if rc:
                raise RuntimeError(f"kv16 attention: {qoq.qoq_status_string(rc)}")
        t16 = per_launch_times(torch, blocker, [calls16], max(iters, len(calls16)))[0]
        del caches16, cache16
        b = wl.attention_bytes(lens, w.H, w.H_kv, w.D)
        b16 = int(lens.sum()) * w.H_kv * w.D * 4 + 2 * w.B * w.H * w.D * 2
        out.append(dict(workload=key, B=w.B, H=w.H, H_kv=w.H_kv, D=w.D,
                        tokens=int(lens.sum()), max_len=max_len,
                        splits=int(L.qoq_kv4_attention_workspace_bytes(w.B, w.H, w.H_kv, w.D, max_len)
                                   // (w.B * w.H * 132 * 4)) or 1,
                        us=round(t * 1e6, 2), bytes=b, gbs=round(b / t / 1e9, 1),
                        hbm_frac=round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                        fp16_kv_us=round(t16 * 1e6, 2), fp16_kv_bytes=b16,
                        fp16_kv_hbm_frac=round(b16 / t16 / 1e9 / HBM_PEAK_GBS, 4),
                        kv4_speedup=round(t16 / t, 2)))
        del caches, cache, o
        torch.cuda.empty_cache()
    return out


VARIANT_SHAPES = [("llama3_8b", "qkv", 256), ("llama3_8b", "gate_up", 256), ("prefill", "prefill", 4096),
                  ("qwen15_72b", "gate_up", 1024), ("qwen15_72b", "down", 1024)]


def variant_comparison(torch, qoq, blocker, dev, ws, iters):
    """The dequantization-overhead comparison: the W4A8 QoQ GEMM against the
    W8A8 per-channel GEMM (no dequantization, twice the weight bytes), the
    per-group W4A4 GEMM (INT4 weights and activations, every group's INT32
    partial sums converted and scaled in the main loop) and the weight-only
    W4A16 GEMM (UINT4 weights dequantized to fp16 for fp16 MFMA, fp16
    activations), GEMM kernels alone on pre-quantized inputs, each at its
    default launch plan and all four at one common 64 x 128 tile (4 waves, 2
    workgroups per CU) so that only the format differs."""
    out = []
    common = "2,1,2,2,4"
    for key, sname, M in VARIANT_SHAPES:
        w = wl.WORKLOADS[key]
        shp = next(x for x in w.shapes if x.name == sname)
        K, N = shp.K, shp.N
        W, X, _ = wl.make_case(w, shp, M)
        Wd = torch.from_numpy(W).to(dev)
        del W
        xd = to_half_device(torch, X, dev)
        pw = qoq.pack_weights(Wd)
        p8, s8 = qoq.w8a8_pack_weights(Wd)
        p4 = qoq.w4a4_pack_weights(Wd)
        p16 = qoq.w4a16_pack_weights(Wd)
        del Wd
        x8, s_x = qoq.quantize_act(xd)
        a4 = qoq.w4a4_quantize_act(xd)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        L = qoq.lib()
        cq = rotated_copies(pw)
        n8 = int(min(512, max(2, -(-ROTATE_BYTES // p8.numel()))))
        c8 = [p8] + [p8.clone() for _ in range(n8 - 1)]
        c4 = rotated_copies(qoq.PackedWeight(p4, pw.s1, N, K))
        n16 = int(min(512, max(2, -(-ROTATE_BYTES // p16.numel()))))
        c16 = [p16] + [p16.clone() for _ in range(n16 - 1)]
        st = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731

        def q_calls(cfg):
            calls = [GemmCall(qoq, torch, x8, s_x, cp, pw.s1, N, y, ws) for cp in cq]
            return calls

        def w8_calls():
            return [lambda cp=cp: L.qoq_w8a8_gemm(x8.data_ptr(), s_x.data_ptr(), M, K, cp.data_ptr(),
                                                  s8.data_ptr(), N, y.data_ptr(), None, st())
                    for cp in c8]

        def w4_calls():
            return [lambda cp=cp: L.qoq_w4a4_gemm(a4.data_ptr(), M, K, cp.data_ptr(), N, y.data_ptr(),
                                                  st()) for cp in c4]

        def w16_calls():
            return [lambda cp=cp: L.qoq_w4a16_gemm(xd.data_ptr(), M, K, cp.data_ptr(), N,
                                                   y.data_ptr(), st()) for cp in c16]

        rec = dict(workload=key, shape=sname, M=M, K=K, N=N)
        ops = wl.algorithmic_ops(M, K, N)
        for label, tune_key, tune_val, make in (
                ("w4a8_qoq", None, None, lambda: q_calls(None)),
                ("w8a8", None, None, w8_calls),
                ("w4a4", None, None, w4_calls),
                ("w4a16", None, None, w16_calls),
                ("w4a8_qoq_common_tile", "gemm", "tile32," + common, lambda: q_calls(None)),
                ("w8a8_common_tile", "variant", common, w8_calls),
                ("w4a4_common_tile", "variant", common, w4_calls),
                ("w4a16_common_tile", "variant", common, w16_calls)):
            qoq.clear_tuning()
            if tune_key:
                qoq.set_tuning(tune_key, tune_val)
            try:
                calls = make()
                for cl in calls[:2]:
                    rc = cl()
                    if rc:
                        raise RuntimeError(f"{label}: {qoq.qoq_status_string(rc)}")
                t = per_launch_times(torch, blocker, [calls], max(iters, len(calls)))[0]
                rec[label + "_us"] = round(t * 1e6, 2)
                rec[label + "_tops"] = round(ops / t / 1e12, 1)
            finally:
                qoq.clear_tuning()
        out.append(rec)
        del cq, c8, c4, c16, pw, p8, p4, p16
        torch.cuda.empty_cache()
    return out


def cpu_baseline(dw, shape, budget_s):
    """The oracle as it stands, on the host, over the decode step's inputs,
    timed stage by stage:
      (i)   weight quantization (both levels; offline in serving, timed once),
      (ii)  per-token activation quantization of the four batches,
      (iii) the exact GEMM as an fp64 BLAS matmul of the integer values
            (exact: every partial sum is an integer below 2^53), on the BLAS
            library's threads,
      (iv)  the fp64 epilogue.
    Stages (ii)-(iv) repeat until about `budget_s` seconds have passed; the
    reported rate is the step's algorithmic operations over their time. The
    literal int64 matmul (the oracle's defining form, single-threaded in
    NumPy) is timed once beside it on the same operands and must agree
    exactly, as on the tiny workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), int(i.get("num_threads", 0)))
                for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:   # threadpoolctl missing: thread count unknown
        blas = []
    cores = len(os.sched_getaffinity(0))
    K, N = shape.K, shape.N
    W, _, _ = wl.make_case(dw, shape, 1)
    t0 = time.perf_counter()
    wq = oracle.quantize_weights(W, wl.GROUP)
    w8 = oracle.dequantize_level2(wq["q4"], wq["s2"], wq["z"], wl.GROUP)
    t_weights = time.perf_counter() - t0
    cases = [wl.make_case(dw, shape, M)[1] for M in dw.Ms]
    ops_pass = sum(wl.algorithmic_ops(M, K, N) for M in dw.Ms)
    t_act = t_gemm = t_epi = 0.0
    passes = 0
    while True:
        for X in cases:
            a = time.perf_counter()
            x8, s_x = oracle.quantize_act(X)
            b = time.perf_counter()
            acc = oracle.int_gemm_fp64(x8, w8)
            c = time.perf_counter()
            oracle.epilogue(acc, s_x, wq["s1"])
            d = time.perf_counter()
            t_act += b - a
            t_gemm += c - b
            t_epi += d - c
        passes += 1
        if t_act + t_gemm + t_epi >= budget_s or passes >= 200:
            break
    run_s = t_act + t_gemm + t_epi
    # the literal int64 form on the same operands (decode step and tiny workload)
    t_int64 = 0.0
    for X in cases:
        x8, _ = oracle.quantize_act(X)
        t0 = time.perf_counter()
        literal = oracle.int_gemm(x8, w8)
        t_int64 += time.perf_counter() - t0
        if not np.array_equal(literal, oracle.int_gemm_fp64(x8, w8)):
            raise AssertionError("fp64 BLAS GEMM differs from the int64 GEMM")
    tw = wl.WORKLOADS["tiny"]
    Wt, Xt, _ = wl.make_case(tw, tw.shapes[0], tw.Ms[0])
    wqt = oracle.quantize_weights(Wt, wl.GROUP)
    w8t = oracle.dequantize_level2(wqt["q4"], wqt["s2"], wqt["z"], wl.GROUP)
    x8t, _ = oracle.quantize_act(Xt)
    if not np.array_equal(oracle.int_gemm(x8t, w8t), oracle.int_gemm_fp64(x8t, w8t)):
        raise AssertionError("fp64 BLAS GEMM differs from the int64 GEMM (tiny)")
    threads = max([t for _, t in blas] or [1])
    return {"value": round(ops_pass * passes / run_s / 1e12, 6), "unit": "TOPS",
            "cores": threads, "kind": "oracle",
            "sample": f"{passes} pass(es) of the decode step's run-time stages (M=1,8,32,64; "
                      f"K=N=4096): per-token quantization, exact GEMM as an fp64 BLAS matmul "
                      f"({blas[0][0] if blas else 'BLAS'}, {threads} threads), fp64 epilogue; "
                      f"{run_s:.1f} s on the host",
            "host_cores": cores,
            "blas_threads": threads,
            "stages_s_per_step": {"act_quant": round(t_act / passes, 6),
                                  "gemm_fp64_blas": round(t_gemm / passes, 6),
                                  "epilogue": round(t_epi / passes, 6)},
            "weight_quant_s": round(t_weights, 3),
            "int64_gemm_s_per_step": round(t_int64, 4),
            "int64_matches_fp64": True}


def platform_info():
    """ROCm / HIP / driver versions and the GPU's current shader clock as the
    driver reports it (read right after the timed region)."""
    info = {}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    try:
        import torch
        info["hip_runtime"] = torch.version.hip
        info["torch"] = torch.__version__
    except Exception:
        pass
    for path in ("/sys/module/amdgpu/version", "/proc/driver/amdgpu/version"):
        try:
            info["driver"] = open(path).read().strip()
            break
        except OSError:
            info["driver"] = None
    return info


def gpu_sclk_mhz():
    """Current shader clock (MHz) from the driver's DPM table, if readable."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if line.strip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    if m:
                        return int(m.group(1))
        except OSError:
            continue
    return None


if __name__ == "__main__":
    main()
