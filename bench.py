#!/usr/bin/env python3
"""Benchmark of the sign-binarised linear layer on one MI355X.

Headline (one JSON line on stdout): the decode GEMV of a Llama-2-7B MLP
projection, X[1,4096] bf16 (six x60 outlier channels) · W_sign[11008,4096]^T
with fp16 scales, fp32 output.

* A step is one pass over R layers, each with its own copy of the packed
  weights and scales (R copies total >= --rotate-gib GiB, so neither L2 nor the
  256 MB Infinity Cache holds them); the R launches are captured once in a HIP
  graph and a step is one replay.  Inputs are resident in HBM before timing.
* value = weight bytes (N·K/8) x R / step time, in GB/s.
* roofline.achieved = algorithmic bytes of one launch (packed signs + X + a + b
  + Y) / average launch time over the timed region (HIP events on the stream
  the graph replays on).
* cpu_baseline = the fp64 oracle on the same workload, timed on the host.
* secondary = the other workloads (prefill GEMM TOPS, batched decode, DBF, the
  NEXT rows), timed the same way.
* Before timing, every line's outputs are checked against a plain fp32 PyTorch
  computation on the GPU: a guard against timing a broken configuration.  The
  parity claims against the fp64 oracle belong to tests/ (each timed
  configuration has a full-size parity test there); here the oracle only runs
  in the cpu_baseline leg.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-secondary] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # dense bf16 MFMA, 256 CU x 4096 flop/clk x 2.4 GHz
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(name: str) -> str:
    p = os.path.join(ROOT, "bit_weight_linear_amd", "csrc", name)
    h = hashlib.sha256()
    for f in (p, os.path.join(ROOT, "bit_weight_linear_amd", "csrc", "obl_common.hpp")):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_src: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; otherwise None."""
    p = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(workload)
    except Exception:
        return None
    if not rec or rec.get("source_sha") != source_sha(kernel_src):
        return None
    return rec.get("hbm_bytes_per_launch")


def load_binding():
    try:
        from bit_weight_linear_amd import binding
    except ImportError:
        from bit_weight_linear_amd import build as b
        log("libobl.so missing: building it")
        b.build()
        from bit_weight_linear_amd import binding
    return binding


class Timed:
    """Captures `launches` (callables) in one HIP graph and times replays."""

    def __init__(self, torch, launches):
        self.torch = torch
        self.stream = torch.cuda.Stream()
        self.stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.stream):
            for f in launches:        # eager warm-up on the capture stream (sizes its library scratch)
                f()
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=self.stream):
            for f in launches:
                f()
        torch.cuda.synchronize()
        self.n = len(launches)

    def run(self, warmup: int, steps: int):
        torch = self.torch
        for _ in range(warmup):
            self.graph.replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            self.graph.replay()
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop)
        return ms / steps, ms / (steps * self.n)   # ms per step, ms per launch


# ------------------------------------------------------------------ guards
# Plain fp32 PyTorch on the GPU (allow_tf32 off); errors on the normalised scale
# |a_j| Σ_k |x_ik b_k| (or its DBF product) as in the tests.
def t_err(torch, Y, Yref, S):
    d = (Y.double() - Yref.double()).abs()
    S = S.double().expand_as(d)
    r = torch.where(S > 0, d / S, torch.where(d > 0, torch.full_like(d, float("inf")), torch.zeros_like(d)))
    return float(r.max())


def t_linear(torch, X, Spm1, a, b):
    """Y = ((X ⊙ b) S^T) ⊙ a in fp32 and its normalised scale."""
    Xb = X.float() * b.float()[None, :]
    Y = (Xb @ Spm1.float().t()) * a.float()[None, :]
    S = Xb.abs().sum(1, keepdim=True) * a.float().abs()[None, :]
    return Y, S


def t_dbf(torch, X, S2, S1, b, m, a):
    T1 = ((X.float() * b.float()[None, :]) @ S2.float().t()) * m.float()[None, :]
    Y = (T1 @ S1.float().t()) * a.float()[None, :]
    S = ((X.float() * b.float()[None, :]).abs().sum(1, keepdim=True) * m.float().abs().sum()
         * a.float().abs()[None, :])
    return Y, S


def onebit_setup(torch, B, WL, i, rotate_bytes):
    c = WL.workload(i)
    dev = torch.device("cuda")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    X = torch.from_numpy(c.X).to(torch.float32).to(tdt[c.x_dtype]).to(dev)
    a0 = torch.from_numpy(c.a).to(torch.float32).to(tdt[c.scale_dtype]).to(dev)
    b0 = torch.from_numpy(c.b).to(torch.float32).to(tdt[c.scale_dtype]).to(dev)
    Spm1 = torch.from_numpy(c.W_sign).to(dev)
    W0 = B.pack_signs(Spm1)
    per_copy = W0.numel() * 4 + a0.numel() * a0.element_size() + b0.numel() * b0.element_size()
    R = max(1, -(-rotate_bytes // per_copy))
    copies = [(W0, a0, b0)] + [(W0.clone(), a0.clone(), b0.clone()) for _ in range(R - 1)]
    Y = torch.empty((c.M, c.N), dtype=tdt[c.y_dtype], device=dev)
    # guard on the timed configuration, first copy
    B.linear(X, W0, a0, b0, out=Y)
    Yref, S = t_linear(torch, X, Spm1, a0, b0)
    err = t_err(torch, Y, Yref, S)
    del Spm1, Yref, S
    launches = [(lambda W=W, a=a, b=b: B.linear(X, W, a, b, out=Y)) for (W, a, b) in copies]
    return c, launches, err, R


def dbf_setup(torch, B, WL, rotate_bytes):
    c = WL.workload(5)
    dev = torch.device("cuda")
    X = torch.from_numpy(c.X).to(torch.float32).to(torch.bfloat16).to(dev)
    sc = [torch.from_numpy(v).to(torch.float32).to(torch.float16).to(dev) for v in (c.b, c.m, c.a)]
    S2d, S1d = torch.from_numpy(c.S2).to(dev), torch.from_numpy(c.S1).to(dev)
    S2 = B.pack_signs(S2d)
    S1 = B.pack_signs(S1d)
    per_copy = (S2.numel() + S1.numel()) * 4 + sum(t.numel() * 2 for t in sc)
    R = max(1, -(-rotate_bytes // per_copy))
    copies = [(S2, S1, *sc)] + [(S2.clone(), S1.clone(), *[t.clone() for t in sc]) for _ in range(R - 1)]
    Y = torch.empty((c.M, c.N), dtype=torch.float32, device=dev)
    ws = torch.empty((c.M, c.Kmid), dtype=torch.float32, device=dev)
    B.dbf_linear(X, S2, S1, *sc, workspace=ws, out=Y)
    err = t_err(torch, Y, *t_dbf(torch, X, S2d, S1d, *sc))
    launches = [(lambda s2=s2, s1=s1, b=b, m=m, a=a: B.dbf_linear(X, s2, s1, b, m, a, workspace=ws, out=Y))
                for (s2, s1, b, m, a) in copies]
    return c, launches, err, R


def dbf_prefill_setup(torch, B, WL, M=512, K=4096, Kmid=3072, N=4096, copies=8):
    """DBF prefill (two MFMA GEMMs with the m mid-scale)."""
    c = WL.dbf_case(M, K, Kmid, N, seed=Kmid, name=f"dbf-prefill-{M}x{K}-{Kmid}-{N}")
    dev = torch.device("cuda")
    X = torch.from_numpy(c.X).to(torch.float32).to(torch.bfloat16).to(dev)
    sc = [torch.from_numpy(v).to(torch.float32).to(torch.float16).to(dev) for v in (c.b, c.m, c.a)]
    S2d, S1d = torch.from_numpy(c.S2).to(dev), torch.from_numpy(c.S1).to(dev)
    S2 = B.pack_signs(S2d)
    S1 = B.pack_signs(S1d)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((M, Kmid), dtype=torch.float32, device=dev)
    B.dbf_linear(X, S2, S1, *sc, workspace=ws, out=Y)
    err = t_err(torch, Y, *t_dbf(torch, X, S2d, S1d, *sc))
    reps = [(S2, S1)] + [(S2.clone(), S1.clone()) for _ in range(copies - 1)]
    launches = [(lambda s2=s2, s1=s1: B.dbf_linear(X, s2, s1, *sc, workspace=ws, out=Y)) for (s2, s1) in reps]
    return c, launches, err, copies


def backward_setup(torch, B, WL, M, K, N, copies):
    """Backward of the layer (dX, da, db) on synthetic dY; guard: max error of
    each output relative to that output's largest magnitude."""
    import numpy as np
    rng = np.random.default_rng(M + K + N)
    X = WL.round_to(rng.standard_normal((M, K)), "bf16")
    dY = WL.round_to(rng.standard_normal((M, N)), "bf16")
    S = WL.random_signs(rng, (N, K))
    a = WL.round_to(np.abs(rng.standard_normal(N)) * 0.02 + 1e-3, "f16")
    b = WL.round_to(np.abs(rng.standard_normal(K)) * 0.02 + 1e-3, "f16")
    dev = torch.device("cuda")
    t = lambda v, dt: torch.from_numpy(v).to(torch.float32).to(dt).to(dev)
    Xd, dYd, ad, bd = t(X, torch.bfloat16), t(dY, torch.bfloat16), t(a, torch.float16), t(b, torch.float16)
    Sd = torch.from_numpy(S).to(dev)
    W = B.pack_signs(Sd)
    Wt = B.transpose_signs(W, N, K)
    ws = torch.empty(M * (N + K), dtype=torch.float32, device=dev)
    dX, da, db, _ = B.linear_backward(dYd, Xd, W, Wt, ad, bd, workspace=ws)
    Sf = Sd.float()
    T = (Xd.float() * bd.float()) @ Sf.t()
    U = (dYd.float() * ad.float()) @ Sf
    refs = (U * bd.float(), (dYd.float() * T).sum(0), (Xd.float() * U).sum(0))
    err = max(float((g.double() - r.double()).abs().max() / r.double().abs().max())
              for g, r in zip((dX, da, db), refs))
    reps = [(W, Wt)] + [(W.clone(), Wt.clone()) for _ in range(copies - 1)]
    launches = [(lambda w=w, wt=wt: B.linear_backward(dYd, Xd, w, wt, ad, bd, workspace=ws)) for (w, wt) in reps]
    return launches, err


def cpu_baseline(WL, budget_s: float = 12.0):
    """Time the fp64 oracle on workload 2 (the headline) for a bounded sample.
    The only place bench.py uses the oracle."""
    import numpy as np
    import oracle as O
    c = WL.workload(2)
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    times = []
    t_end = time.perf_counter() + budget_s
    while len(times) < 3 or (time.perf_counter() < t_end and len(times) < 50):
        t0 = time.perf_counter()
        O.onebit_linear(c.X, c.W_sign, c.a, c.b)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    wbytes = c.N * c.K / 8
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": round(wbytes / t / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} full calls of workload 1x4096x11008 (fp64 dense W = W_sign*(a b^T) "
                      f"then X W^T), median {t * 1e3:.1f} ms per call; weight bytes N*K/8 per call; "
                      f"dense-W formation is single-threaded NumPy, the product uses {threads} BLAS threads; "
                      f"host os.cpu_count() = {os.cpu_count()}, affinity {affinity}, "
                      f"OPENBLAS_NUM_THREADS = {os.environ.get('OPENBLAS_NUM_THREADS')}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the benchmark, run one plain device-to-device copy of this many MiB "
                         "(a reference kernel of known traffic for hardware-counter runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer has no multi-GPU path here (one GPU holds a "
              "whole layer's packed weights); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_weight_linear_amd import workloads as WL

    B = load_binding()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rot = int(args.rotate_gib * (1 << 30))

    # ---------------- headline: workload 2, M = 1 decode GEMV
    torch.backends.cuda.matmul.allow_tf32 = False    # the guards compare against plain fp32 products
    c, launches, err, R = onebit_setup(torch, B, WL, 2, rot)
    log(f"[bench] {c.name}: guard vs fp32 torch, max normalised error {err:.3e}; {R} weight copies")
    assert err <= 1e-4, "the timed configuration disagrees with the fp32 guard"
    t = Timed(torch, launches)
    ms_step, ms_launch = t.run(args.warmup, args.steps)
    wbytes = c.N * c.K // 8
    alg_bytes = wbytes + c.M * c.K * 2 + c.N * 2 + c.K * 2 + c.M * c.N * 4
    value = wbytes * R / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes / (ms_launch * 1e-3) / 1e9
    traffic = measured_traffic("gemv_lut.hip", "decode-gemv-1x4096x11008")
    out = {
        "metric": "1-bit linear: weight GB/s (% HBM peak) at M=1; TOPS (% MFMA peak) at M=2048",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": c.name, "M": c.M, "K": c.K, "N": c.N, "x_dtype": c.x_dtype,
                   "scale_dtype": c.scale_dtype, "y_dtype": c.y_dtype, "layers_per_step": R,
                   "weight_bytes_per_layer": wbytes, "parallelism": "single-gpu",
                   "step": f"{R} launches over distinct weight copies, one HIP graph replay"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "us_per_launch": round(ms_launch * 1e3, 4),
        "hbm_frac_weight_bytes": round(value / HBM_PEAK_GBS, 4),
        "check_vs_torch_fp32": float(f"{err:.3e}"),
        "parity": "against the fp64 oracle in tests/test_gpu_parity.py (test_workload2_decode_gemv, full size)",
    }
    del launches, t
    torch.cuda.empty_cache()
    # Context for the headline: the runtime's own device-to-device copy of the same weight bytes,
    # launched the same way (R distinct sources, one graph replay).  A copy streams the bytes once
    # and writes as many, with no arithmetic: its per-launch time is a practical floor for a
    # kernel that must read these weights from HBM once per launch.
    srcs = [torch.ones(wbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    dst = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
    tc = Timed(torch, [(lambda s_=s_: dst.copy_(s_)) for s_ in srcs])
    _, ms_copy = tc.run(args.warmup, args.steps)
    out["launch_floor_context"] = {
        "what": f"device-to-device copy of {wbytes} bytes per launch (torch copy_), {R} distinct sources "
                f"in one graph replay, same arrangement as the timed GEMV launches",
        "us_per_launch": round(ms_copy * 1e3, 4),
        "read_GBps": round(wbytes / (ms_copy * 1e-3) / 1e9, 1),
        "gemv_over_copy": round(ms_launch / ms_copy, 3)}
    log(f"[bench] context: copy of the weight bytes {ms_copy * 1e3:.2f} us per launch "
        f"(GEMV {ms_launch * 1e3:.2f} us)")
    del srcs, dst, tc
    torch.cuda.empty_cache()
    # The fixed cost of a launch in the same arrangement: a kernel that spins for zero cycles
    # (torch's own test helper), R of them in one graph replay.  No kernel launched this way
    # takes less; what the GEMV and the copy add on top of it is their memory and arithmetic.
    try:
        te = Timed(torch, [(lambda: torch.cuda._sleep(0)) for _ in range(R)])
        _, ms_empty = te.run(args.warmup, args.steps)
        out["launch_floor_context"]["empty_kernel_us_per_launch"] = round(ms_empty * 1e3, 4)
        out["launch_floor_context"]["gemv_above_empty_us"] = round((ms_launch - ms_empty) * 1e3, 4)
        log(f"[bench] context: empty kernel {ms_empty * 1e3:.2f} us per launch")
        del te
    except (AttributeError, RuntimeError) as e:   # helper missing on this build
        log(f"[bench] context: no empty-kernel timing ({e})")

    # ---------------- secondary workloads
    if not args.no_secondary:
        sec = {}
        # workload 4: prefill GEMM, M = 2048
        c4, l4, e4, R4 = onebit_setup(torch, B, WL, 4, min(rot, 64 << 20))
        assert e4 <= 1e-2, "workload 4 disagrees with the fp32 guard"
        t4 = Timed(torch, l4)
        ms4_step, ms4 = t4.run(2, max(3, args.steps // 4))
        flops = 2.0 * c4.M * c4.N * c4.K
        tflops = flops / (ms4 * 1e-3) / 1e12
        sec[c4.name] = {"us_per_launch": round(ms4 * 1e3, 2), "TOPS": round(tflops, 2),
                        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4), "bound": "mfma",
                        "check_vs_torch_fp32": float(f"{e4:.3e}"), "copies": R4}
        log(f"[bench] {c4.name}: {ms4 * 1e3:.1f} us, {tflops:.1f} TFLOP/s")
        del l4, t4
        torch.cuda.empty_cache()
        # workloads 1, 3: decode kernel
        for i in (3, 1):
            ci, li, ei, Ri = onebit_setup(torch, B, WL, i, rot if i == 3 else (64 << 20))
            assert ei <= 1e-4, f"workload {i} disagrees with the fp32 guard"
            ti = Timed(torch, li)
            _, msi = ti.run(args.warmup, args.steps)
            wb = ci.N * ci.K / 8
            ab = (wb + ci.M * ci.K * (4 if ci.x_dtype == "f32" else 2)
                  + (ci.N + ci.K) * (4 if ci.scale_dtype == "f32" else 2) + ci.M * ci.N * 4)
            sec[ci.name] = {"us_per_launch": round(msi * 1e3, 3),
                            "weight_GBps": round(wb / (msi * 1e-3) / 1e9, 1),
                            "algorithmic_bytes": int(ab), "ideal_us_hbm": round(ab / HBM_PEAK_GBS / 1e3, 4),
                            "hbm_frac": round(ab / (msi * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "bound": "latency (launch and one HBM round trip; the HBM time is a fraction of it)",
                            "check_vs_torch_fp32": float(f"{ei:.3e}"), "copies": Ri}
            log(f"[bench] {ci.name}: {msi * 1e3:.2f} us")
            del li, ti
        # workload 5: DBF
        c5, l5, e5, R5 = dbf_setup(torch, B, WL, rot)
        assert e5 <= 1e-4, "workload 5 disagrees with the fp32 guard"
        t5 = Timed(torch, l5)
        _, ms5 = t5.run(args.warmup, args.steps)
        wb5 = c5.Kmid * (c5.K + c5.N) / 8
        ab5 = wb5 + c5.M * c5.K * 2 + (c5.K + c5.Kmid + c5.N) * 2 + 2 * c5.M * c5.Kmid * 4 + c5.M * c5.N * 4
        sec[c5.name] = {"us_per_call": round(ms5 * 1e3, 3), "weight_GBps": round(wb5 / (ms5 * 1e-3) / 1e9, 1),
                        "algorithmic_bytes": int(ab5), "ideal_us_hbm": round(ab5 / HBM_PEAK_GBS / 1e3, 4),
                        "hbm_frac": round(ab5 / (ms5 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "bound": "latency (two stages, one launch each: stage 2 reads the exact bf16 terms of T1)",
                        "check_vs_torch_fp32": float(f"{e5:.3e}"), "copies": R5,
                        "stages_per_call": 2}
        log(f"[bench] {c5.name}: {ms5 * 1e3:.2f} us per call")
        del l5, t5
        # DBF prefill (M = 512, Kmid = 3072: 1.5 sign bits per weight)
        c6, l6, e6, R6 = dbf_prefill_setup(torch, B, WL)
        assert e6 <= 1.5e-2, "the DBF prefill disagrees with the fp32 guard"
        t6 = Timed(torch, l6)
        _, ms6 = t6.run(2, max(3, args.steps // 4))
        fl6 = 2.0 * c6.X.shape[0] * c6.S2.shape[0] * (c6.S2.shape[1] + c6.S1.shape[0])
        tf6 = fl6 / (ms6 * 1e-3) / 1e12
        sec[c6.name] = {"us_per_call": round(ms6 * 1e3, 2), "TOPS": round(tf6, 2),
                        "mfma_frac": round(tf6 / BF16_PEAK_TFLOPS, 4),
                        "check_vs_torch_fp32": float(f"{e6:.3e}"), "copies": R6}
        log(f"[bench] {c6.name}: {ms6 * 1e3:.1f} us per call, {tf6:.1f} TFLOP/s")
        del l6, t6
        # backward of the layer at the batched-decode shape (two sign contractions + the grads kernel)
        l7, e7 = backward_setup(torch, B, WL, 16, 4096, 4096, copies=64)
        assert e7 <= 1e-4, "the backward disagrees with the fp32 guard"
        t7 = Timed(torch, l7)
        _, ms7 = t7.run(args.warmup, args.steps)
        sec["backward-16x4096x4096"] = {"us_per_call": round(ms7 * 1e3, 3),
                                        "weight_GBps": round(2 * 4096 * 4096 / 8 / (ms7 * 1e-3) / 1e9, 1),
                                        "check_vs_torch_fp32": float(f"{e7:.3e}"), "copies": 64,
                                        "note": "weight bytes counted twice: W and its transposed packing"}
        log(f"[bench] backward-16x4096x4096: {ms7 * 1e3:.2f} us per call")
        del l7, t7
        # SVID conversion of the headline layer's dense fp16 weight (32 power iterations)
        rng8 = np.random.default_rng(8)
        Wd = torch.from_numpy(WL.round_to(rng8.standard_normal((11008, 4096)) * 0.02, "f16")).to(torch.float16).cuda()
        P8, a8, b8 = B.svid(Wd, iters=32)
        assert bool(torch.isfinite(a8.float()).all() and (a8.float() > 0).all() and (b8.float() > 0).all()), \
            "SVID scales not finite and positive"
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(3):
            B.svid(Wd, iters=32)
        ev1.record()
        torch.cuda.synchronize()
        ms8 = ev0.elapsed_time(ev1) / 3
        passes = 32 + 2                          # |W| reads: one per (fused) iteration, the final row pass, Sign(W)
        sec["svid-11008x4096-f16-32iters"] = {"ms_per_conversion": round(ms8, 3),
                                              "weight_read_GBps": round(passes * Wd.numel() * 2 / (ms8 * 1e-3) / 1e9, 1)}
        log(f"[bench] svid-11008x4096-f16-32iters: {ms8:.3f} ms per conversion")
        del Wd, P8, a8, b8
        # LayerNorm after the layer: the row kernel alone at the prefill output shape
        # (fp32 Y -> bf16 Z, fp16 gamma/beta), over 4 copies of Y so no replay hits in cache
        M9, N9 = 2048, 14336
        rng9 = np.random.default_rng(9)
        Y9 = [torch.from_numpy(rng9.standard_normal((M9, N9)) * 2 + 1).to(torch.float32).cuda() for _ in range(4)]
        g9 = torch.from_numpy(WL.round_to(rng9.standard_normal(N9) * 0.5 + 1, "f16")).to(torch.float16).cuda()
        be9 = torch.from_numpy(WL.round_to(rng9.standard_normal(N9) * 0.1, "f16")).to(torch.float16).cuda()
        Z9 = torch.empty((M9, N9), dtype=torch.bfloat16, device="cuda")
        B.layernorm(Y9[0], 1e-5, g9, be9, out=Z9)
        z9ref = torch.nn.functional.layer_norm(Y9[0], (N9,), g9.float(), be9.float(), 1e-5)
        e9 = float(((Z9.float() - z9ref).abs() / (z9ref.abs() + 1.0)).max())
        del z9ref
        assert e9 <= 2.0 ** -7, "the LayerNorm disagrees with the fp32 guard"
        t9 = Timed(torch, [(lambda y=y: B.layernorm(y, 1e-5, g9, be9, out=Z9)) for y in Y9])
        _, ms9 = t9.run(args.warmup, args.steps)
        by9 = M9 * N9 * (4 + 2) + 2 * N9 * 2
        sec["layernorm-2048x14336-f32-bf16"] = {
            "us_per_launch": round(ms9 * 1e3, 3), "GBps": round(by9 / (ms9 * 1e-3) / 1e9, 1),
            "hbm_frac": round(by9 / (ms9 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bound": "hbm",
            "algorithmic_bytes": by9, "check_vs_torch_fp32": float(f"{e9:.3e}")}
        log(f"[bench] layernorm-2048x14336: {ms9 * 1e3:.2f} us, {by9 / (ms9 * 1e-3) / 1e9:.0f} GB/s")
        del t9, Y9, Z9
        # the decode layer followed by LayerNorm in one call (headline shape)
        c10 = WL.workload(2)
        X10 = torch.from_numpy(c10.X).to(torch.float32).to(torch.bfloat16).cuda()
        S10 = torch.from_numpy(c10.W_sign).cuda()
        W10 = B.pack_signs(S10)
        a10 = torch.from_numpy(c10.a).to(torch.float32).to(torch.float16).cuda()
        b10 = torch.from_numpy(c10.b).to(torch.float32).to(torch.float16).cuda()
        reps10 = [(W10, a10, b10)] + [(W10.clone(), a10.clone(), b10.clone()) for _ in range(R - 1)]
        ws10 = torch.empty((1, c10.N), dtype=torch.float32, device="cuda")
        Z10 = torch.empty((1, c10.N), dtype=torch.float32, device="cuda")
        B.linear_layernorm(X10, W10, a10, b10, 1e-5, workspace=ws10, out=Z10)
        y10, _ = t_linear(torch, X10, S10, a10, b10)
        e10 = float((Z10 - torch.nn.functional.layer_norm(y10, (c10.N,), None, None, 1e-5)).abs().max())
        del S10, y10
        assert e10 <= 1e-3, "the layer + LayerNorm disagrees with the fp32 guard"
        t10 = Timed(torch, [(lambda w=w, a=a, b=b: B.linear_layernorm(X10, w, a, b, 1e-5, workspace=ws10, out=Z10))
                            for (w, a, b) in reps10])
        _, ms10 = t10.run(args.warmup, args.steps)
        sec[f"linear-layernorm-{c10.name}"] = {"us_per_call": round(ms10 * 1e3, 3),
                                               "weight_GBps": round(wbytes / (ms10 * 1e-3) / 1e9, 1),
                                               "check_vs_torch_fp32_abs": float(f"{e10:.3e}"), "copies": R,
                                               "launches_per_call": 2}
        log(f"[bench] linear-layernorm-{c10.name}: {ms10 * 1e3:.2f} us per call")
        del t10, reps10
        out["secondary"] = sec

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = nbytes
        del src, dst

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(WL)
        log(f"[bench] cpu baseline {out['cpu_baseline']['value']} GB/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
