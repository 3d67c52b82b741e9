#!/usr/bin/env python3
"""Benchmark: fused masked multi-head attention forward on one MI355X.

One step = one call of the library's hot path (one kernel launch) over one
batch of seeded synthetic input already resident in HBM. W warm-up steps,
then exactly K steps are timed between synchronisations with HIP events on
the stream the kernel is launched on. The K timed steps are captured once as
a HIP graph and replayed, so the figure is the GPU's throughput, not the
host's launch rate; the eager (launch-per-call) time is reported beside it.

Prints one JSON line: metric, value (effective TFLOP/s, masked-out work not
counted), us_per_call, the roofline of the kernel and the fp64 CPU oracle's
rate on the host cores (cpu_baseline). For HBM-bound workloads a cold-cache
figure is added (cold_cache): the median per-call time with the caches flushed
before each call. ``--config N`` picks workload N. The default is workload 4,
the largest single-GPU configuration: pre-LayerNorm cross-attention, bfloat16,
B=32 H=16 Lq=Lk=2048 D=64 (model width 1024), residual added, no mask.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "masked-MHA fwd effective TFLOP/s + µs/call; % of MFMA/HBM roofline (1 GPU)"
PEAK_TFLOPS = {"f32": 157.3, "f16": 2500.0, "bf16": 2500.0}  # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0
ESIZE = {"f32": 4, "f16": 2, "bf16": 2}
KERNEL_NAME = "mha_fwd_kernel"
SOFTMAX_CONFIG_ID = 6
SOFTMAX_KERNEL_NAME = "mha_softmax_rows"
DECODE_CONFIG_ID = 7
DECODE_KERNEL_NAME = "mha_decode"
BWD_CONFIG_ID = 8
BWD_KERNEL_NAME = "mha_bwd"
BWD_METRIC = "masked-MHA bwd effective TFLOP/s + µs/call; % of MFMA roofline (1 GPU)"
SOFTMAX_METRIC = "row softmax of a materialised score tensor: GB/s; % of HBM roofline (1 GPU)"


# ---------------------------------------------------------------------------
# work accounting (plain counting from the mask definitions)
# ---------------------------------------------------------------------------
def legal_matrix(w: W.Workload, b: int) -> np.ndarray:
    """bool [Lq, Lk]: legal (query, key) pairs of batch entry b (shared by heads)."""
    i = np.arange(w.Lq)[:, None]
    j = np.arange(w.Lk)[None, :]
    ok = np.ones((w.Lq, w.Lk), bool)
    if w.kind & W.CAUSAL:
        ok &= j <= i
    if w.kind & W.PADDING:
        ok &= j < w.lens[b]
    if w.kind & W.ADDITIVE:
        ok &= ~np.isneginf(W.to_f64(w.add[b, 0], w.dtype))
    return ok


def work(w: W.Workload):
    """(effective FLOPs, algorithmic bytes, legal pairs per (b, query row))."""
    E = ESIZE[w.dtype]
    pairs_row = np.stack([legal_matrix(w, b).sum(axis=1) for b in range(w.B)])  # [B, Lq]
    flops = 4.0 * w.D * float(pairs_row.sum()) * w.H
    keys_used = sum(int(legal_matrix(w, b).any(axis=0).sum()) for b in range(w.B))
    kv = 2.0 * keys_used * w.H * w.D * E
    if w.prenorm:
        F = w.H * w.D
        io = 2.0 * w.B * w.Lq * F * E + 2.0 * F * E  # x (also the residual) in, out; gamma, beta
    else:
        io = 2.0 * w.B * w.H * w.Lq * w.D * E  # Q in, O out
    mask = 0.0
    if w.kind & W.PADDING:
        mask = 4.0 * w.B
    elif w.kind & W.ADDITIVE:
        mask = float(w.B * w.Lq * w.Lk * E)
    return flops, io + kv + mask, pairs_row


def _code_only(src: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed, so a
    comment edit does not change the hash. String and character literals are
    kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


# The sources each profiled kernel family is built from: a summary stays valid
# while these are unchanged in code (comments and layout ignored).
KERNEL_SOURCES = {
    KERNEL_NAME: ("mha_common.hpp", "mha_kernel_f32.hpp", "mha_kernel_half.hpp", "mha_launch.hpp",
                  "mha_inst_bf16.hip", "mha_inst_f16.hip", "mha_inst_f32.hip"),
    SOFTMAX_KERNEL_NAME: ("mha_common.hpp", "mha_softmax.hpp", "mha_softmax.hip"),
    DECODE_KERNEL_NAME: ("mha_common.hpp", "mha_decode.hpp", "mha_decode.hip"),
    BWD_KERNEL_NAME: ("mha_common.hpp", "mha_bwd.hpp", "mha_bwd_f32.hpp", "mha_bwd.hip"),
}


def kernel_source_hash(kernel: str = KERNEL_NAME) -> str:
    """Hash of the code (comments and layout ignored) of one kernel family's sources."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "masked_head_attention_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kernel]):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def stored_counter(workload: str, key: str = "hbm_bytes_per_launch", kernel: str = KERNEL_NAME):
    """A per-launch figure (HBM bytes, executed MFMA FLOPs) from a committed
    rocprofv3 --pmc summary, if it was taken on the current kernel sources;
    else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        txt = f.read()
    m = re.search(r"^kernel_sources_sha256_16:\s*(\S+)", txt, re.M)
    t = re.search(r"^" + re.escape(key) + r":\s*([0-9.eE+]+)", txt, re.M)
    if not m or not t or m.group(1) != kernel_source_hash(kernel):
        return None
    return float(t.group(1))


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------
def gpu_setup(w: W.Workload, workspace: bool = True):
    """Device copies of w's inputs and an output buffer; for a bfloat16 pre-LN
    workload (with ``workspace``) also the workspace of mha_prenorm_cross_fwd_ws."""
    import torch

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.int32:
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    d = {n: dev(getattr(w, n)) for n in ("q", "k", "v", "x", "gamma", "beta")}
    d["mask"] = dev(w.lens) if w.kind & W.PADDING else (dev(w.add) if w.kind & W.ADDITIVE else None)
    d["out"] = torch.empty_like(d["x"] if w.prenorm else d["q"])
    d["ws"] = None
    if workspace and w.prenorm and w.dtype == "bf16":
        import masked_head_attention_amd as M

        need = M.prenorm_cross_workspace_size(w.B, w.H, w.Lq, w.Lk, w.D, M.BF16)
        d["ws"] = torch.empty(need, dtype=torch.uint8, device="cuda")
    return d


def make_step(w: W.Workload, d):
    import masked_head_attention_amd as M

    if w.prenorm:
        res = d["x"] if w.residual else None

        def step():
            M.prenorm_cross_fwd(d["x"], d["k"], d["v"], d["gamma"], d["beta"], w.eps,
                                residual=res, mask=d["mask"], kind=w.kind, scale=w.scale,
                                out=d["out"], workspace=d.get("ws"))
    else:
        def step():
            M.fwd(d["q"], d["k"], d["v"], mask=d["mask"], kind=w.kind, scale=w.scale,
                  out=d["out"])
    return step


def time_gpu(step, K: int, Wm: int, eager: bool):
    """Seconds per step over exactly K steps (graph replay unless eager)."""
    import torch

    for _ in range(Wm):
        step()
    torch.cuda.synchronize()
    g = None
    if not eager:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(K):
                step()
        g.replay()  # one untimed replay of the captured steps
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if g is not None:
        g.replay()
    else:
        for _ in range(K):
            step()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3 / K


def time_cold(step, calls: int, flush_mib: int = 512):
    """Median seconds per call with the caches cold: before each call a fill
    kernel writes flush_mib MiB on the same stream (more than the 256 MB
    Infinity Cache and the L2s hold) and a second kernel reads another
    flush_mib MiB, which writes the fill's dirty lines back to HBM before the
    timed call; then the call alone is timed between HIP events. Per-call
    events include the launch gap, which graph replay hides."""
    import torch

    buf = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda")
    rd = torch.ones((flush_mib << 20) // 4, dtype=torch.float32, device="cuda")
    times = []
    for _ in range(calls + 1):  # the first call is untimed
        buf.fill_(1)
        rd.sum()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        step()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) * 1e-3)
    del buf, rd
    return float(np.median(times[1:]))


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------
def cpu_baseline(w: W.Workload, pairs_row: np.ndarray, target_s: float):
    import oracle

    rng = np.random.default_rng(1234)
    all_rows = w.B * w.H * w.Lq

    def rows_for(n):
        idx = rng.choice(all_rows, size=min(n, all_rows), replace=False)
        b, rem = idx // (w.H * w.Lq), idx % (w.H * w.Lq)
        h, i = rem // w.Lq, rem % w.Lq
        if w.prenorm:
            return np.stack([b, i, h], 1), b, i
        return np.stack([b, h, i], 1), b, i

    add64 = w.f64("add")
    args = {}
    if w.prenorm:
        x = w.f64("x")
        args = dict(x=x, k=w.f64("k"), v=w.f64("v"), gamma=w.f64("gamma"), beta=w.f64("beta"),
                    residual=x if w.residual else None)
    else:
        args = dict(q=w.f64("q"), k=w.f64("k"), v=w.f64("v"))

    def run(rows):
        if w.prenorm:
            oracle.prenorm_rows(args["x"], args["k"], args["v"], args["gamma"], args["beta"],
                                w.eps, rows, residual=args["residual"], kind=w.kind, lens=w.lens,
                                add=add64, scale=w.scale)
        else:
            oracle.mha_rows(args["q"], args["k"], args["v"], rows, w.kind, w.lens, add64,
                            w.scale)

    # warm up (thread pool, first touch), calibrate on a small sample, size the
    # timed sample to ~target_s, then repeat it until target_s has elapsed
    run(rows_for(min(all_rows, 64))[0])
    n0 = max(64, min(all_rows, 2048))
    rows, b, i = rows_for(n0)
    t0 = time.perf_counter()
    run(rows)
    t_cal = time.perf_counter() - t0
    per_row = t_cal / len(rows)
    n = int(min(all_rows, max(len(rows), target_s / max(per_row, 1e-9))))
    rows, b, i = rows_for(n)
    reps = 0
    t0 = time.perf_counter()
    while True:
        run(rows)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    flops = 4.0 * w.D * float(pairs_row[b, i].sum()) * reps
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"{len(rows)} of {all_rows} (b,h,query) rows drawn at random (seed 1234)"
                  f"{f', whole workload x{reps}' if reps > 1 else ''}; {dt:.1f} s of fp64 "
                  "three-pass oracle work",
        "seconds": dt,
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=4,
                    choices=sorted(W.CONFIGS) + [SOFTMAX_CONFIG_ID, DECODE_CONFIG_ID,
                                                 BWD_CONFIG_ID],
                    help=f"workload; {SOFTMAX_CONFIG_ID} = the row softmax of a materialised "
                         f"1x32x2048x2048 float16 score tensor; {DECODE_CONFIG_ID} = decode, one "
                         "new token per sequence against a float16 H=32 D=128 cache; "
                         f"{BWD_CONFIG_ID} = the backward of workload 3")
    ap.add_argument("--eager", action="store_true",
                    help="time launch-per-call steps instead of a graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timing of HBM-bound workloads")
    ap.add_argument("--no-workspace", action="store_true",
                    help="bfloat16 pre-LN: time mha_prenorm_cross_fwd (K/V rewritten tile by tile "
                         "in LDS) instead of mha_prenorm_cross_fwd_ws")
    ap.add_argument("--cold-calls", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run only a plain device copy of this size (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: every (batch, head) of this path is "
              f"independent, so N={args.gpus} GPUs would each run the one-GPU kernel on a "
              f"1/N share with no exchange; no multi-GPU figure is produced.", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)  # untimed first copy
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(5):
            dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        sec = s.elapsed_time(e) * 1e-3 / 5
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 6,
                          "us_per_copy": sec * 1e6, "hbm_GBs_read_plus_write": 2 * n * 4 / sec / 1e9}))
        return 0

    if args.config == SOFTMAX_CONFIG_ID:
        return main_softmax(args)
    if args.config == DECODE_CONFIG_ID:
        return main_decode(args)
    if args.config == BWD_CONFIG_ID:
        return main_bwd(args)

    import masked_head_attention_amd as M

    w = W.config(args.config)
    flops, alg_bytes, pairs_row = work(w)
    d = gpu_setup(w, workspace=not args.no_workspace)
    M.init()
    step = make_step(w, d)
    M.get_flags(clear=True)
    t_step = time_gpu(step, args.steps, args.warmup, args.eager)
    t_eager = t_step if args.eager else time_gpu(step, min(args.steps, 100), 5, True)
    flags = M.get_flags(clear=True)

    ai = flops / alg_bytes
    ridge = PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge:
        roof = {"bound": "mfma", "achieved": flops / t_step / 1e12,
                "peak": PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": alg_bytes / t_step / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_counter(w.name)
    executed = stored_counter(w.name, "executed_mfma_flops_per_launch")
    if executed is not None and roof["bound"] == "mfma":
        # executed MFMA work includes masked entries inside computed tiles
        roof["executed_mfma_frac"] = executed / t_step / 1e12 / PEAK_TFLOPS[w.dtype]
    cold = None
    if roof["bound"] == "hbm" and not args.no_cold:
        t_cold = time_cold(step, args.cold_calls)
        cold = {"us_per_call": t_cold * 1e6, "calls": args.cold_calls, "flush_mib": 512,
                "achieved": alg_bytes / t_cold / 1e9, "unit": "GB/s",
                "frac": alg_bytes / t_cold / 1e9 / PEAK_HBM_GBS,
                "timing": "median of per-call HIP events; before each call 512 MiB written and "
                          "another 512 MiB read, so the caches hold neither inputs nor dirty lines"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, pairs_row, args.cpu_seconds)

    value = flops / t_step / 1e12
    cfg = {"workload": w.name, "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "D": w.D,
           "mask": {0: "none", 1: "causal", 2: "padding", 3: "causal+padding", 4: "additive",
                    5: "causal+additive"}[w.kind] + (" pre-LN cross-attention" if w.prenorm else ""),
           "seed": w.seed, "effective_flops": flops, "algorithmic_bytes": alg_bytes,
           "timing": "eager launches" if args.eager else "HIP graph replay of the K steps"}
    if d.get("ws") is not None:
        cfg["workspace_bytes"] = d["ws"].numel()
        roof["timed"] = ("whole call (float16 K/V copy kernel + the attention kernel on the "
                         "copies + the attention kernel for heads beyond float16's range)")
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t_step * 1e3, "us_per_call": t_step * 1e6,
        "eager_us_per_call": t_eager * 1e6, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded, workloads.py recipe)",
        "config": cfg, "roofline": roof, "cold_cache": cold, "cpu_baseline": cpu,
        "device_flags": flags,
        "kernel_sources_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(line))
    return 0


def softmax_cpu_baseline(w, target_s: float):
    """The fp64 oracle on a random sample of rows, repeated to ~target_s;
    reported as algorithmic GB/s over the sample (read + write of the rows)."""
    import oracle

    rng = np.random.default_rng(1234)
    flat = w.s.reshape(w.rows, w.cols)
    E = ESIZE[w.dtype]

    def sample(n):
        idx = rng.choice(w.rows, size=min(n, w.rows), replace=False)
        return W.to_f64(flat[idx], w.dtype)

    oracle.softmax_rows(sample(16), w.scale)  # warm up
    x = sample(256)
    t0 = time.perf_counter()
    oracle.softmax_rows(x, w.scale)
    per_row = (time.perf_counter() - t0) / len(x)
    x = sample(int(min(w.rows, max(len(x), target_s / max(per_row, 1e-9)))))
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.softmax_rows(x, w.scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    return {"value": 2.0 * x.size * E * reps / dt / 1e9, "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{len(x)} of {w.rows} rows drawn at random (seed 1234), x{reps}; "
                      f"{dt:.1f} s of fp64 three-pass oracle work",
            "seconds": dt}


def main_softmax(args):
    """The row-softmax workload: one call = one softmax over the whole tensor."""
    import torch

    import masked_head_attention_amd as M

    w = W.softmax_config()
    E = ESIZE[w.dtype]
    alg_bytes = 2.0 * w.rows * w.cols * E  # every score read once, every weight written once
    s = torch.from_numpy(np.ascontiguousarray(w.s)).cuda()
    out = torch.empty_like(s)
    M.init()

    def step():
        M.softmax_rows(s, out=out, scale=w.scale)

    M.get_flags(clear=True)
    t_step = time_gpu(step, args.steps, args.warmup, args.eager)
    t_eager = t_step if args.eager else time_gpu(step, min(args.steps, 100), 5, True)
    flags = M.get_flags(clear=True)
    achieved = alg_bytes / t_step / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": stored_counter(w.name, kernel=SOFTMAX_KERNEL_NAME)}
    cold = None
    if not args.no_cold:
        t_cold = time_cold(step, args.cold_calls)
        cold = {"us_per_call": t_cold * 1e6, "calls": args.cold_calls, "flush_mib": 512,
                "achieved": alg_bytes / t_cold / 1e9, "unit": "GB/s",
                "frac": alg_bytes / t_cold / 1e9 / PEAK_HBM_GBS,
                "timing": "median of per-call HIP events; before each call 512 MiB written and "
                          "another 512 MiB read, so the caches hold neither inputs nor dirty lines"}
    cpu = None if args.no_cpu_baseline else softmax_cpu_baseline(w, args.cpu_seconds)
    line = {
        "metric": SOFTMAX_METRIC, "value": achieved, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": t_step * 1e3,
        "us_per_call": t_step * 1e6, "eager_us_per_call": t_eager * 1e6,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded, workloads.py recipe)",
        "config": {"workload": w.name, "shape": list(w.shape), "rows": w.rows, "cols": w.cols,
                   "scale": w.scale, "seed": w.seed, "algorithmic_bytes": alg_bytes,
                   "timing": "eager launches" if args.eager else "HIP graph replay of the K steps"},
        "roofline": roof, "cold_cache": cold, "cpu_baseline": cpu, "device_flags": flags,
        "kernel_sources_sha256_16": kernel_source_hash(SOFTMAX_KERNEL_NAME),
    }
    print(json.dumps(line))
    return 0


def decode_work(w: W.Workload):
    """(effective FLOPs, algorithmic bytes) of one decode call: q and out once,
    K and V for every legal cache row, the lengths and the float32 lse."""
    E = ESIZE[w.dtype]
    keys = float(np.clip(w.lens, 0, w.Lk).sum()) * w.H
    flops = 4.0 * w.D * keys
    alg = 2.0 * w.B * w.H * w.D * E + 2.0 * keys * w.D * E + 4.0 * w.B + 4.0 * w.B * w.H
    return flops, alg


def decode_cpu_baseline(w: W.Workload, target_s: float):
    """The fp64 oracle's decode on a random sample of (b, h) heads, repeated to
    ~target_s; reported as effective TFLOP/s over the sample's legal keys."""
    import oracle

    rng = np.random.default_rng(1234)
    n = min(64, w.B * w.H)
    idx = rng.choice(w.B * w.H, size=n, replace=False)
    bs, hs = idx // w.H, idx % w.H
    q = W.to_f64(w.q.reshape(w.B, w.H, w.D)[bs, hs][:, None], w.dtype)
    k = W.to_f64(w.k[bs, hs][:, None], w.dtype)
    v = W.to_f64(w.v[bs, hs][:, None], w.dtype)
    lens = np.ascontiguousarray(w.lens[bs])
    oracle.decode(q[:2], k[:2], v[:2], lens[:2], w.scale)  # warm up
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(q, k, v, lens, w.scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    flops = 4.0 * w.D * float(np.clip(lens, 0, w.Lk).sum()) * reps
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{n} of {w.B * w.H} (b,h) heads drawn at random (seed 1234), x{reps}; "
                      f"{dt:.1f} s of fp64 three-pass oracle work",
            "seconds": dt}


def main_decode(args):
    """The decode workload: one call = one new token for every sequence and
    head (the split kernel and, when keys are split, the merge kernel)."""
    import torch

    import masked_head_attention_amd as M

    w = W.decode_config()
    flops, alg_bytes = decode_work(w)
    d = gpu_setup(w)
    q = d["q"].view(w.B, w.H, w.D)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    code = {"f32": M.F32, "f16": M.F16, "bf16": M.BF16}[w.dtype]
    ws = torch.empty(max(1, M.decode_workspace_size(w.B, w.H, w.Lk, w.D, code)),
                     dtype=torch.uint8, device="cuda")
    M.init()

    def step():
        M.decode(q, d["k"], d["v"], d["mask"], scale=w.scale, out=out, lse=lse, workspace=ws)

    M.get_flags(clear=True)
    t_step = time_gpu(step, args.steps, args.warmup, args.eager)
    t_eager = t_step if args.eager else time_gpu(step, min(args.steps, 100), 5, True)
    flags = M.get_flags(clear=True)
    achieved = alg_bytes / t_step / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": stored_counter(w.name, kernel=DECODE_KERNEL_NAME),
            "timed": "whole call (split kernel + merge kernel)"}
    cold = None
    if not args.no_cold:
        t_cold = time_cold(step, args.cold_calls)
        cold = {"us_per_call": t_cold * 1e6, "calls": args.cold_calls, "flush_mib": 512,
                "achieved": alg_bytes / t_cold / 1e9, "unit": "GB/s",
                "frac": alg_bytes / t_cold / 1e9 / PEAK_HBM_GBS,
                "timing": "median of per-call HIP events; before each call 512 MiB written and "
                          "another 512 MiB read, so the caches hold neither inputs nor dirty lines"}
    cpu = None if args.no_cpu_baseline else decode_cpu_baseline(w, args.cpu_seconds)
    line = {
        "metric": METRIC, "value": flops / t_step / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": t_step * 1e3,
        "us_per_call": t_step * 1e6, "eager_us_per_call": t_eager * 1e6,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded, workloads.py recipe)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Lq": 1, "Lk": w.Lk, "D": w.D,
                   "mask": "cache lengths", "seed": w.seed, "effective_flops": flops,
                   "algorithmic_bytes": alg_bytes,
                   "timing": "eager launches" if args.eager else "HIP graph replay of the K steps"},
        "roofline": roof, "cold_cache": cold, "cpu_baseline": cpu, "device_flags": flags,
        "kernel_sources_sha256_16": kernel_source_hash(DECODE_KERNEL_NAME),
    }
    print(json.dumps(line))
    return 0


def bwd_cpu_baseline(w: W.Workload, g: np.ndarray, pairs_row: np.ndarray, target_s: float):
    """The fp64 oracle's backward on a random sample of (b, h) heads, repeated
    to ~target_s; reported as effective TFLOP/s (10 D per legal pair)."""
    import oracle

    rng = np.random.default_rng(1234)
    n = min(16, w.B * w.H)
    idx = rng.choice(w.B * w.H, size=n, replace=False)
    bs, hs = idx // w.H, idx % w.H
    q = W.to_f64(w.q[bs, hs][:, None], w.dtype)
    k = W.to_f64(w.k[bs, hs][:, None], w.dtype)
    v = W.to_f64(w.v[bs, hs][:, None], w.dtype)
    go = W.to_f64(g[bs, hs][:, None], w.dtype)
    lens = None if w.lens is None else np.ascontiguousarray(w.lens[bs])
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.mha_bwd(q, k, v, go, w.kind, lens, None, w.scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    flops = 10.0 * w.D * float(pairs_row[bs].sum()) * reps
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{n} of {w.B * w.H} (b,h) heads drawn at random (seed 1234), x{reps}; "
                      f"{dt:.1f} s of fp64 oracle backward work",
            "seconds": dt}


def main_bwd(args):
    """The backward workload: one call = dQ, dK, dV of workload 3 (two kernels)."""
    import torch

    import masked_head_attention_amd as M

    w = W.config(W.BWD_CONFIG)
    g = W.grad_output(w)
    fwd_flops, _, pairs_row = work(w)
    flops = fwd_flops * 10.0 / 4.0  # five products of 2 D per legal pair, not two
    E = ESIZE[w.dtype]
    alg_bytes = 7.0 * w.B * w.H * w.Lq * w.D * E  # q, k, v, dO in; dq, dk, dv out (Lq = Lk)
    d = gpu_setup(w)
    go = torch.from_numpy(np.ascontiguousarray(g)).cuda()
    dq, dk, dv = (torch.empty_like(d[n]) for n in ("q", "k", "v"))
    code = {"f32": M.F32, "f16": M.F16, "bf16": M.BF16}[w.dtype]
    ws = torch.empty(max(1, M.bwd_workspace_size(w.B, w.H, w.Lq, code)), dtype=torch.uint8,
                     device="cuda")
    M.init()

    def step():
        M.bwd(d["q"], d["k"], d["v"], go, mask=d["mask"], kind=w.kind, scale=w.scale, dq=dq,
              dk=dk, dv=dv, workspace=ws)

    M.get_flags(clear=True)
    t_step = time_gpu(step, args.steps, args.warmup, args.eager)
    t_eager = t_step if args.eager else time_gpu(step, min(args.steps, 100), 5, True)
    flags = M.get_flags(clear=True)
    roof = {"bound": "mfma", "achieved": flops / t_step / 1e12, "peak": PEAK_TFLOPS[w.dtype],
            "unit": "TFLOP/s", "frac": flops / t_step / 1e12 / PEAK_TFLOPS[w.dtype],
            "traffic": stored_counter(w.name + "-bwd", kernel=BWD_KERNEL_NAME),
            "timed": "whole call (dq kernel + dkv kernel)"}
    executed = stored_counter(w.name + "-bwd", "executed_mfma_flops_per_launch",
                              kernel=BWD_KERNEL_NAME)
    if executed is not None:
        roof["executed_mfma_frac"] = executed / t_step / 1e12 / PEAK_TFLOPS[w.dtype]
    cpu = None if args.no_cpu_baseline else bwd_cpu_baseline(w, g, pairs_row, args.cpu_seconds)
    line = {
        "metric": BWD_METRIC, "value": flops / t_step / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": t_step * 1e3,
        "us_per_call": t_step * 1e6, "eager_us_per_call": t_eager * 1e6,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded, workloads.py recipe)",
        "config": {"workload": w.name + "-bwd", "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk,
                   "D": w.D, "mask": "causal", "seed": w.seed, "effective_flops": flops,
                   "algorithmic_bytes": alg_bytes,
                   "timing": "eager launches" if args.eager else "HIP graph replay of the K steps"},
        "roofline": roof, "cpu_baseline": cpu, "device_flags": flags,
        "kernel_sources_sha256_16": kernel_source_hash(BWD_KERNEL_NAME),
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
