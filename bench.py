#!/usr/bin/env python3
"""Benchmark of the EntropyCache denoising step on one MI355X.

Prints ONE JSON line (see the repository's design notes for the contract):
  metric / value / unit ...  whole-job throughput, inputs resident in HBM
  roofline                   the dominant kernel against its bound, timed live
                             with HIP events on the stream it runs on
  cpu_baseline               the float64 oracle on a bounded sample of the same
                             workload, on this host's cores
Workloads:
  entropy   4096 x 126464 bf16 logits, one fused entropy pass per step (GB/s)
  step      LLaDA-8B-shaped layer, L = 1024, EntropyCache loop (steps/s)
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

METRIC = "denoise steps/s + HBM GB/s of entropy pass, L=1k–32k; fraction of roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def _log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _src_hash(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "entropy_gated_kv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, src: str, per_launch_units: float):
    """HBM bytes per launch from the committed counter summary, or None if the
    kernel source changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_hash") != _src_hash(src):
        return None
    return rec.get("bytes_per_launch")


def _cpu_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# --------------------------------------------------------------------------- entropy
def entropy_leg(steps: int, warmup: int, cpu_baseline: bool) -> dict:
    import numpy as np
    import torch

    from entropy_gated_kv_amd import lib as L
    from synth import configs as C
    from synth import generators as G

    cfg = C.ENTROPY_ONLY
    _log(f"generating {cfg.rows}x{cfg.vocab} synthetic logits")
    z = G.entropy_logits(cfg)
    x = torch.from_numpy(z).to(torch.bfloat16).cuda()
    n, V = x.shape
    H = torch.empty(n, device="cuda", dtype=torch.float32)
    A = torch.empty(n, device="cuda", dtype=torch.int32)
    P = torch.empty(n, device="cuda", dtype=torch.float32)
    E = torch.empty(1, device="cuda", dtype=torch.float32)
    F = torch.empty(1, device="cuda", dtype=torch.int32)
    ws = torch.zeros(L.ec_entropy_workspace_bytes(n, V), device="cuda", dtype=torch.uint8)

    def one():
        L.ec_entropy_max(x, cfg.tau, H, E, F, ws, row_argmax=A, row_top1=P)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        one()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    bytes_per = n * V * 2 + n * 12            # logits read once + H, argmax, p1 written
    gbs = bytes_per / (kern_ms * 1e-3) / 1e9
    out = {
        "ms_per_step": wall * 1e3 / steps,
        "kernel_ms": kern_ms,
        "GB_per_s": gbs,
        "frac": gbs / HBM_PEAK_GBS,
        "bytes_per_launch": bytes_per,
        "e_max": float(E.item()),
        "flag": int(F.item()),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": _traffic("entropy_kernel<bf16>", "entropy.hip", 1),
                     "kernel": "entropy_kernel<bf16> (one fused launch per pass)"},
    }
    _log(f"entropy pass: {kern_ms * 1e3:.1f} us/launch, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM peak)")
    if cpu_baseline:
        out["cpu_baseline"] = entropy_cpu_baseline(z, V)
    return out


def entropy_cpu_baseline(z, V: int) -> dict:
    import numpy as np

    import oracle as O

    rows, budget, t0 = 0, 12.0, time.perf_counter()
    while time.perf_counter() - t0 < budget and rows < z.shape[0]:
        O.softmax_entropy(z[rows].astype(np.float64))
        rows += 1
    dt = time.perf_counter() - t0
    gbs = rows * V * 2 / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of 4096 rows, one row at a time (NumPy float64, single thread), {dt:.1f} s"}


# --------------------------------------------------------------------------- main
def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="entropy", choices=["entropy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the design notes describe how the step would shard)", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    res = entropy_leg(args.steps, args.warmup, not args.no_cpu_baseline)
    line = {
        "metric": METRIC,
        "value": round(res["GB_per_s"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "entropy_4096x126464_bf16", "rows": 4096, "vocab": 126464,
                   "tau": 2.0},
        "roofline": res["roofline"],
    }
    if "cpu_baseline" in res:
        line["cpu_baseline"] = res["cpu_baseline"]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
