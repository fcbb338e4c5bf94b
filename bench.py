#!/usr/bin/env python3
"""Benchmark of the EntropyCache denoising step on one MI355X.

Prints ONE JSON line (see the repository's design notes for the contract):
  metric / value / unit ...  whole-job throughput, inputs resident in HBM
  roofline                   the dominant kernel against its bound, timed live
                             with HIP events on the stream it runs on
  cpu_baseline               the float64 oracle on a bounded sample of the same
                             workload, on this host's cores
Workloads:
  step      LLaDA-8B-shaped layer (d 4096, 32 x 128 heads, V 126464), L = 1024 =
            512 prompt + 512 generated in blocks of 32, EntropyCache loop at
            tau = 1.0 (k = 64): one step = select, embed, QKV refresh,
            attention, O-projection, LM head, entropy pass, unmask + decision.
            value = denoise steps/s.  Also: tau sweep, vanilla (tau = -inf).
  entropy   4096 x 126464 bf16 logits, one entropy pass (GB/s); reported as
            the "entropy_pass" object next to the step line.
  stack32   the 32-layer LLaDA-shaped stack (RMSNorm + SwiGLU 12288), L = 2048:
            end-to-end steps/s at tau = 1.0 and vanilla ("stack32").
  long      the Dream-shaped layer at L = 8224 / 32800, steady state: partial
            and full step times, attention MFMA fraction ("long_context").
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
    """Hash of the code of kernel sources: comments and blank space are left
    out, so only a change to the code itself voids recorded counters."""
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "entropy_gated_kv_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# kernels whose HBM traffic is recorded: the name fragment the counter rows
# carry, the source file, and which launches count (all, or the largest grid)
TRAFFIC_KERNELS = {
    "entropy_partials_kernel<bf16>": ("entropy_partials_kernel<ec::bf16_t>", "entropy.hip", "largest"),
    "lmhead_packed_kernel<3>": ("lmhead_packed_kernel<3>", "gemm.hip", "all"),
}


def record_traffic(fetch_dir: str, write_dir: str) -> dict:
    """Turn two `rocprofv3 --pmc` runs of `bench.py --profile-mode` (FETCH_SIZE,
    then WRITE_SIZE; CSV output directories) into profiles/traffic.json.  Each
    counter is scaled by what it reads for the profile mode's 1 GiB copies."""
    import csv
    import glob

    def rows(d):
        (path,) = glob.glob(os.path.join(d, "*counter_collection.csv"))
        with open(path) as f:
            return list(csv.DictReader(f))

    f_rows, w_rows = rows(fetch_dir), rows(write_dir)
    gib_kib = float(1 << 20)
    copy_grid = str(1 << 17)       # the 1 GiB copies' grid (threads)

    def mean(rs, frag, grid=None):
        v = [float(r["Counter_Value"]) for r in rs
             if frag in r["Kernel_Name"] and (grid is None or r["Grid_Size"] == grid)]
        if not v:
            raise RuntimeError(f"no counter rows for {frag}")
        return sum(v) / len(v), len(v)

    cal_f, _ = mean(f_rows, "copyBuffer", copy_grid)
    cal_w, _ = mean(w_rows, "copyBuffer", copy_grid)
    sf, sw = gib_kib / cal_f, gib_kib / cal_w
    rec = {"_calibration": {"copy_bytes": 1 << 30, "fetch_kib": cal_f, "write_kib": cal_w,
                            "fetch_scale": sf, "write_scale": sw}}
    for key, (frag, src, which) in TRAFFIC_KERNELS.items():
        grid = None
        if which == "largest":
            grid = str(max(int(r["Grid_Size"]) for r in f_rows if frag in r["Kernel_Name"]))
        fk, n = mean(f_rows, frag, grid)
        wk, _ = mean(w_rows, frag, grid)
        rec[key] = {"src_hash": _src_hash(src), "fetch_kib": fk, "write_kib": wk,
                    "bytes_per_launch": round((fk * sf + wk * sw) * 1024), "launches": n}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def _kernel_key(r):
    import re
    name = re.sub(r"\(anonymous namespace\)::", "", r["Kernel_Name"])
    name = re.sub(r"^void ", "", name.split("(")[0]).replace("ec::", "")
    grid = r["Grid_Size"] if "Grid_Size" in r else r["Grid_Size_X"]          # counter / trace CSVs
    wg = r["Workgroup_Size"] if "Workgroup_Size" in r else r["Workgroup_Size_X"]
    return name, int(grid) // max(1, int(wg))


def summarize_trace(trace_dir: str, min_us: float) -> str:
    """Markdown table of a `rocprofv3 --kernel-trace` run (CSV output
    directory), per kernel and grid: calls, the calls longer than min_us
    (device-gated launches that exit at once are shorter), the median and
    maximum duration of those, and the total time of all calls."""
    import collections
    import csv
    import glob
    import statistics

    groups = collections.defaultdict(list)
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                groups[_kernel_key(r)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    out = [f"| kernel | workgroups | calls | calls > {min_us:g} us | median of those (us) | max (us) | total (ms) |",
           "|---|---|---|---|---|---|---|"]
    for (name, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        big = [x for x in v if x > min_us]
        med = f"{statistics.median(big):.1f}" if big else "-"
        out.append(f"| `{name}` | {wg} | {len(v)} | {len(big)} | {med} | {max(v):.1f} | {sum(v) / 1e3:.2f} |")
    return "\n".join(out) + "\n"


def summarize_counters(dirs) -> str:
    """Markdown table of `rocprofv3 --pmc` runs (CSV output directories), per
    kernel and grid, over the dispatches that did work (device-gated launches
    that exit at once are counted but left out of the means):
      time           median dispatch duration (counter-run timestamps)
      GFLOP          bf16 MFMA flops per dispatch, SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512
      TFLOP/s, frac  GFLOP / time, and that over the 2.5 PFLOP/s bf16 peak
      MFMA busy      SQ_VALU_MFMA_BUSY_CYCLES / (time x 2.4 GHz x 1024 SIMDs)
      clock          GRBM_GUI_ACTIVE / 8 XCDs / time (dispatches over 200 us;
                     shorter windows carry the profiler's own cycles)
      VALU, wait     SQ_ACTIVE_INST_VALU and SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES
      LDS conflict   SQ_LDS_BANK_CONFLICT over SQ_ACTIVE_INST_LDS"""
    import collections
    import csv
    import glob
    import re
    import statistics

    disp = {}                                    # (run, dispatch) -> (key, us, counters)
    for ri, d in enumerate(dirs):
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    name = re.sub(r"\(anonymous namespace\)::", "", r["Kernel_Name"])
                    name = re.sub(r"^void ", "", name.split("(")[0]).replace("ec::", "")
                    key = (name, int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
                    us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
                    rec = disp.setdefault((ri, r["Dispatch_Id"]), (key, us, {}))
                    rec[2][r["Counter_Name"]] = float(r["Counter_Value"])
    groups = collections.defaultdict(list)
    for (ri, _), (key, us, c) in disp.items():
        groups[key].append((us, c))
    rows = []
    for key, ds in groups.items():
        if not key[0].startswith(("attn", "gemm", "lmhead", "entropy", "select", "rmsnorm", "value_drift")):
            continue
        big = max(c.get("SQ_WAVE_CYCLES", c.get("SQ_BUSY_CYCLES", 0.0)) for _, c in ds)
        act = [(us, c) for us, c in ds
               if c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) > 0
               or c.get("SQ_WAVE_CYCLES", 0) > 0.05 * big > 0]
        if not act:
            continue
        def med(f):
            v = [f(us, c) for us, c in act if f(us, c) is not None]
            return statistics.median(v) if v else None
        us = med(lambda u, c: u)
        gf = med(lambda u, c: c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9 if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c else None)
        busy = med(lambda u, c: c["SQ_VALU_MFMA_BUSY_CYCLES"] / (u * 2400.0 * 1024) if "SQ_VALU_MFMA_BUSY_CYCLES" in c else None)
        clk = med(lambda u, c: c["GRBM_GUI_ACTIVE"] / 8 / u / 1000 if "GRBM_GUI_ACTIVE" in c and u > 200 else None)
        valu = med(lambda u, c: c["SQ_ACTIVE_INST_VALU"] / c["SQ_WAVE_CYCLES"] if c.get("SQ_WAVE_CYCLES") else None)
        wait = med(lambda u, c: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"] if c.get("SQ_WAVE_CYCLES") else None)
        ldsc = med(lambda u, c: c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"] if c.get("SQ_ACTIVE_INST_LDS") else None)
        rows.append((key, len(act), len(ds), us, gf, busy, clk, valu, wait, ldsc))
    fmt = lambda v, f: "" if v is None else format(v, f)
    out = ["| kernel | workgroups | dispatches (with work / all) | time us | bf16 MFMA GFLOP | TFLOP/s | "
           "frac of 2.5 PF | MFMA busy | clock GHz | VALU / wave-cycles | wait / wave-cycles | "
           "LDS conflict / LDS cycles |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for key, na, nd, us, gf, busy, clk, valu, wait, ldsc in sorted(rows, key=lambda r: -(r[4] or 0) * r[1]):
        tf = gf / us * 1e3 if gf and us else None
        out.append(f"| `{key[0]}` | {key[1]} | {na} / {nd} | {fmt(us, '.1f')} | {fmt(gf, '.2f')} | "
                   f"{fmt(tf, '.0f')} | {fmt(tf / 2500 if tf else None, '.3f')} | {fmt(busy, '.3f')} | "
                   f"{fmt(clk, '.2f')} | {fmt(valu, '.3f')} | {fmt(wait, '.3f')} | {fmt(ldsc, '.3f')} |")
    return "\n".join(out)


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
    # HIP events on the launch stream around the whole timed region: the
    # average pass (partials, combine and decide kernels, back to back)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        one()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = a.elapsed_time(b) / steps
    bytes_per = n * V * 2 + n * 12            # logits read once + H, argmax, p1 written
    gbs = bytes_per / (kern_ms * 1e-3) / 1e9
    out = {
        "ms_per_step": wall * 1e3 / steps,
        "kernel_ms": kern_ms,
        "GB_per_s": gbs,
        "rows_per_s": n / (kern_ms * 1e-3),
        "frac": gbs / HBM_PEAK_GBS,
        "bytes_per_launch": bytes_per,
        "e_max": float(E.item()),
        "flag": int(F.item()),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": _traffic("entropy_partials_kernel<bf16>", "entropy.hip", 1),
                     "kernel": "entropy pass: entropy_partials_kernel<bf16> + combine + decide"},
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


# --------------------------------------------------------------------------- step
PHASES = ("select", "embed", "qkv", "attn", "oproj", "ffn", "lmhead", "entropy", "decide")


def step_leg(steps: int, warmup: int, cpu_baseline: bool) -> dict:
    import numpy as np
    import torch

    from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence
    from synth import configs as C
    from synth import generators as G

    cfg = C.LLADA_LAYER
    tau = 1.0
    _log(f"generating weights of {cfg.name}")
    w = G.model_weights(cfg)
    toks, masked = G.initial_sequence(cfg)
    dm = DeviceModel(cfg.model, cfg.dtype, cfg.L, w)
    # No logits buffer: the packed LM head writes each candidate's softmax
    # statistics instead of its logits, and the step decides from those (the
    # with-logits rate is reported below)
    ds = DeviceSequence(dm, toks, masked, history_cap=cfg.gen_len, max_block=cfg.block_len,
                        keep_logits=False)
    sched = C.unmask_schedule(cfg)
    init = (ds.tokens.clone(), ds.is_masked.clone())
    stream = torch.cuda.current_stream()

    def reset():   # device-side copies only (no host synchronisation)
        ds.tokens.copy_(init[0])
        ds.is_masked.copy_(init[1])
        ds.history_len.zero_()
        ds.full_flag.fill_(1)

    def run(n_steps, tau_, events=None, flags=None, k=cfg.k):
        i = 0
        while i < n_steps:
            for j, (bs, bl, n) in enumerate(sched):
                if i >= n_steps:
                    break
                if flags is not None:
                    flags[i].copy_(ds.full_flag[0])
                ev = None if events is None else events[i]
                ds.step(tau_, k, bs, bl, n, phase_events=ev)
                i += 1
            else:
                reset()

    # Inside the timed region only the dominant kernel (the LM head) is
    # bracketed by events, on every EV_EVERY-th timed step: a pair of event
    # records costs a few microseconds of stream time, which on every step
    # would take about 1% off the measured rate.
    EV_EVERY = 4
    LM = PHASES.index("lmhead")
    n_ev = 2 * len(PHASES)

    def event_set(only_lm):
        """Events for one step: every phase, or (only_lm) the LM head alone."""
        evs = [None] * n_ev
        for k in range(n_ev):
            if only_lm and k // 2 != LM:
                continue
            evs[k] = torch.cuda.Event(enable_timing=True)
            evs[k].record()                 # materialise the event handle
        return evs

    # The timed steps are spread over the whole generation, so the headline
    # does not depend on how many are timed: n_seq = min(steps, schedule
    # length) sequences start at evenly spaced points of the schedule
    # (snapshots of one untimed trajectory; every sequence then follows that
    # same deterministic trajectory), and timed step i advances sequence
    # i mod n_seq by one denoising step.  With the whole schedule timed, the
    # timed steps are exactly the trajectory's steps, each once; fewer timed
    # steps are an evenly spaced sample of it.  A sequence that finishes
    # starts again from the prompt.  Sequences share one workspace (scratch).
    # Each timed step then runs on a different sequence's state, as in
    # serving several sequences, which measures about 1-2% slower than one
    # sequence stepping alone (the tau sweep below).
    n_seq = max(1, min(steps, len(sched)))
    phases = [j * len(sched) // n_seq for j in range(n_seq)]
    seqs = [DeviceSequence(dm, toks, masked, history_cap=cfg.gen_len, max_block=cfg.block_len,
                           ws=ds.ws, keep_logits=False) for _ in range(n_seq)]
    sched_flags = torch.zeros(len(sched), dtype=torch.int32, device="cuda")

    def stage():
        """Put sequence j at schedule index phases[j]; record the flag each
        schedule index runs with (the trajectory is deterministic)."""
        reset()
        j = 0
        for s_idx, (bs, bl, nn) in enumerate(sched):
            while j < n_seq and phases[j] == s_idx:
                seqs[j].copy_state_from(ds)
                j += 1
            sched_flags[s_idx].copy_(ds.full_flag[0])
            ds.step(tau, cfg.k, bs, bl, nn)
        return list(phases)

    def seq_step(pos, i, ev=None):
        j = i % n_seq
        if pos[j] == len(sched):                  # finished: a fresh sequence
            sq = seqs[j]
            sq.tokens.copy_(init[0])
            sq.is_masked.copy_(init[1])
            sq.history_len.zero_()
            sq.full_flag.fill_(1)
            pos[j] = 0
        bs, bl, nn = sched[pos[j]]
        seqs[j].step(tau, cfg.k, bs, bl, nn, phase_events=ev)
        pos[j] += 1
        return pos[j] - 1

    pos = stage()
    for i in range(warmup):
        seq_step(pos, i)
    torch.cuda.synchronize()
    timed_events = [event_set(True) if i % EV_EVERY == 0 else None for i in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    idx = [seq_step(pos, warmup + i, timed_events[i]) for i in range(steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_steps = [i for i in range(steps) if timed_events[i] is not None]
    lm_ms = float(np.mean([timed_events[i][2 * LM].elapsed_time(timed_events[i][2 * LM + 1])
                           for i in ev_steps]))

    # untimed replay of the same (deterministic) steps with every phase
    # bracketed, for the breakdown; the step modes come from the trajectory
    pos = stage()
    for i in range(warmup):
        seq_step(pos, i)
    torch.cuda.synchronize()
    bd_events = [event_set(False) for _ in range(steps)]
    for i in range(steps):
        seq_step(pos, warmup + i, bd_events[i])
    torch.cuda.synchronize()
    fl = sched_flags.cpu().numpy()[idx]
    del seqs
    phase_ms = {}
    by_mode = {"partial": {}, "full": {}}
    for k, name in enumerate(PHASES):
        if name == "ffn":
            continue
        t = np.array([ev[2 * k].elapsed_time(ev[2 * k + 1]) for ev in bd_events])
        phase_ms[name] = float(t.mean())
        for mode, want in (("partial", 0), ("full", 1)):
            if (fl == want).any():
                by_mode[mode][name] = float(t[fl == want].mean())
    # LM-head algorithmic bytes per launch: W_lm read once, the candidates'
    # activations read and their softmax statistics written, 16 bytes per row
    # and group of three column tiles (the launch plan at this V on 256 CUs);
    # m = mean candidate count over the launches the events timed (the
    # block's still-masked positions at each step)
    d, V = cfg.model.d, cfg.model.vocab
    cand = []
    left, cur = cfg.block_len, None
    for bs, bl, nn in sched:
        if bs != cur:
            cur, left = bs, bl
        cand.append(left)
        left -= nn
    m = float(np.mean([cand[idx[i]] for i in ev_steps]))
    lm_bytes = int(V * d * 2 + m * d * 2 + m * ((V + 191) // 192) * 16)
    lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
    decide_ms = phase_ms["select"] + phase_ms["entropy"] + phase_ms["decide"]
    # each phase against its roofline: max(bytes / HBM peak, flops / bf16 MFMA peak),
    # partial steps at 96 selected rows (32 block rows + k = 64), full steps at L
    mm = cfg.model
    L_, hd = cfg.L, mm.n_q_heads * mm.head_dim
    nqkv = (mm.n_q_heads + 2 * mm.n_kv_heads) * mm.head_dim
    kv_bytes = 2 * mm.n_kv_heads * L_ * mm.head_dim * 2
    def ideal_us(nbytes, flops):
        return max(nbytes / (HBM_PEAK_GBS * 1e3), flops / (BF16_PEAK_TFLOPS * 1e6))
    n_p = cfg.block_len + cfg.k
    ideal = {
        "partial": {"qkv": ideal_us(nqkv * d * 2, 2.0 * n_p * d * nqkv),
                    "attn": ideal_us(kv_bytes, 4.0 * n_p * L_ * hd),
                    "oproj": ideal_us(d * hd * 2, 2.0 * n_p * hd * d),
                    "lmhead": ideal_us(lm_bytes, 2.0 * m * d * V)},
        "full": {"qkv": ideal_us(nqkv * d * 2 + L_ * d * 2, 2.0 * L_ * d * nqkv),
                 "attn": ideal_us(kv_bytes, 4.0 * L_ * L_ * hd),
                 "oproj": ideal_us(d * hd * 2, 2.0 * L_ * hd * d),
                 "lmhead": ideal_us(lm_bytes, 2.0 * m * d * V)},
    }
    phase_roofline = {
        mode: {name: {"us": round(by_mode[mode][name] * 1e3, 2), "ideal_us": round(iu, 2),
                      "frac": round(iu / (by_mode[mode][name] * 1e3), 3)}
               for name, iu in ideal[mode].items() if name in by_mode[mode]}
        for mode in ideal}
    # Each phase's events cost stream time of their own: the evented replay of
    # the timed steps exceeds their event-free time by this much per phase
    # (every phase the step runs records its pair, the empty decide phase
    # included; a layer without FFN records none for it); the phase figures
    # above are raw and include it.
    evented = [k for k, name in enumerate(PHASES) if name != "ffn" or cfg.model.d_ffn > 0]
    phase_sum_ms = float(np.mean([sum(ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in evented)
                                  for ev in bd_events]))
    event_ovh_us = (phase_sum_ms - wall * 1e3 / steps) * 1e3 / len(evented)
    out = {
        "value": steps / wall,
        "ms_per_step": wall * 1e3 / steps,
        "partial_fraction": float(1.0 - fl.mean()),
        "phases_us": {k: round(v * 1e3, 2) for k, v in phase_ms.items()},
        "phase_event_overhead_us": round(event_ovh_us, 2),
        "decision_overhead_frac": decide_ms / sum(phase_ms.values()),
        "phase_roofline": phase_roofline,
        "roofline": {"bound": "hbm", "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(lm_gbs / HBM_PEAK_GBS, 4),
                     "traffic": _traffic("lmhead_packed_kernel<3>", "gemm.hip", 1),
                     "kernel": "LM head on the packed weight, three column tiles per workgroup, "
                               "softmax statistics in place of logits (lmhead_packed_kernel<3>)",
                     "bytes_per_launch": lm_bytes, "avg_launch_us": round(lm_ms * 1e3, 2)},
    }
    _log(f"step: {out['value']:.1f} steps/s, {out['ms_per_step'] * 1e3:.1f} us/step, "
         f"partial fraction {out['partial_fraction']:.2f}; LM head {lm_ms * 1e3:.1f} us = {lm_gbs:.0f} GB/s")
    _log("phases (us, separate pass): " + ", ".join(f"{k} {v * 1e3:.1f}" for k, v in phase_ms.items()))

    # tau sweep and vanilla, then the history length k at tau = 1: one whole
    # generation each.  Every run also reports how many of its decoded tokens
    # equal vanilla decoding's (a proxy, on synthetic weights, for how far
    # reusing stale K/V moves the decisions).
    def generation(t, k):
        reset()
        torch.cuda.synchronize()
        fl2 = torch.zeros(len(sched), dtype=torch.int32, device="cuda")
        t1 = time.perf_counter()
        run(len(sched), t, None, fl2, k)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t1
        return ({"steps_per_s": round(len(sched) / dt, 2),
                 "partial_fraction": round(float(1.0 - fl2.float().mean().item()), 3)},
                ds.tokens.cpu().numpy())

    vanilla, van_tok = generation(float("-inf"), cfg.k)
    gen = np.asarray(masked, dtype=bool)                     # generated positions
    sweep = {}
    for t in (0.5, 1.0, 2.0):
        rec, tok = generation(t, cfg.k)
        rec["token_agreement_vs_vanilla"] = round(float((tok[gen] == van_tok[gen]).mean()), 4)
        sweep[str(t)] = rec
    sweep["-inf"] = vanilla
    out["tau_sweep"] = sweep
    out["speedup_vs_vanilla_at_tau_1"] = round(sweep["1.0"]["steps_per_s"] / sweep["-inf"]["steps_per_s"], 3)
    _log(f"tau sweep: {sweep}")
    kab = {}
    for k in (1, 16, 64, 256):
        rec, tok = generation(1.0, k)
        rec["token_agreement_vs_vanilla"] = round(float((tok[gen] == van_tok[gen]).mean()), 4)
        kab[str(k)] = rec
    out["k_ablation_tau_1"] = kab
    _log(f"k ablation (tau 1.0): {kab}")

    # the same tau = 1 generation when the step also returns the candidates'
    # logits (a logits buffer: the LM head writes them and the entropy pass
    # reads them back), and that LM head's time from events on every step of
    # a second run
    dl = DeviceSequence(dm, toks, masked, history_cap=cfg.gen_len, max_block=cfg.block_len, ws=ds.ws)
    fl_l = torch.zeros(len(sched), dtype=torch.int32, device="cuda")
    def gen_logits(events):
        dl.tokens.copy_(init[0])
        dl.is_masked.copy_(init[1])
        dl.history_len.zero_()
        dl.full_flag.fill_(1)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i, (bs, bl, nn) in enumerate(sched):
            fl_l[i].copy_(dl.full_flag[0])
            dl.step(tau, cfg.k, bs, bl, nn, phase_events=None if events is None else events[i])
        torch.cuda.synchronize()
        return time.perf_counter() - t1
    dt_l = gen_logits(None)
    lm_ev = [event_set(True) for _ in sched]
    gen_logits(lm_ev)
    lm_l_us = float(np.mean([e[2 * LM].elapsed_time(e[2 * LM + 1]) for e in lm_ev])) * 1e3
    out["with_logits"] = {"steps_per_s": round(len(sched) / dt_l, 2),
                          "partial_fraction": round(float(1.0 - fl_l.float().mean().item()), 3),
                          "lmhead_us": round(lm_l_us, 2),
                          "note": "tau = 1 generation with a logits buffer; lmhead_us from events on "
                                  "every step of a second run"}
    _log(f"with logits: {out['with_logits']}")
    del dl

    # sliding-window decoding: the same unmask counts, the block being the 32
    # positions from the first masked one (block_start = -1)
    def sliding(t):
        reset()
        torch.cuda.synchronize()
        fl2 = torch.zeros(len(sched), dtype=torch.int32, device="cuda")
        t1 = time.perf_counter()
        for i, (bs, bl, nn) in enumerate(sched):
            fl2[i].copy_(ds.full_flag[0])
            ds.step(t, cfg.k, -1, bl, nn)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t1
        return ({"steps_per_s": round(len(sched) / dt, 2),
                 "partial_fraction": round(float(1.0 - fl2.float().mean().item()), 3),
                 "still_masked": int(ds.is_masked.sum().item())}, ds.tokens.cpu().numpy())

    sl_van, sl_van_tok = sliding(float("-inf"))
    sl_ec, sl_tok = sliding(tau)
    done = gen & (ds.is_masked.cpu().numpy() == 0)
    sl_ec["token_agreement_vs_vanilla"] = round(float((sl_tok[done] == sl_van_tok[done]).mean()), 4)
    out["sliding_window_32"] = {"entropycache_tau_1": sl_ec, "vanilla": sl_van,
                                "speedup_vs_vanilla": round(sl_ec["steps_per_s"] / sl_van["steps_per_s"], 3)}
    _log(f"sliding window: {out['sliding_window_32']}")

    # block diffusion: block-causal attention over blocks of 32 (the prompt's
    # 16 blocks committed first, untimed), the entropy gate inside the current
    # block, each finished block committed after its last step.  Timed: the
    # 352 denoising steps and the 16 commits of the generated blocks.
    def block_diffusion(t):
        reset()
        for b0 in range(0, cfg.prompt_len, cfg.block_len):
            ds.commit(cfg.k, b0, cfg.block_len)
        torch.cuda.synchronize()
        fl2 = torch.zeros(len(sched), dtype=torch.int32, device="cuda")
        t1 = time.perf_counter()
        for i, (bs, bl, nn) in enumerate(sched):
            fl2[i].copy_(ds.full_flag[0])
            ds.step(t, cfg.k, bs, bl, nn, block_causal=True)
            if i + 1 == len(sched) or sched[i + 1][0] != bs:
                ds.commit(cfg.k, bs, bl)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t1
        return ({"steps_per_s": round(len(sched) / dt, 2),
                 "partial_fraction": round(float(1.0 - fl2.float().mean().item()), 3)},
                ds.tokens.cpu().numpy())

    bd_van, bd_van_tok = block_diffusion(float("-inf"))
    bd_ec, bd_tok = block_diffusion(tau)
    bd_ec["token_agreement_vs_vanilla"] = round(float((bd_tok[gen] == bd_van_tok[gen]).mean()), 4)
    out["block_diffusion_32"] = {
        "entropycache_tau_1": bd_ec, "vanilla": bd_van,
        "speedup_vs_vanilla": round(bd_ec["steps_per_s"] / bd_van["steps_per_s"], 3),
        "note": "block-causal attention; full step = the current block's 32 rows; "
                "steps/s counts denoising steps, the time includes the 16 block commits"}
    _log(f"block diffusion: {out['block_diffusion_32']}")

    # KV drift on full steps (untimed): the E that triggered each full step
    # next to the Value drift that step measured
    reset()
    ds.enable_drift()
    pairs = []
    e_prev = None
    for bs, bl, nn in sched:
        full = int(ds.full_flag.item())
        ds.step(tau, cfg.k, bs, bl, nn)
        if full and e_prev is not None:
            dm_, dx_ = ds.kv_drift[0].tolist()
            pairs.append((e_prev, dm_, dx_))
        e_prev = float(ds.e_max.item())
    ds.struct.kv_drift = None
    if pairs:
        a = np.array(pairs)
        r = float(np.corrcoef(a[:, 0], a[:, 1])[0, 1]) if len(a) > 2 else float("nan")
        out["kv_drift_tau_1"] = {
            "full_steps": len(pairs), "drift_mean": round(float(a[:, 1].mean()), 5),
            "drift_max": round(float(a[:, 2].max()), 5), "corr_trigger_E_vs_mean_drift": round(r, 4),
            "note": "1 - cos of stale vs recomputed Value vectors per position (layer 0); "
                    "synthetic weights, so the correlation is not the pages' observation"}
        _log(f"kv drift: {out['kv_drift_tau_1']}")
    if cpu_baseline:
        out["cpu_baseline"] = step_cpu_baseline(cfg, w, toks, masked, sched, tau)
    return out


def step_cpu_baseline(cfg, w, toks, masked, sched, tau) -> dict:
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    model = O.Model.from_arrays(cfg.model, cfg.dtype, w)
    st = O.init_state(model, toks, masked)
    n, n_full, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < 20.0 and n < len(sched):
        bs, bl, nn = sched[n]
        n_full += st.flag
        O.step(model, st, tau, cfg.k, bs, bl, nn, keep_logits=False)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 4), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} steps of the tau=1.0 trajectory ({n_full} full, {n - n_full} partial), "
                      f"NumPy float64, {dt:.1f} s"}


# --------------------------------------------------------------------------- long context
def long_context_leg(cfg, tok_table, steps: int = 64, warmup: int = 8, cpu_baseline: bool = True) -> dict:
    """Steady-state long-context step (Dream-shaped layer, no LM head): a
    prefill (full step), `warmup` untimed steps, then `steps` timed steps.
    Step t decides from two synthetic decoded rows, flat when t % 8 == 7, so
    every step after such a step is full (all L rows) and the others recompute
    the fixed 96 rows.  Per-step kernel time comes from events around each
    step; attention, QKV and O-projection times from a separate pass with the
    phase events of ec_step."""
    import numpy as np
    import torch

    from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence, to_device
    from synth import generators as G

    m = cfg.model
    _log(f"{cfg.name}: generating weights")
    w = G.model_weights(cfg, tok_table=tok_table)
    toks, masked = G.initial_sequence(cfg)
    hist = [int(p) for p in G.long_context_history(cfg)]
    dm = DeviceModel(m, cfg.dtype, cfg.L, w)
    ds = DeviceSequence(dm, toks, masked, history_cap=cfg.k, max_block=cfg.block_len)
    ds.load_state(toks, masked, hist, 1)
    n_total = 1 + warmup + steps + 2 * cfg.full_every
    dec = torch.stack([to_device(G.decision_logits(cfg, t), cfg.dtype) for t in range(n_total)])
    stream = torch.cuda.current_stream()

    def one(t, ev=None):
        ds.step_external(cfg.tau, cfg.k, cfg.prefix_len, cfg.block_len, dec[t], phase_events=ev)

    def is_full(t):
        return t == 0 or (t - 1) % cfg.full_every == cfg.full_every - 1

    for t in range(0, 1 + warmup):
        one(t)
    torch.cuda.synchronize()
    t_lo = 1 + warmup
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    flags = torch.zeros(steps, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        flags[i].copy_(ds.full_flag[0])
        ev[i][0].record(stream)
        one(t_lo + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fl = flags.cpu().numpy()
    want = np.array([int(is_full(t_lo + i)) for i in range(steps)])
    if not np.array_equal(fl, want):
        raise RuntimeError(f"{cfg.name}: unexpected step modes {fl.tolist()}")
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    part_ms, full_ms = float(ms[fl == 0].mean()), float(ms[fl == 1].mean())

    # phase breakdown: one partial and one full step, each repeated
    n_ev = 2 * len(PHASES)

    def phase_pass(t_first, count):
        sets = []
        for i in range(count):
            evs = []
            for _ in range(n_ev):
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                evs.append(e)
            sets.append(evs)
        torch.cuda.synchronize()
        out = {}
        for i in range(count):
            one(t_first + i, sets[i])
        torch.cuda.synchronize()
        for k, name in enumerate(PHASES):
            out[name] = float(np.mean([e[2 * k].elapsed_time(e[2 * k + 1]) for e in sets]))
        return out

    t_next = t_lo + steps
    # t_next is a multiple of 8 plus 1 + warmup: find the next partial and full steps
    tp = next(t for t in range(t_next, n_total) if not is_full(t))
    for t in range(t_next, tp):
        one(t)
    ph_part = phase_pass(tp, 4)
    tf = next(t for t in range(tp + 4, n_total) if is_full(t))
    for t in range(tp + 4, tf):
        one(t)
    ph_full = phase_pass(tf, 1)
    n_part, L = cfg.block_len + cfg.k, cfg.L
    Hq, Hkv, dh = m.n_q_heads, m.n_kv_heads, m.head_dim

    def attn(rows, t_ms):
        flops = 4.0 * rows * L * Hq * dh
        tf_s = flops / (t_ms * 1e-3) / 1e12
        return {"us": round(t_ms * 1e3, 2), "gflop": round(flops / 1e9, 2),
                "tflops": round(tf_s, 1), "mfma_frac": round(tf_s / BF16_PEAK_TFLOPS, 4),
                "kv_bytes": 2 * Hkv * L * dh * 2}

    out = {
        "L": L, "steps_per_s": round(steps / wall, 2), "ms_per_step": round(wall * 1e3 / steps, 4),
        "partial_step_us": round(part_ms * 1e3, 2), "full_step_us": round(full_ms * 1e3, 2),
        "n_partial": int((fl == 0).sum()), "n_full": int((fl == 1).sum()),
        "partial_phases_us": {k: round(v * 1e3, 2) for k, v in ph_part.items()
                              if k not in ("ffn", "lmhead")},
        "full_phases_us": {k: round(v * 1e3, 2) for k, v in ph_full.items()
                           if k not in ("ffn", "lmhead")},
        "attention_partial": attn(n_part, ph_part["attn"]),
        "attention_full": attn(L, ph_full["attn"]),
    }
    _log(f"{cfg.name}: {out['steps_per_s']} steps/s; partial {out['partial_step_us']} us, "
         f"full {out['full_step_us']} us; attention partial {out['attention_partial']}, "
         f"full {out['attention_full']}")
    if cpu_baseline:
        out["cpu_baseline"] = long_context_cpu_baseline(cfg, w, toks, masked, hist)
    del ds, dm, dec
    torch.cuda.empty_cache()
    return out


def long_context_cpu_baseline(cfg, w, toks, masked, hist, budget_s: float = 15.0) -> dict:
    """The oracle's partial steady-state steps (96 rows against a seeded cache)."""
    import numpy as np

    import oracle as O
    from synth import generators as G
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    model = O.Model.from_arrays(cfg.model, cfg.dtype, w)
    st = O.init_state(model, toks, masked)
    m = cfg.model
    st.K = [G.random_matrix(cfg.seed, (21,), (m.n_kv_heads, cfg.L, m.head_dim), 1.0, cfg.dtype).astype(np.float64)]
    st.V = [G.random_matrix(cfg.seed, (22,), (m.n_kv_heads, cfg.L, m.head_dim), 1.0, cfg.dtype).astype(np.float64)]
    st.history, st.flag = list(hist), 0
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and n < 8:
        z = G.decision_logits(cfg, 1 + n)               # peaked rows: every step stays partial
        O.step_external(model, st, cfg.tau, cfg.k, cfg.prefix_len, cfg.block_len, z)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 4), "unit": "partial steps/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} partial steps (96 rows, L = {cfg.L}) from a seeded cache, NumPy float64, {dt:.1f} s"}


# --------------------------------------------------------------------------- 32-layer stack
def stack_leg(n_steps: int = 66) -> dict:
    """End-to-end denoise steps/s of the 32-layer LLaDA-shaped stack (RMSNorm,
    MHA 32 x 128, SwiGLU 12288, L = 2048 = 1792 + 256 in blocks of 32, k = 64,
    V = 126464) over the first `n_steps` steps of the schedule at tau = 1.0,
    and the same steps with tau = -inf (vanilla: every step full).  Weights
    are generated and uploaded one layer at a time."""
    import numpy as np
    import torch

    from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence
    from synth import configs as C
    from synth import generators as G

    cfg = C.LLADA_STACK
    m = cfg.model
    t_gen = time.perf_counter()

    _log(f"{cfg.name}: generating and uploading weights layer by layer")
    w = G.model_weights_streamed(cfg)
    dm = DeviceModel(m, cfg.dtype, cfg.L, w)
    del w
    _log(f"{cfg.name}: weights in HBM after {time.perf_counter() - t_gen:.1f} s")
    toks, masked = G.initial_sequence(cfg)
    ds = DeviceSequence(dm, toks, masked, history_cap=cfg.gen_len, max_block=cfg.block_len,
                        keep_logits=False)   # as in the step leg: statistics in place of logits
    sched = C.unmask_schedule(cfg)[:n_steps]
    init = (ds.tokens.clone(), ds.is_masked.clone())

    def reset():
        ds.tokens.copy_(init[0])
        ds.is_masked.copy_(init[1])
        ds.history_len.zero_()
        ds.full_flag.fill_(1)

    def run(tau, flags=None, events=None):
        for i, (bs, bl, nn) in enumerate(sched):
            if flags is not None:
                flags[i].copy_(ds.full_flag[0])
            if events is not None:
                events[i][0].record()
            ds.step(tau, cfg.k, bs, bl, nn)
            if events is not None:
                events[i][1].record()

    def run_host_mode(tau):
        # the host reads each step's mode (a 4-byte copy that waits for the
        # previous step) and launches only that mode's kernels
        return [ds.step_host_mode(tau, cfg.k, bs, bl, nn) for bs, bl, nn in sched]

    reset()
    for bs, bl, nn in sched[:3]:                 # warm-up (one full, two partial steps)
        ds.step(1.0, cfg.k, bs, bl, nn)
    out = {"workload": "llada8b_stack32_L2048 (32 layers, d 4096, 32x128, SwiGLU 12288, V 126464, "
                       "k 64, tau 1.0)", "steps": len(sched)}
    for tau, key in ((1.0, "entropycache"), (float("-inf"), "vanilla")):
        reset()
        flags = torch.zeros(len(sched), dtype=torch.int32, device="cuda")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sched]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(tau, flags, ev)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        fl = flags.cpu().numpy()
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        rec = {"steps_per_s": round(len(sched) / wall, 3), "ms_per_step": round(wall * 1e3 / len(sched), 3),
               "partial_fraction": round(float(1.0 - fl.mean()), 3)}
        if (fl == 1).any():
            rec["full_step_ms"] = round(float(ms[fl == 1].mean()), 3)
        if (fl == 0).any():
            rec["partial_step_ms"] = round(float(ms[fl == 0].mean()), 3)
        out[key] = rec
        _log(f"{cfg.name} tau={tau}: {rec}")
    out["speedup_vs_vanilla"] = round(out["entropycache"]["steps_per_s"] / out["vanilla"]["steps_per_s"], 3)
    reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    modes = run_host_mode(1.0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out["entropycache_host_mode"] = {
        "steps_per_s": round(len(sched) / wall, 3), "ms_per_step": round(wall * 1e3 / len(sched), 3),
        "partial_fraction": round(1.0 - float(np.mean(modes)), 3),
        "note": "mode read by the host before each step; only that mode's kernels launched"}
    _log(f"{cfg.name} host-read mode: {out['entropycache_host_mode']}")
    # the per-step roofline: the sum of every kernel's ideal (HBM bytes at 8 TB/s
    # on partial steps, bf16 MFMA flops at 2.5 PFLOP/s on full steps)
    d, hd, ff, L_ = m.d, m.n_q_heads * m.head_dim, m.d_ffn, cfg.L
    nqkv = (m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim
    layer_w = (nqkv * d + hd * d + 3 * ff * d) * 2
    kv = 2 * m.n_kv_heads * L_ * m.head_dim * 2
    lm_w = m.vocab * d * 2
    part_ms = (m.n_layers * (layer_w + kv) + lm_w) / (HBM_PEAK_GBS * 1e6)
    full_fl = m.n_layers * (2.0 * L_ * d * (nqkv + hd + 3 * ff) + 4.0 * L_ * L_ * hd)
    full_ms = full_fl / (BF16_PEAK_TFLOPS * 1e9) + lm_w / (HBM_PEAK_GBS * 1e6)
    ec = out["entropycache"]
    out["roofline"] = {"partial_step_ideal_ms": round(part_ms, 3), "full_step_ideal_ms": round(full_ms, 3),
                       "partial_frac": round(part_ms / ec["partial_step_ms"], 3) if "partial_step_ms" in ec else None,
                       "full_frac": round(full_ms / ec["full_step_ms"], 3) if "full_step_ms" in ec else None}
    _log(f"{cfg.name} roofline: {out['roofline']}")
    del ds, dm
    torch.cuda.empty_cache()
    return out


def stack_cpu_baseline(budget_s: float = 20.0) -> dict:
    """The float64 oracle on a bounded sample of the 32-layer stack: one layer's
    partial step (96 selected rows against an L = 2048 cache; the vocabulary,
    which a layer does not touch beyond one embedding row per token, cut to
    1024) and the LM head over the block's 32 rows on 1/16 of W_lm.  The step
    time is extrapolated as 32 x layer + 16 x head slice (labelled so)."""
    import numpy as np

    import oracle as O
    from synth import configs as C
    from synth import generators as G

    cfg = C.scaled(C.LLADA_STACK, name="stack_one_layer", model_n_layers=1, model_vocab=1024)
    w = G.model_weights(cfg)
    model = O.Model.from_arrays(cfg.model, cfg.dtype, w)
    toks, masked = G.initial_sequence(cfg)
    st = O.init_state(model, toks, masked)       # empty cache: the timing does not depend on it
    rows = np.arange(cfg.prompt_len - cfg.k, cfg.prompt_len + cfg.block_len)   # 96 rows
    n, t_layer = 0, 0.0
    t0 = time.perf_counter()
    while n < 3 and (n == 0 or time.perf_counter() - t0 < budget_s):
        t1 = time.perf_counter()
        x = O.forward_rows(model, st, rows)
        t_layer += time.perf_counter() - t1
        n += 1
    V, d = C.LLADA_STACK.model.vocab, cfg.model.d
    w_slice = np.random.default_rng(0).standard_normal((V // 16, d))
    t1 = time.perf_counter()
    O.linear(x[-cfg.block_len:], w_slice)
    t_head = 16 * (time.perf_counter() - t1)
    step_s = C.LLADA_STACK.model.n_layers * t_layer / n + t_head
    return {"value": round(1.0 / step_s, 4), "unit": "partial steps/s (extrapolated)",
            "cores": _cpu_cores(), "kind": "oracle",
            "sample": f"one layer's partial step (96 rows, L = {cfg.L}) x {n} and the LM head over "
                      f"{cfg.block_len} rows on 1/16 of W_lm, NumPy float64; step = 32 x layer + "
                      f"16 x head slice"}


# --------------------------------------------------------------------------- profiling
def profile_mfma_mode(workload: str) -> int:
    """A short, fixed sequence of one workload's kernels for counter runs:
      dream8k  the Dream-shaped layer at L = 8224 in steady state: a prefill,
               seven partial steps and the full step after a flat decision;
      dream32k the same at L = 32800;
      llada    one block (22 steps) of the LLaDA-shaped layer;
      stack    three steps of the 32-layer stack (one full, two partial),
               each launching only its mode's kernels."""
    import torch

    from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence, to_device
    from synth import configs as C
    from synth import generators as G

    if workload in ("dream8k", "dream32k"):
        cfg = C.DREAM_8K if workload == "dream8k" else C.DREAM_32K
        w = G.model_weights(cfg)
        toks, masked = G.initial_sequence(cfg)
        dm = DeviceModel(cfg.model, cfg.dtype, cfg.L, w)
        ds = DeviceSequence(dm, toks, masked, history_cap=cfg.k, max_block=cfg.block_len)
        ds.load_state(toks, masked, [int(p) for p in G.long_context_history(cfg)], 1)
        for t in range(9):               # t = 0 full (prefill), 1..7 partial, 8 full
            ds.step_external(cfg.tau, cfg.k, cfg.prefix_len, cfg.block_len,
                             to_device(G.decision_logits(cfg, t), cfg.dtype))
    elif workload == "llada":
        sc = C.LLADA_LAYER
        w = G.model_weights(sc)
        toks, masked = G.initial_sequence(sc)
        dm = DeviceModel(sc.model, sc.dtype, sc.L, w)
        ds = DeviceSequence(dm, toks, masked, history_cap=sc.gen_len, max_block=sc.block_len,
                            keep_logits=False)
        for bs, bl, nn in C.unmask_schedule(sc)[:22]:
            ds.step(1.0, sc.k, bs, bl, nn)
    elif workload == "stack":
        sc = C.LLADA_STACK
        dm = DeviceModel(sc.model, sc.dtype, sc.L, G.model_weights_streamed(sc))
        toks, masked = G.initial_sequence(sc)
        ds = DeviceSequence(dm, toks, masked, history_cap=sc.gen_len, max_block=sc.block_len,
                            keep_logits=False)
        for bs, bl, nn in C.unmask_schedule(sc)[:3]:
            ds.step(1.0, sc.k, bs, bl, nn, mode=L_mode(ds))
    else:
        raise SystemExit(f"unknown workload {workload}")
    torch.cuda.synchronize()
    _log(f"{workload} steps done")
    return 0


def L_mode(ds) -> int:
    """The step mode read from the flag (only that mode's kernels launch)."""
    from entropy_gated_kv_amd import lib as L
    return L.EC_MODE_FULL if int(ds.full_flag.item()) else L.EC_MODE_PARTIAL


def profile_mode() -> int:
    """A short, fixed sequence for hardware-counter runs (rocprofv3 --pmc):
    a 1 GiB device copy (the calibration of FETCH_SIZE / WRITE_SIZE), five
    entropy passes over the 4096 x 126464 logits, and one block (22 steps) of
    the LLaDA-shaped EntropyCache loop as the benchmark runs it (no logits
    buffer)."""
    import torch

    from entropy_gated_kv_amd import lib as L
    from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence
    from synth import configs as C
    from synth import generators as G

    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    _log("calibration copies done (1 GiB each)")
    cfg = C.ENTROPY_ONLY
    x = torch.from_numpy(G.entropy_logits(cfg)).to(torch.bfloat16).cuda()
    n, V = x.shape
    H = torch.empty(n, device="cuda")
    E = torch.empty(1, device="cuda")
    F = torch.empty(1, device="cuda", dtype=torch.int32)
    ws = torch.zeros(L.ec_entropy_workspace_bytes(n, V), device="cuda", dtype=torch.uint8)
    for _ in range(5):
        L.ec_entropy_max(x, cfg.tau, H, E, F, ws)
    torch.cuda.synchronize()
    del x
    _log("entropy passes done")
    sc = C.LLADA_LAYER
    w = G.model_weights(sc)
    toks, masked = G.initial_sequence(sc)
    dm = DeviceModel(sc.model, sc.dtype, sc.L, w)
    ds = DeviceSequence(dm, toks, masked, history_cap=sc.gen_len, max_block=sc.block_len,
                        keep_logits=False)
    for bs, bl, nn in C.unmask_schedule(sc)[:22]:
        ds.step(1.0, sc.k, bs, bl, nn)
    torch.cuda.synchronize()
    _log("22 steps done")
    return 0


# --------------------------------------------------------------------------- main
def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=352)
    ap.add_argument("--warmup", type=int, default=22)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-entropy", action="store_true")
    ap.add_argument("--skip-long", action="store_true", help="skip the long-context legs")
    ap.add_argument("--skip-stack", action="store_true", help="skip the 32-layer stack leg")
    ap.add_argument("--skip-step", action="store_true",
                    help="skip the step leg (diagnostics only: no headline value)")
    ap.add_argument("--profile-mode", action="store_true",
                    help="run the fixed short sequence used for hardware-counter runs")
    ap.add_argument("--profile-mfma", choices=("dream8k", "dream32k", "llada", "stack"),
                    help="run one workload's fixed short sequence, for counter runs")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown table of a rocprofv3 --kernel-trace run and exit")
    ap.add_argument("--min-us", type=float, default=3.0,
                    help="with --summarize-trace: calls at most this long count as gated exits")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="print a markdown table of rocprofv3 --pmc runs (CSV directories)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two counter runs of --profile-mode")
    args = ap.parse_args()
    if args.record_traffic:
        print(json.dumps(record_traffic(*args.record_traffic), indent=1))
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return 0
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.min_us))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the design notes describe how the step would shard)", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.profile_mode:
        return profile_mode()
    if args.profile_mfma:
        return profile_mfma_mode(args.profile_mfma)
    if args.skip_step:
        line = {"metric": METRIC, "value": None, "unit": "steps/s", "n_gpus": 1,
                "note": "diagnostic run without the step leg (no headline value)"}
    else:
        res = step_leg(args.steps, args.warmup, not args.no_cpu_baseline)
        line = {
            "metric": METRIC,
            "value": round(res["value"], 2),
            "unit": "steps/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(res["ms_per_step"], 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "llada8b_layer_L1024_tau1.0", "L": 1024, "prompt": 512, "gen": 512,
                       "block": 32, "d_model": 4096, "heads": "32x128", "vocab": 126464, "k": 64,
                       "tau": 1.0, "layers": 1},
            "roofline": res["roofline"],
            "partial_fraction": round(res["partial_fraction"], 3),
            "phases_us": res["phases_us"],
            "phase_event_overhead_us": res["phase_event_overhead_us"],
            "decision_overhead_frac": round(res["decision_overhead_frac"], 4),
            "phase_roofline": res["phase_roofline"],
            "tau_sweep": res["tau_sweep"],
            "speedup_vs_vanilla_at_tau_1": res["speedup_vs_vanilla_at_tau_1"],
            "k_ablation_tau_1": res["k_ablation_tau_1"],
            "kv_drift_tau_1": res.get("kv_drift_tau_1"),
            "sliding_window_32": res.get("sliding_window_32"),
            "block_diffusion_32": res.get("block_diffusion_32"),
            "lm_head_output": "softmax statistics per group of column tiles (no logits buffer)",
            "with_logits": res.get("with_logits"),
        }
        if "cpu_baseline" in res:
            line["cpu_baseline"] = res["cpu_baseline"]
    if not args.skip_stack:
        line["stack32"] = stack_leg()
        if not args.no_cpu_baseline:
            line["stack32"]["cpu_baseline"] = stack_cpu_baseline()
    if not args.skip_long:
        from synth import configs as C
        from synth import generators as G
        _log("generating the Dream-shaped token table")
        tok = G.tok_emb(C.DREAM_8K)
        line["long_context"] = {
            "workload": "dream7b_layer_steady_state (d 3584, 28/4 x 128, V 152064, 96 rows, full every 8th)",
            "L8224": long_context_leg(C.DREAM_8K, tok, cpu_baseline=not args.no_cpu_baseline),
            "L32800": long_context_leg(C.DREAM_32K, tok, cpu_baseline=False),
        }
        del tok
    if not args.skip_entropy:
        ent = entropy_leg(200, 30, not args.no_cpu_baseline)   # ~40 ms timed, clocks settled
        line["entropy_pass"] = {"GB_per_s": round(ent["GB_per_s"], 1), "us_per_pass": round(ent["kernel_ms"] * 1e3, 2), "rows_per_s": round(ent["rows_per_s"], 1),
                                "roofline": ent["roofline"], "workload": "entropy_4096x126464_bf16",
                                "cpu_baseline": ent.get("cpu_baseline")}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
