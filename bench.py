"""Benchmark of the hot path: token scoring (sp_score) + chunk selection
(sp_select) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
               [--copy-probe-mib MIB] [--cooperative] [--select workload|threshold]
               [--window W [--stride S]]

--workload takes any workload of synth (default: the 8B shape at M = 32K); the
ragged batch is timed through sp_score_varlen + sp_select_varlen.
--select threshold times the threshold selection (SP_SELECT_THRESHOLD, the
Implementation Guide program's chunk selection with its 128-token fill and
2000-token cap) instead of the workload's selection.
--window W [--stride S] scores the workload's prompt in sliding windows
(sp_window_layout, sp_score_windows; stride W/2 by default), each window with
its own synthetic queries and keys.
--cooperative launches the scoring kernel cooperatively (SP_LAUNCH_COOPERATIVE)
instead of with the default ordinary launch.

A step scores one prompt of the workload (inputs already resident in HBM) and
selects its tokens. W untimed steps, then exactly K timed steps between device
synchronisations; prints one JSON line. Throughput = prompt tokens per second.
Several copies of K are rotated so that no step finds its keys in the 256 MB
Infinity Cache left over from the previous one.

The roofline block reports the dominant kernel's algorithmic bytes (one read
of K and Q) over its average duration. The library records HIP events on the
scoring stream immediately before and after each launch of its scoring
kernel (sp_profile_score_kernel), so the duration excludes the small prep
kernel (the scoring kernel itself ends by writing the importance). A pair of
timing events costs a step about 6 us of device time, so they bracket the
scoring kernel of every KERNEL_EVENT_EVERY-th timed step only (all steps run
the same shape); the per-call breakdown in "detail" (sp_score including its
prep, selection and gaps) comes from a short evented pass after the timed
region.
HBM traffic comes from the rocprofv3 counter summary under profiles/ when it
was taken on the code of the current kernel sources (else null); `--traffic-from FETCH_DB WRITE_DB` writes that summary from two
rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE) that
included `--copy-probe-mib` (the copy calibrates the counters' units). The CPU
baseline times the oracle on the host cores on a bounded sample (a subset of
layers, scaled to the full workload).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "prompt tokens scored/s (sp_score+select) at 8B shape M=32K; % HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="spec8b_m32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--select", choices=("workload", "threshold"), default="workload",
                    help="the workload's selection, or the Implementation Guide program's "
                         "threshold selection (min_tok 128, max_keep 2000)")
    ap.add_argument("--window", type=int, default=0,
                    help="score the prompt in sliding windows of this many tokens")
    ap.add_argument("--stride", type=int, default=0,
                    help="window stride (default: half the window)")
    ap.add_argument("--cooperative", action="store_true",
                    help="launch the scoring kernel cooperatively (SP_LAUNCH_COOPERATIVE)")
    ap.add_argument("--cpu-layers", type=int, default=1 << 30,
                    help="layers of the workload the CPU baseline scores (default: all)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write the traffic summary from two rocprofv3 --pmc databases and exit")
    args = ap.parse_args()
    if args.window and not args.stride:
        args.stride = max(1, args.window // 2)
    return args


SCORE_KERNEL = "sp::score_kernel<"
# the calibration probe is the run's only elementwise add
PROBE_KERNEL_HINTS = ("elementwise", "add")


def _code_only(text: str) -> str:
    """C/C++ source without // comments and blank lines (a comment edit does
    not change the code the counters were taken on)."""
    out = []
    for line in text.splitlines():
        i = line.find("//")
        if i >= 0 and line.count('"', 0, i) % 2 == 0:
            line = line[:i]
        line = line.rstrip()
        if line:
            out.append(line)
    return "\n".join(out)


def kernel_source_sha() -> str:
    """Fingerprint of the code of every source the scoring kernels and their
    plan come from (sp_score*: the kernels, their launch and the planner)."""
    csrc = os.path.join(ROOT, "attention_token_scoring_amd", "csrc")
    names = sorted(n for n in os.listdir(csrc)
                   if n.startswith("sp_score") or n == "sp_internal.h")
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def pmc_per_dispatch(db_path: str, counter: str):
    """[(kernel name, counter value summed over the dispatch's instances)] in
    dispatch order, from a rocprofv3 database."""
    import sqlite3
    con = sqlite3.connect(db_path)
    cur = con.cursor()
    rows = cur.execute(
        "select kernel_name, sum(value) from counters_collection where counter_name = ? "
        "group by dispatch_id order by dispatch_id", (counter,)).fetchall()
    return [(r[0], float(r[1])) for r in rows]


def write_traffic(fetch_db: str, write_db: str, workload: str, copy_mib: int):
    """HBM bytes per scoring-kernel launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the copy probe
    (copy_mib MiB read and written)."""
    out = {"workload": workload, "source_sha": kernel_source_sha(), "copy_probe_mib": copy_mib}
    for key, db, counter in (("fetch", fetch_db, "FETCH_SIZE"), ("write", write_db, "WRITE_SIZE")):
        rows = pmc_per_dispatch(db, counter)
        score = [v for n, v in rows if SCORE_KERNEL in n]
        probes = [v for n, v in rows if all(h in n.lower() for h in PROBE_KERNEL_HINTS)]
        if not score or len(probes) != 1:
            raise SystemExit(f"{db}: no {counter} for the scoring kernel, or not exactly one probe")
        copy_kib = probes[0]
        factor = (copy_mib * 1024.0) / copy_kib
        out[key] = {"counter": counter, "score_kib_per_dispatch": float(np.mean(score)),
                    "dispatches": len(score), "copy_probe_kib": copy_kib, "scale": factor,
                    "bytes_per_launch": float(np.mean(score)) * 1024.0 * factor}
    out["bytes_per_launch"] = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def load_traffic(workload: str):
    """Counter-measured HBM bytes per launch of the scoring kernel, if the
    summary matches the current kernel source and workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != kernel_source_sha() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


THRESHOLD_MIN_TOK, THRESHOLD_MAX_KEEP = 128, 2000
KERNEL_EVENT_EVERY = 4


def select_params(sp, sel):
    extra = dict(min_tok=THRESHOLD_MIN_TOK, max_keep=THRESHOLD_MAX_KEEP) \
        if sel.mode == "threshold" else {}
    return sp.select_params(chunk=sel.chunk, pool_k=sel.pool_k, mode=sel.mode,
                            keep_rate=sel.keep_rate, mass=sel.mass,
                            boost_first_n=sel.boost_first_n,
                            boost_first_mult=sel.boost_first_mult,
                            boost_last_n=sel.boost_last_n, boost_last_mult=sel.boost_last_mult,
                            **extra)


def workload_desc(w, sel) -> dict:
    d = {"workload": f"{w.name}: L={w.L} H={w.H} Hkv={w.Hkv} d={w.d} M={w.M} N={w.N} "
                     f"{'bf16' if w.dtype else 'f32'}; select {sel.mode} "
                     f"{sel.mass if sel.mode == 'mass' else sel.keep_rate} chunk {sel.chunk} "
                     f"pool {sel.pool_k}",
         "L": w.L, "H": w.H, "Hkv": w.Hkv, "d": w.d, "M": w.M, "N": w.N,
         "select": sel.mode, "chunk": sel.chunk, "pool_k": sel.pool_k}
    if sel.mode == "mass":
        d["mass"] = sel.mass
    else:
        d["keep_rate"] = sel.keep_rate
    if sel.mode == "threshold":
        d["min_tok"], d["max_keep"] = THRESHOLD_MIN_TOK, THRESHOLD_MAX_KEEP
    if sel.boost_first_n or sel.boost_last_n:
        d["boosts"] = [sel.boost_first_n, sel.boost_first_mult, sel.boost_last_n,
                       sel.boost_last_mult]
    return d


def cpu_baseline(w, sel, Qh, Kh, layers: int, min_seconds: float = 10.0):
    """The oracle as it is, on the host cores: score `layers` layers of the
    workload (all of them by default) and select on the result, repeated until
    about min_seconds of CPU work; the scoring time is scaled to all L layers
    (its cost is linear in L)."""
    import oracle
    threads = os.cpu_count() or 1
    layers = max(1, min(layers, w.L))
    t_score = t_sel = 0.0
    reps = 0
    while t_score + t_sel < min_seconds and reps < 100:
        t0 = time.perf_counter()
        imp = oracle.score(Qh[:layers], Kh[:layers], nthreads=threads)
        t1 = time.perf_counter()
        if sel.mode == "threshold":
            oracle.select_threshold(imp.astype(np.float32), sel.chunk, sel.keep_rate,
                                    min_tok=THRESHOLD_MIN_TOK, max_keep=THRESHOLD_MAX_KEEP)
        else:
            oracle.select(imp.astype(np.float32), **oracle.select_params(sel))
        t2 = time.perf_counter()
        t_score += t1 - t0
        t_sel += t2 - t1
        reps += 1
    t_full = (t_score * (w.L / layers) + t_sel) / reps
    return {"value": w.M / t_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: {reps} repetitions of oracle scoring of layers 0-{layers - 1} "
                      f"of {w.L} ({t_score:.1f} s in all"
                      + (f", scaled x{w.L / layers:g} to all layers" if layers < w.L else "")
                      + f") plus selection ({t_sel * 1e3:.1f} ms in all); fp64, OpenMP over "
                      f"{threads} threads"}


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args.traffic_from[0], args.traffic_from[1], args.workload,
                      args.copy_probe_mib or 1024)
        return
    if args.gpus != 1:
        print("bench.py: the scoring path runs on one GPU (no multi-GPU sharding); --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import attention_token_scoring_amd as sp
    import synth

    w = synth.WORKLOADS[args.workload]
    sel = w.selects[0]
    if args.select == "threshold":
        # the Implementation Guide program's selection at its defaults (keep
        # rate 0.3 unless the workload fixes one, 128-token fill, 2000-token cap)
        sel = dataclasses.replace(sel, mode="threshold", pool_k=1, keep_rate=sel.keep_rate or 0.3,
                                  mass=0.0, boost_first_n=0, boost_last_n=0)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.window:
        if w.R != 1:
            print("bench.py: --window takes a single-prompt workload", file=sys.stderr)
            sys.exit(2)
        windowed(args, w, sel, sp, torch, dev)
        return
    if w.R != 1:
        ragged(args, w, sel, sp, torch, dev)
        return

    Qh, Kh, M = synth.make_request(w)
    k_bytes = Kh.nbytes
    copies = max(2, math.ceil(512e6 / k_bytes) + 1)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    Q = to_dev(Qh)
    K0 = to_dev(Kh)
    Ks = [K0] + [K0.clone() for _ in range(copies - 1)]
    launch = sp.SP_LAUNCH_COOPERATIVE if args.cooperative else sp.SP_LAUNCH_RESIDENT
    desc = sp.score_desc(w.L, w.H, w.Hkv, w.d, w.N, sp.SP_BF16 if w.dtype else sp.SP_F32, 0.0, launch)
    ws = torch.empty(sp.sp_score_workspace_bytes(desc, M), dtype=torch.uint8, device=dev)
    imp = torch.empty(M, dtype=torch.float32, device=dev)
    kept = torch.empty(M, dtype=torch.int32, device=dev)
    pos = torch.empty(M, dtype=torch.int32, device=dev)
    nk = torch.empty(1, dtype=torch.int32, device=dev)
    params = select_params(sp, sel)
    plan = sp.sp_score_plan(desc, M)

    if args.copy_probe_mib:
        # counter calibration: one elementwise kernel that reads and writes
        # exactly copy_probe_mib MiB
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)  # contents do not matter
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.add(a, 1, out=b)
        torch.cuda.synchronize()
        del a, b

    def step(i, ev=None, kev=None):
        if kev is not None:
            sp.sp_profile_score_kernel(kev[0], kev[1])
        if ev is not None:
            ev[0].record()
        sp.sp_score(Q, Ks[i % copies], M, out=imp, workspace=ws, launch=launch)
        if ev is not None:
            ev[1].record()
        if kev is not None:
            sp.sp_profile_score_kernel()
        sp.sp_select(imp, params, kept_idx=kept, pos_ids=pos, n_kept=nk)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # events the library records around the scoring kernel of every
    # KERNEL_EVENT_EVERY-th timed step; torch creates an event on its first record
    kevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range((args.steps + KERNEL_EVENT_EVERY - 1) // KERNEL_EVENT_EVERY)]
    for a, b in kevs:
        a.record()
        b.record()
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_begin.record()
    host_s = 0.0  # host time spent issuing the steps (a step the host issues
    # more slowly than the device runs it is host-bound)
    for i in range(args.steps):
        h0 = time.perf_counter()
        step(i, None, kevs[i // KERNEL_EVENT_EVERY] if i % KERNEL_EVENT_EVERY == 0 else None)
        host_s += time.perf_counter() - h0
    t_end.record()
    torch.cuda.synchronize()
    w1 = time.perf_counter()

    ms_total_ev = t_begin.elapsed_time(t_end)
    ms_wall = (w1 - w0) * 1e3
    ms_per_step = ms_wall / args.steps
    # breakdown pass (outside the timed region): each sp_score call, prep included
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(min(args.steps, 50))]
    d_begin = torch.cuda.Event(enable_timing=True)
    d_end = torch.cuda.Event(enable_timing=True)
    d_begin.record()
    for i, ev in enumerate(evs):
        step(i, ev)
    d_end.record()
    torch.cuda.synchronize()
    score_ms = [a.elapsed_time(b) for a, b in evs]
    score_avg_s = float(np.mean(score_ms)) / 1e3
    diag_step_ms = d_begin.elapsed_time(d_end) / len(evs)
    kernel_ms = [a.elapsed_time(b) for a, b in kevs]
    kernel_avg_s = float(np.mean(kernel_ms)) / 1e3
    alg_bytes = (w.L * w.Hkv * (M + w.N) * w.d + w.L * w.H * w.N * w.d) * (2 if w.dtype else 4)
    achieved = alg_bytes / kernel_avg_s / 1e9
    traffic = load_traffic(w.name)

    out = {
        "metric": METRIC,
        "value": M / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype else "f32",
        "data": "synthetic",
        "config": dict(workload_desc(w, sel), launch=launch_name(args)),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "detail": {"score_kernel_ms_avg": kernel_avg_s * 1e3,
                   "score_kernel_ms_min": float(np.min(kernel_ms)),
                   "score_kernel_launches_timed": len(kevs),
                   "ms_per_step_events": ms_total_ev / args.steps,
                   "breakdown_pass": {"steps": len(evs), "ms_per_step": diag_step_ms,
                                      "sp_score_ms_avg": score_avg_s * 1e3,
                                      "sp_score_ms_min": float(np.min(score_ms)),
                                      "select_and_gaps_ms_avg": diag_step_ms - score_avg_s * 1e3},
                   "host_issue_ms_per_step": host_s * 1e3 / args.steps,
                   "alg_bytes_per_score_launch": alg_bytes, "k_copies": copies,
                   "plan": plan, "n_kept": int(nk.cpu()[0])},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, sel, Qh, Kh, args.cpu_layers)
    print(json.dumps(out), flush=True)


def launch_name(args) -> str:
    return "cooperative" if args.cooperative else "resident"


def windowed(args, w, sel, sp, torch, dev):
    """One prompt of the workload scored in sliding windows (each window with
    its own synthetic queries and keys, as a speculator run per window gives):
    one step is sp_score_windows + sp_select over the prompt's M tokens. The
    roofline figure uses the sp_score_windows call's duration (one scoring
    kernel per window plus its prep kernel)."""
    import synth

    starts, lens, keeps = sp.sp_window_layout(w.M, args.window, args.stride)
    ww = dataclasses.replace(w, R=len(lens), M=0, len_range=())
    Qh, Kh, cu = synth.make_ragged(ww, lens)
    R = len(lens)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    Q = to_dev(Qh)
    K = to_dev(Kh)
    del Qh, Kh
    launch = sp.SP_LAUNCH_COOPERATIVE if args.cooperative else sp.SP_LAUNCH_RESIDENT
    desc = sp.score_desc(w.L, w.H, w.Hkv, w.d, w.N, sp.SP_BF16 if w.dtype else sp.SP_F32, 0.0, launch)
    ws = torch.empty(sp.sp_score_workspace_bytes(desc, int(lens.max())), dtype=torch.uint8,
                     device=dev)
    imp = torch.empty(w.M, dtype=torch.float32, device=dev)
    kept = torch.empty(w.M, dtype=torch.int32, device=dev)
    pos = torch.empty(w.M, dtype=torch.int32, device=dev)
    nk = torch.empty(1, dtype=torch.int32, device=dev)
    params = select_params(sp, sel)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        sp.sp_score_windows(Q, K, cu, keeps, out=imp, workspace=ws, launch=launch)
        if ev is not None:
            ev[1].record()
        sp.sp_select(imp, params, kept_idx=kept, pos_ids=pos, n_kept=nk)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    w0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - w0) * 1e3 / args.steps
    score_s = float(np.mean([a.elapsed_time(b) for a, b in evs])) / 1e3
    alg_bytes = int(sum(w.L * w.Hkv * (int(m) + w.N) * w.d + w.L * w.H * w.N * w.d
                        for m in lens)) * (2 if w.dtype else 4)
    achieved = alg_bytes / score_s / 1e9
    out = {
        "metric": METRIC,
        "value": w.M / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype else "f32",
        "data": "synthetic",
        "config": dict(workload_desc(w, sel), launch=launch_name(args),
                       workload=f"{w.name} in sliding windows of {args.window} tokens, stride "
                                f"{args.stride}: {R} windows",
                       window=args.window, stride=args.stride),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "detail": {"sp_score_windows_ms_avg": score_s * 1e3, "alg_bytes_per_step": alg_bytes,
                   "windows": R, "n_kept": int(nk.cpu()[0])},
    }
    print(json.dumps(out), flush=True)


def ragged(args, w, sel, sp, torch, dev):
    """A batch of R prompts of different lengths: one step is sp_score_varlen
    + sp_select_varlen over the whole batch. The batch's keys (tens of GB) are
    far larger than the Infinity Cache, so one copy suffices. The roofline
    figure uses the sp_score_varlen call's duration (one scoring kernel per
    request plus its prep kernel), a lower bound for the kernels' rate."""
    import synth

    Qh, Kh, cu = synth.make_ragged(w)
    total = int(cu[-1])
    R = len(cu) - 1

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    Q = to_dev(Qh)
    K = to_dev(Kh)
    del Qh, Kh
    launch = sp.SP_LAUNCH_COOPERATIVE if args.cooperative else sp.SP_LAUNCH_RESIDENT
    desc = sp.score_desc(w.L, w.H, w.Hkv, w.d, w.N, sp.SP_BF16 if w.dtype else sp.SP_F32, 0.0, launch)
    maxM = int(np.max(np.diff(cu)))
    ws = torch.empty(sp.sp_score_workspace_bytes(desc, maxM), dtype=torch.uint8, device=dev)
    imp = torch.empty(total, dtype=torch.float32, device=dev)
    kept = torch.empty(total, dtype=torch.int32, device=dev)
    pos = torch.empty(total, dtype=torch.int32, device=dev)
    nk = torch.empty(R, dtype=torch.int32, device=dev)
    params = select_params(sp, sel)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        sp.sp_score_varlen(Q, K, cu, out=imp, workspace=ws, launch=launch)
        if ev is not None:
            ev[1].record()
        sp.sp_select_varlen(imp, cu, params, kept_idx=kept, pos_ids=pos, n_kept=nk)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    w0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - w0) * 1e3 / args.steps
    score_s = float(np.mean([a.elapsed_time(b) for a, b in evs])) / 1e3
    Ms = np.diff(cu)
    alg_bytes = int(sum(w.L * w.Hkv * (int(m) + w.N) * w.d + w.L * w.H * w.N * w.d for m in Ms)) * (2 if w.dtype else 4)
    achieved = alg_bytes / score_s / 1e9
    out = {
        "metric": METRIC,
        "value": total / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype else "f32",
        "data": "synthetic",
        "config": dict(workload_desc(w, sel), launch=launch_name(args), M=total, workload=f"{w.name}: R={R} prompts, M in "
                       f"[{int(Ms.min())}, {int(Ms.max())}], sum {total}; L={w.L} H={w.H} "
                       f"Hkv={w.Hkv} d={w.d} N={w.N}"),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "detail": {"sp_score_varlen_ms_avg": score_s * 1e3, "alg_bytes_per_step": alg_bytes,
                   "requests": R, "n_kept_total": int(nk.sum().cpu())},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
