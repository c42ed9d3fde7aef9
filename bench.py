"""Benchmark of the hot path: token scoring (sp_score) + chunk selection
(sp_select) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only]
               [--no-cpu-baseline] [--cooperative] [--select workload|threshold]
               [--window W [--stride S]] [--read-probe] [--copy-probe-mib MIB]

A step scores one prompt of the workload (inputs already resident in HBM) and
selects its tokens; the ragged batch is timed through sp_score_varlen +
sp_select_varlen. Throughput = prompt tokens per second. Several copies of K
are rotated so that no step finds its keys in the 256 MB Infinity Cache left
over from the previous one.

Per workload: a settle phase (steps for --settle-s seconds, 1 s by default:
after idle the device's power management needs ~15 ms of sustained load
before the scoring kernel runs at its steady speed, and after a heavy run of
other work in another process, such as the GPU test suite, ~0.3 s, during
which the 8B/32K scoring kernel measured 333 us instead of 324), then W
untimed warm-up steps, then exactly K timed steps between
device synchronisations (no timing events inside), then sp_score_status must
report a complete call. After the timed region a kernel pass of
--kernel-steps steps (>= 50) records HIP events the library places on the
scoring stream immediately before and after each launch of the scoring kernel
(sp_profile_score_kernel): the roofline block is the dominant kernel's
algorithmic bytes (one read of K and Q) over the mean of those durations (the
median is in `detail`). A breakdown pass brackets the sp_score call and the
selection.

The line's headline is the --workload (default: the 8B shape at M = 32K, run
with the driver's --steps/--warmup); unless --only is given, the other four
workloads follow with their own step counts and go into detail.workloads (each
with its throughput, its kernel-event roofline and the oracle timed on the host
cores on a bounded sample).

--select threshold times the threshold selection (the Implementation Guide
program's chunk selection with its 128-token fill and 2000-token cap).
--window W [--stride S] scores the workload's prompt in sliding windows.
--read-probe sweeps the plain streaming-read probe (sp_read_probe) over launch
shapes: the practical HBM read ceiling.
HBM traffic comes from the rocprofv3 counter summary under profiles/ when it
was taken on the current kernel sources (else null); `--traffic-from FETCH_DB
WRITE_DB` writes that summary from two rocprofv3 --pmc runs of this script
(FETCH_SIZE, then WRITE_SIZE) that included `--copy-probe-mib` (the copy
calibrates the counters' units).
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
ALL_WORKLOADS = ("spec8b_m32k", "tiny", "spec0.8b_m4608", "spec8b_m128k", "ragged16_8b")
# timed steps and warm-up steps of the workloads that follow the headline
OTHER_STEPS = {"tiny": (400, 20), "spec0.8b_m4608": (400, 20), "spec8b_m32k": (100, 10),
               "spec8b_m128k": (40, 5), "ragged16_8b": (10, 2)}
# seconds of oracle work each workload's CPU baseline aims at
CPU_SECONDS = {"tiny": 3.0, "spec0.8b_m4608": 5.0, "spec8b_m32k": 10.0, "spec8b_m128k": 6.0,
               "ragged16_8b": 6.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="spec8b_m32k")
    ap.add_argument("--only", action="store_true", help="time the --workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of steps before the warm-up (power management settles)")
    ap.add_argument("--kernel-steps", type=int, default=60,
                    help="steps of the evented kernel pass after the timed region (>= 50)")
    ap.add_argument("--select", choices=("workload", "threshold"), default="workload",
                    help="the workload's selection, or the Implementation Guide program's "
                         "threshold selection (min_tok 128, max_keep 2000)")
    ap.add_argument("--window", type=int, default=0,
                    help="score the prompt in sliding windows of this many tokens")
    ap.add_argument("--stride", type=int, default=0,
                    help="window stride (default: half the window)")
    ap.add_argument("--cooperative", action="store_true",
                    help="launch the scoring kernel cooperatively (SP_LAUNCH_COOPERATIVE)")
    ap.add_argument("--read-probe", action="store_true",
                    help="sweep the streaming-read probe over launch shapes and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write the traffic summary from two rocprofv3 --pmc databases and exit")
    args = ap.parse_args()
    if args.window and not args.stride:
        args.stride = max(1, args.window // 2)
    args.kernel_steps = max(50, args.kernel_steps)
    return args


# the scoring kernel's plain launch (sp_score); the fused launch
# (sp_score_select) is the instantiation with true in its second place, the
# launch of several requests (sp_score_varlen) the one that takes PackArgs
SCORE_KERNEL = "sp::score_kernel<"
SCORE_KERNEL_PLAIN = ", false, sp::ScoreArgs>(sp::ScoreArgs)"
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
        score = [v for n, v in rows if SCORE_KERNEL in n and SCORE_KERNEL_PLAIN in n]
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


def select_params(sp, sel):
    extra = dict(min_tok=THRESHOLD_MIN_TOK, max_keep=THRESHOLD_MAX_KEEP) \
        if sel.mode == "threshold" else {}
    return sp.select_params(chunk=sel.chunk, pool_k=sel.pool_k, mode=sel.mode,
                            keep_rate=sel.keep_rate, mass=sel.mass,
                            boost_first_n=sel.boost_first_n,
                            boost_first_mult=sel.boost_first_mult,
                            boost_last_n=sel.boost_last_n, boost_last_mult=sel.boost_last_mult,
                            **extra)


def sel_desc(sel) -> str:
    v = sel.mass if sel.mode == "mass" else sel.keep_rate
    return f"{sel.mode} {v}"


def workload_desc(w, sel) -> dict:
    d = {"workload": f"{w.name}: L={w.L} H={w.H} Hkv={w.Hkv} d={w.d} M={w.M} N={w.N} "
                     f"{'bf16' if w.dtype else 'f32'}; select {sel_desc(sel)} chunk {sel.chunk} "
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Threads the oracle may use: the CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def _oracle_select(oracle, imp, sel, base_index=0):
    if sel.mode == "threshold":
        return oracle.select_threshold(imp.astype(np.float32), sel.chunk, sel.keep_rate,
                                       min_tok=THRESHOLD_MIN_TOK, max_keep=THRESHOLD_MAX_KEEP)
    return oracle.select(imp.astype(np.float32), base_index=base_index,
                         **oracle.select_params(sel))


def cpu_baseline(w, sel, requests, min_seconds: float, threads: int | None = None,
                 max_layers: int | None = None):
    """The oracle as it is, on the host cores: score and select the given
    requests [(Q, K, M)] (a bounded sample of the workload), repeated until
    about min_seconds of CPU work or scoring only the first max_layers layers
    (the scoring cost is linear in the layer count, so the time is scaled to
    all L layers). Tokens/s = scored prompt tokens / the oracle's time."""
    import oracle
    threads = threads or host_threads()
    t_score = t_sel = 0.0
    reps = 0
    tokens = 0
    layers = w.L if max_layers is None else max(1, min(max_layers, w.L))
    while (t_score + t_sel < min_seconds or reps == 0) and reps < 1000:
        for Qh, Kh, M in requests:
            t0 = time.perf_counter()
            imp = oracle.score(Qh[:layers], Kh[:layers], nthreads=threads)
            t1 = time.perf_counter()
            _oracle_select(oracle, imp, sel)
            t2 = time.perf_counter()
            t_score += (t1 - t0) * (w.L / layers)
            t_sel += t2 - t1
            tokens += M
        reps += 1
    value = tokens / (t_score + t_sel)
    what = ", ".join(str(M) for _, _, M in requests[:4]) + (" ..." if len(requests) > 4 else "")
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{w.name}: {reps} repetition(s) of oracle scoring + selection of "
                      f"{len(requests)} prompt(s) (M = {what})"
                      + (f", scoring layers 0-{layers - 1} of {w.L} scaled x{w.L / layers:g}"
                         if layers < w.L else f", all {w.L} layers")
                      + f"; {t_score:.1f} s scoring (scaled), {t_sel * 1e3:.1f} ms selection; "
                        f"fp64, OpenMP over {threads} threads"}


def to_dev(torch, a, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def _events(torch, n):
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    return evs


def run_steps(torch, sp, step, steps: int, warmup: int, settle_s: float, kernel_steps: int,
              ws):
    """Settle, warm up, time exactly `steps` steps, check the scoring calls'
    status, then the evented kernel pass and the breakdown pass."""
    t0 = time.perf_counter()
    n_settle = 0
    while True:
        step(n_settle)
        n_settle += 1
        if n_settle % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= settle_s:
                break
    for i in range(warmup):
        step(i)
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_begin.record()
    for i in range(steps):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    w1 = time.perf_counter()
    if sp.sp_score_status(ws):
        raise SystemExit("bench.py: a scoring call's bounded waits timed out (scores invalid)")
    out = {"ms_per_step": (w1 - w0) * 1e3 / steps,
           "ms_per_step_events": t_begin.elapsed_time(t_end) / steps,
           "settle_steps": n_settle, "steps": steps, "warmup": warmup}
    # kernel pass: events around every scoring kernel launch
    kevs = _events(torch, kernel_steps)
    for a, b in kevs:  # (torch creates an event on its first record)
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i, ev in enumerate(kevs):
        step(i, kev=ev)
    torch.cuda.synchronize()
    kms = np.array([a.elapsed_time(b) for a, b in kevs])
    # breakdown pass: the sp_score call and the selection
    sev = _events(torch, 50)
    xev = _events(torch, 50)
    for i in range(50):
        step(i, sev=sev[i], xev=xev[i])
    torch.cuda.synchronize()
    if sp.sp_score_status(ws):
        raise SystemExit("bench.py: a scoring call's bounded waits timed out (scores invalid)")
    sms = np.array([a.elapsed_time(b) for a, b in sev])
    xms = np.array([a.elapsed_time(b) for a, b in xev])
    out.update(kernel_ms_mean=float(kms.mean()), kernel_ms_median=float(np.median(kms)),
               kernel_ms_min=float(kms.min()), kernel_launches=len(kms),
               sp_score_ms_mean=float(sms.mean()), select_ms_mean=float(xms.mean()))
    return out


def alg_bytes_of(w, Ms) -> int:
    """One read of K (prompt and look-ahead keys) and Q per request."""
    es = 2 if w.dtype else 4
    return int(sum(w.L * w.Hkv * (int(m) + w.N) * w.d + w.L * w.H * w.N * w.d for m in Ms)) * es


def roofline(alg_bytes, kernel_s, traffic):
    achieved = alg_bytes / kernel_s / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic}


def bench_single(args, w, sels, sp, torch, dev, steps, warmup, cpu_s):
    """One prompt per step (sp_score + sp_select); sels[0] is the workload's
    selection, any others are timed in steps of their own."""
    import synth

    Qh, Kh, M = synth.make_request(w)
    copies = max(2, math.ceil(512e6 / Kh.nbytes) + 1)
    Q = to_dev(torch, Qh, dev)
    K0 = to_dev(torch, Kh, dev)
    Ks = [K0] + [K0.clone() for _ in range(copies - 1)]
    launch = sp.SP_LAUNCH_COOPERATIVE if args.cooperative else sp.SP_LAUNCH_RESIDENT
    desc = sp.score_desc(w.L, w.H, w.Hkv, w.d, w.N, sp.SP_BF16 if w.dtype else sp.SP_F32, 0.0,
                         launch)
    ws = torch.empty(sp.sp_score_workspace_bytes(desc, M), dtype=torch.uint8, device=dev)
    imp = torch.empty(M, dtype=torch.float32, device=dev)
    kept = torch.empty(M, dtype=torch.int32, device=dev)
    pos = torch.empty(M, dtype=torch.int32, device=dev)
    nk = torch.empty(1, dtype=torch.int32, device=dev)
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

    def make_step(params):
        # (the selection's workspace: several workgroups select a long prompt)
        nb = sp.sp_select_workspace_bytes(1, M, params)
        sel_ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb > 0 else False

        def step(i, kev=None, sev=None, xev=None):
            if kev is not None:
                sp.sp_profile_score_kernel(kev[0], kev[1])
            if sev is not None:
                sev[0].record()
            sp.sp_score(Q, Ks[i % copies], M, out=imp, workspace=ws, launch=launch)
            if sev is not None:
                sev[1].record()
            if kev is not None:
                sp.sp_profile_score_kernel()
            if xev is not None:
                xev[0].record()
            sp.sp_select(imp, params, kept_idx=kept, pos_ids=pos, n_kept=nk, workspace=sel_ws)
            if xev is not None:
                xev[1].record()
        return step

    res = run_steps(torch, sp, make_step(select_params(sp, sels[0])), steps, warmup,
                    args.settle_s, args.kernel_steps, ws)
    res["n_kept"] = int(nk.cpu()[0])
    alg = alg_bytes_of(w, [M])
    out = {"value": M / (res["ms_per_step"] / 1e3), "unit": "tokens/s", "M": M,
           "roofline": roofline(alg, res["kernel_ms_mean"] / 1e3, load_traffic(w.name)),
           "timing": res, "alg_bytes_per_score_launch": alg, "k_copies": copies, "plan": plan,
           "config": workload_desc(w, sels[0])}
    if len(sels) > 1:
        modes = {}
        for sel in sels:
            r = run_steps(torch, sp, make_step(select_params(sp, sel)), max(10, steps // 2),
                          warmup, args.settle_s, 50, ws)
            modes[sel_desc(sel)] = {"value": M / (r["ms_per_step"] / 1e3),
                                    "ms_per_step": r["ms_per_step"],
                                    "select_ms_mean": r["select_ms_mean"],
                                    "n_kept": int(nk.cpu()[0])}
        out["select_modes"] = modes
    if sels[0].mode != "threshold":
        # the same step as one launch (sp_score_select: the selection runs in
        # the scoring launch, after its scores)
        fparams = select_params(sp, sels[0])

        def fused_step(i, kev=None, sev=None, xev=None):
            if kev is not None:
                sp.sp_profile_score_kernel(kev[0], kev[1])
            if sev is not None:
                sev[0].record()
            sp.sp_score_select(Q, Ks[i % copies], fparams, M=M, out=imp, kept_idx=kept, pos_ids=pos,
                               n_kept=nk, workspace=ws, launch=launch)
            if sev is not None:
                sev[1].record()
            if kev is not None:
                sp.sp_profile_score_kernel()
            if xev is not None:
                xev[0].record()
                xev[1].record()

        r = run_steps(torch, sp, fused_step, steps, warmup, args.settle_s, 50, ws)
        out["fused"] = {"value": M / (r["ms_per_step"] / 1e3), "ms_per_step": r["ms_per_step"],
                        "kernel_ms_mean": r["kernel_ms_mean"], "n_kept": int(nk.cpu()[0])}
    del Q, Ks, K0, ws
    torch.cuda.empty_cache()
    if cpu_s > 0:
        if w.name in ("tiny", "spec0.8b_m4608"):
            out["cpu_baseline"] = cpu_baseline(w, sels[0], [(Qh, Kh, M)], cpu_s)
            # the per-core figure: one thread
            out["cpu_baseline_1thread"] = cpu_baseline(w, sels[0], [(Qh, Kh, M)], cpu_s / 2,
                                                       threads=1)
        else:
            layers = None if w.M <= 32768 else 8
            out["cpu_baseline"] = cpu_baseline(w, sels[0], [(Qh, Kh, M)], cpu_s,
                                               max_layers=layers)
    return out


def bench_ragged(args, w, sel, sp, torch, dev, steps, warmup, cpu_s):
    """A batch of R prompts of different lengths: one step is sp_score_varlen
    + sp_select_varlen over the whole batch. The batch's keys (tens of GB) are
    far larger than the Infinity Cache, so one copy suffices. The roofline
    figure uses the sp_score_varlen call's duration (its scoring launches:
    requests alone, or several of similar length in one launch), a lower
    bound for the kernels' rate."""
    import synth

    Qh, Kh, cu = synth.make_ragged(w)
    total = int(cu[-1])
    R = len(cu) - 1
    Ms = np.diff(cu)
    Q = to_dev(torch, Qh, dev)
    K = to_dev(torch, Kh, dev)
    launch = sp.SP_LAUNCH_COOPERATIVE if args.cooperative else sp.SP_LAUNCH_RESIDENT
    desc = sp.score_desc(w.L, w.H, w.Hkv, w.d, w.N, sp.SP_BF16 if w.dtype else sp.SP_F32, 0.0,
                         launch)
    ws_bytes = sp.sp_score_batch_workspace_bytes(desc, cu)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    launches = int(sp.sp_score_batch_plan(desc, cu, ws_bytes).max()) + 1
    imp = torch.empty(total, dtype=torch.float32, device=dev)
    kept = torch.empty(total, dtype=torch.int32, device=dev)
    pos = torch.empty(total, dtype=torch.int32, device=dev)
    nk = torch.empty(R, dtype=torch.int32, device=dev)
    params = select_params(sp, sel)

    def step(i, kev=None, sev=None, xev=None):
        ev = kev if kev is not None else sev
        if ev is not None:
            ev[0].record()
        sp.sp_score_varlen(Q, K, cu, out=imp, workspace=ws, launch=launch)
        if ev is not None:
            ev[1].record()
        if xev is not None:
            xev[0].record()
        sp.sp_select_varlen(imp, cu, params, kept_idx=kept, pos_ids=pos, n_kept=nk)
        if xev is not None:
            xev[1].record()

    res = run_steps(torch, sp, step, steps, warmup, args.settle_s, args.kernel_steps, ws)
    res["n_kept_total"] = int(nk.sum().cpu())
    alg = alg_bytes_of(w, Ms)
    out = {"value": total / (res["ms_per_step"] / 1e3), "unit": "tokens/s", "M": total,
           "roofline": roofline(alg, res["kernel_ms_mean"] / 1e3, None),
           "roofline_basis": "sp_score_varlen call (all its scoring launches)",
           "timing": res, "alg_bytes_per_step": alg, "requests": R, "score_launches": launches,
           "config": dict(workload_desc(w, sel), M=total,
                          workload=f"{w.name}: R={R} prompts, M in [{int(Ms.min())}, "
                                   f"{int(Ms.max())}], sum {total}; L={w.L} H={w.H} "
                                   f"Hkv={w.Hkv} d={w.d} N={w.N}")}
    del Q, K, ws
    torch.cuda.empty_cache()
    if cpu_s > 0:
        # sample: the shortest and the longest request, scoring 8 of the 32
        # layers (scaled), then the whole batch's tokens per second estimated
        # from their per-token rate
        reqs = []
        for r in sorted({int(np.argmin(Ms)), int(np.argmax(Ms))}):
            k0 = int(cu[r]) + r * w.N
            reqs.append((Qh[r], np.ascontiguousarray(Kh[:, :, k0:k0 + int(Ms[r]) + w.N]),
                         int(Ms[r])))
        out["cpu_baseline"] = cpu_baseline(w, sel, reqs, cpu_s, max_layers=8)
    return out


def bench_windowed(args, w, sel, sp, torch, dev):
    """One prompt of the workload scored in sliding windows (each window with
    its own synthetic queries and keys, as a speculator run per window gives):
    one step is sp_score_windows + sp_select over the prompt's M tokens. The
    roofline figure uses the sp_score_windows call's duration (its scoring
    launches: windows are of one length, so several share a launch)."""
    import synth

    starts, lens, keeps = sp.sp_window_layout(w.M, args.window, args.stride)
    ww = dataclasses.replace(w, R=len(lens), M=0, len_range=())
    Qh, Kh, cu = synth.make_ragged(ww, lens)
    R = len(lens)
    Q = to_dev(torch, Qh, dev)
    K = to_dev(torch, Kh, dev)
    del Qh, Kh
    launch = sp.SP_LAUNCH_COOPERATIVE if args.cooperative else sp.SP_LAUNCH_RESIDENT
    desc = sp.score_desc(w.L, w.H, w.Hkv, w.d, w.N, sp.SP_BF16 if w.dtype else sp.SP_F32, 0.0,
                         launch)
    ws_bytes = sp.sp_score_batch_workspace_bytes(desc, cu)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    launches = int(sp.sp_score_batch_plan(desc, cu, ws_bytes).max()) + 1
    imp = torch.empty(w.M, dtype=torch.float32, device=dev)
    kept = torch.empty(w.M, dtype=torch.int32, device=dev)
    pos = torch.empty(w.M, dtype=torch.int32, device=dev)
    nk = torch.empty(1, dtype=torch.int32, device=dev)
    params = select_params(sp, sel)

    def step(i, kev=None, sev=None, xev=None):
        ev = kev if kev is not None else sev
        if ev is not None:
            ev[0].record()
        sp.sp_score_windows(Q, K, cu, keeps, out=imp, workspace=ws, launch=launch)
        if ev is not None:
            ev[1].record()
        if xev is not None:
            xev[0].record()
        sp.sp_select(imp, params, kept_idx=kept, pos_ids=pos, n_kept=nk)
        if xev is not None:
            xev[1].record()

    res = run_steps(torch, sp, step, args.steps, args.warmup, args.settle_s, args.kernel_steps,
                    ws)
    alg = alg_bytes_of(w, lens)
    return {"value": w.M / (res["ms_per_step"] / 1e3), "ms_per_step": res["ms_per_step"],
            "roofline": roofline(alg, res["kernel_ms_mean"] / 1e3, None),
            "config": dict(workload_desc(w, sel), launch=launch_name(args),
                           workload=f"{w.name} in sliding windows of {args.window} tokens, "
                                    f"stride {args.stride}: {R} windows",
                           window=args.window, stride=args.stride),
            "detail": {"timing": res, "alg_bytes_per_step": alg, "windows": R,
                       "score_launches": launches,
                       "roofline_basis": "sp_score_windows call (all its scoring launches)",
                       "n_kept": int(nk.cpu()[0])}}


def read_probe(args, sp, torch, dev):
    """The practical HBM read ceiling: sp_read_probe (one plain streaming read
    of a buffer the size of the 8B / 32K workload's keys) over launch shapes;
    two buffers alternate so that no launch finds its data in the Infinity
    Cache."""
    import synth
    w = synth.WORKLOADS["spec8b_m32k"]
    nbytes = w.L * w.Hkv * (w.M + w.N) * w.d * 2
    bufs = [torch.zeros(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    res = []
    for depth in (4, 8, 16):
        for grid in (128, 192, 222, 240, 256, 512, 1024, 4096):
            for i in range(3):
                sp.sp_read_probe(bufs[i % 2], grid, depth, flag)
            evs = _events(torch, 30)
            for i, (a, b) in enumerate(evs):
                a.record()
                sp.sp_read_probe(bufs[i % 2], grid, depth, flag)
                b.record()
            torch.cuda.synchronize()
            t = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
            res.append({"depth": depth, "grid": grid, "us_median": round(float(np.median(t)), 1),
                        "us_min": round(float(t.min()), 1),
                        "GBps_median": round(nbytes / float(np.median(t)) / 1e3, 1)})
    best = max(res, key=lambda r: r["GBps_median"])
    print(json.dumps({"probe": "sp_read_probe", "bytes": nbytes, "best": best,
                      "frac_of_peak": best["GBps_median"] / HBM_PEAK_GBS, "sweep": res,
                      "flag": int(flag.cpu()[0])}), flush=True)


def launch_name(args) -> str:
    return "cooperative" if args.cooperative else "resident"


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args.traffic_from[0], args.traffic_from[1], args.workload,
                      args.copy_probe_mib or 1024)
        return
    if args.gpus != 1:
        print("bench.py: this path runs on one GPU (there is no multi-GPU sharding to time); "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import attention_token_scoring_amd as sp
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.read_probe:
        read_probe(args, sp, torch, dev)
        return

    def sels_of(w):
        sels = list(w.selects)
        if args.select == "threshold":
            # the Implementation Guide program's selection at its defaults (keep
            # rate 0.3 unless the workload fixes one, 128-token fill, 2000-token cap)
            s = sels[0]
            sels = [dataclasses.replace(s, mode="threshold", pool_k=1,
                                        keep_rate=s.keep_rate or 0.3, mass=0.0,
                                        boost_first_n=0, boost_last_n=0)]
        return sels

    w = synth.WORKLOADS[args.workload]
    cpu_on = not args.no_cpu_baseline
    if args.window:
        if w.R != 1:
            print("bench.py: --window takes a single-prompt workload", file=sys.stderr)
            sys.exit(2)
        r = bench_windowed(args, w, sels_of(w)[0], sp, torch, dev)
        out = headline_line(args, w, r["value"], r["ms_per_step"], r["config"], r["roofline"])
        out["detail"] = r["detail"]
        print(json.dumps(out), flush=True)
        return

    def run(name, steps, warmup, cpu_s):
        ww = synth.WORKLOADS[name]
        print(f"bench.py: {name}", file=sys.stderr, flush=True)
        if ww.R != 1:
            return bench_ragged(args, ww, sels_of(ww)[0], sp, torch, dev, steps, warmup, cpu_s)
        return bench_single(args, ww, sels_of(ww), sp, torch, dev, steps, warmup, cpu_s)

    head = run(args.workload, args.steps, args.warmup,
               CPU_SECONDS.get(args.workload, 10.0) if cpu_on else 0.0)
    workloads = {args.workload: summary(head)}
    if not args.only:
        for name in ALL_WORKLOADS:
            if name == args.workload:
                continue
            steps, warmup = OTHER_STEPS[name]
            workloads[name] = summary(run(name, steps, warmup,
                                          CPU_SECONDS[name] if cpu_on else 0.0))
    cfg = dict(head["config"], launch=launch_name(args))
    out = headline_line(args, w, head["value"], head["timing"]["ms_per_step"], cfg,
                        head["roofline"])
    t = head["timing"]
    out["detail"] = {
        "score_kernel_ms_mean": t["kernel_ms_mean"], "score_kernel_ms_median": t["kernel_ms_median"],
        "score_kernel_ms_min": t["kernel_ms_min"], "score_kernel_launches_timed": t["kernel_launches"],
        "roofline_frac_median": roofline(head.get("alg_bytes_per_score_launch",
                                                  head.get("alg_bytes_per_step")),
                                         t["kernel_ms_median"] / 1e3, None)["frac"],
        "ms_per_step_events": t["ms_per_step_events"], "settle_steps": t["settle_steps"],
        "sp_score_ms_mean": t["sp_score_ms_mean"], "select_ms_mean": t["select_ms_mean"],
        "plan": head.get("plan"), "workloads": workloads,
    }
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    print(json.dumps(out), flush=True)


def summary(r):
    """The figures of one workload for detail.workloads."""
    t = r["timing"]
    s = {"config": r["config"]["workload"], "value": r["value"], "unit": "tokens/s",
         "ms_per_step": t["ms_per_step"], "steps": t["steps"], "warmup": t["warmup"],
         "roofline": r["roofline"], "score_kernel_ms_mean": t["kernel_ms_mean"],
         "score_kernel_ms_median": t["kernel_ms_median"], "sp_score_ms_mean": t["sp_score_ms_mean"],
         "select_ms_mean": t["select_ms_mean"]}
    for k in ("plan", "select_modes", "fused", "cpu_baseline", "cpu_baseline_1thread", "roofline_basis",
              "requests", "score_launches"):
        if k in r:
            s[k] = r[k]
    return s


def headline_line(args, w, value, ms_per_step, config, roof):
    return {
        "metric": METRIC,
        "value": value,
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
        "config": config,
        "roofline": roof,
    }


def release_device_memory():
    """Return torch's cached device memory while the runtime is whole: under
    a profiler, whose finalisation runs at exit, teardown work left to the
    interpreter's exit would run after it."""
    if "torch" in sys.modules:
        torch = sys.modules["torch"]
        if torch.cuda.is_initialized():
            torch.cuda.synchronize()
            torch.cuda.empty_cache()


if __name__ == "__main__":
    try:
        main()
    finally:
        release_device_memory()
