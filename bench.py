#!/usr/bin/env python3
"""Benchmark of batched speculative-sampling verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

One step = one spec_verify call (the whole path: normaliser + acceptance scan +
correction / bonus draw) over one batch of synthetic logits already resident in
HBM.  Steps cycle through R distinct input sets (>= 1 GiB in total) so that the
256 MB Infinity Cache cannot serve a repeated batch.  Prints one JSON line.

Metric: verified draft positions per second (B*G per call; every submitted draft
position is verified, including those after the first rejection, since all are
processed in parallel), with the achieved HBM bandwidth of the dominant kernel
against the 8 TB/s peak.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak) at B=64,V=128k"
PEAK_HBM_GBS = 8000.0
KERNEL = "k_verify"  # the kernel that streams the logits (and draws) in the timed workload
_CSRC = ROOT / "rejection_sampling_verify_02_amd" / "csrc"
_SHARED = ("sv_common.h", "sv_device.h", "sv_lanes.h")
# Per timed operation: the kernel whose HBM traffic is summarised, the workload the counters
# are taken on, its algorithmic bytes per launch, and the sources the summary is tied to
# (by hash: a summary taken on other sources is not used).
COUNTED = {
    "verify": dict(kernel="k_verify", workload="zipf_bf16_b64", desc="B=64, G=4, V=128256, bf16",
                   alg=147750912, sources=("spec_verify.hip", "sv_draw.h") + _SHARED,
                   why="The excess is the second read of the two rows at each rejecting sequence's first "
                       "rejection (2 x 256.5 KB each; most sequences of this workload reject), plus the bonus "
                       "chunk's re-read and the partials, records and segment masses.  Every other logit is "
                       "fetched from HBM once."),
    "overlap": dict(kernel="k_overlap", workload="overlap_zipf_bf16_b64", desc="B=64, G=4, V=128256, bf16",
                    alg=131334144, sources=("spec_overlap.hip",) + _SHARED,
                    why="Every logit is read twice, first for the normalisers and then for the overlap terms; "
                        "the excess is the part of the second read that misses the XCD's L2."),
    "sample": dict(kernel="k_verify", workload="sample_bf16_b256", desc="B=256, V=128256, bf16",
                   alg=65667072, sources=("spec_verify.hip", "sv_draw.h") + _SHARED,
                   why="The excess is each row's one re-read segment (1 KiB) and the partials and segment "
                       "masses handed between workgroups."),
    "tree": dict(kernel="k_tree_rows", workload="tree_bf16_b16_n32", desc="16 trees of 32 nodes, V=128256, bf16",
                 alg=210698956, sources=("spec_tree.hip", "sv_draw.h") + _SHARED,
                 why="k_tree_rows reads every target row and the draft rows of nodes with children once; the "
                     "residual masses the walk needs and the draw read their rows in k_tree_draw."),
    "typical": dict(kernel="k_typical", workload="typical_zipf_bf16_b64", desc="B=64, G=4, V=128256, bf16",
                    alg=82083840, sources=("spec_typical.hip",) + _SHARED,
                    why="Every logit is read once; the excess is the partials handed between workgroups."),
}


def counters_path(op: str) -> Path:
    c = COUNTED[op]
    return ROOT / "profiles" / f"{c['kernel']}_{c['workload']}_counters.json"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime that torch has already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n: int) -> list[int]:
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(ev.value)
        return out

    def record(self, ev: int, stream: int) -> None:
        self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        self.hip.hipEventSynchronize(ctypes.c_void_p(b))
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, evs) -> None:
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def make_sets(cid: int, n_sets: int, dev):
    """R input sets of one workload on the device; draft tokens drawn by the library itself
    (each draft row is its own G = 0 call: X ~ q by inverse CDF with the draft uniforms, or
    the draft argmax at temperature 0).  The top-k workload's third group needs the
    target's kept set, found here with torch.topk (input preparation, outside the timed
    path)."""
    import torch
    import rejection_sampling_verify_02_amd as sv
    from rejection_sampling_verify_02_amd import workloads as wl

    sets, host = [], []
    for s in range(n_sets):
        t0 = time.time()
        raw = wl.make_config(cid, seed=wl.CONFIGS[cid].seed + 1000 * s)
        cfg = raw.cfg
        B, G, V = raw.B, raw.G, raw.V

        def dev_t(a):
            t = torch.from_numpy(np.ascontiguousarray(a))
            return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

        target, draft = dev_t(raw.target), dev_t(raw.draft)
        if len(raw.disjoint_rows):
            # the draft's top-k support disjoint from the target's: -1e4 on the target's kept
            # set {z >= k-th largest} (ties included), position by position
            rows = torch.as_tensor(raw.disjoint_rows, device=dev)
            zt = target[rows, :G].float()
            tau = torch.topk(zt, cfg.top_k, dim=-1).values[..., -1:]
            d = draft[rows]
            d[zt >= tau] = torch.tensor(-1e4, dtype=d.dtype, device=dev)
            draft[rows] = d
        drows = draft.reshape(B * G, 1, V)
        if cfg.temperature == 0:
            _, tok = sv.spec_verify(drows, None, None, None, None, 0.0, 0)
        else:
            u_draft = dev_t(raw.u_draft.reshape(B * G))
            _, tok = sv.spec_verify(drows, None, None, None, u_draft, cfg.temperature, cfg.top_k)
        tokens = tok.reshape(B, G).contiguous()
        fixed = torch.from_numpy(raw.fixed_tokens).to(dev)
        tokens = torch.where(fixed >= 0, fixed, tokens)
        greedy = cfg.temperature == 0
        sets.append(dict(target=target, draft=None if greedy else draft, tokens=tokens,
                         u_accept=None if greedy else dev_t(raw.u_accept),
                         u_sample=None if greedy else dev_t(raw.u_sample)))
        if len(raw.disjoint_rows):  # the host copy for the CPU baseline gets the same draft
            hd = draft.cpu()
            hd = hd.view(torch.int16).numpy().view(np.uint16) if hd.dtype == torch.bfloat16 else hd.numpy()
        else:
            hd = raw.draft
        host.append(dict(target=raw.target, draft=hd, u_accept=raw.u_accept, u_sample=raw.u_sample))
        log(f"[bench] input set {s + 1}/{n_sets} ready ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize(dev)
    for s, h in zip(sets, host):
        h["tokens"] = s["tokens"].cpu().numpy()
    return sets, host


def counters_traffic(op: str):
    """HBM bytes per launch of the operation's kernel from its committed rocprofv3 counter
    summary, or None when the summary is missing or was taken on a different source."""
    path = counters_path(op)
    if not path.exists():
        return None, "no counter summary"
    c = json.loads(path.read_text())
    if c.get("source_sha256") != source_sha(op):
        return None, "kernel changed since the counters were taken"
    return float(c["traffic_bytes_per_launch"]), c.get("note", "")


def cpu_baseline(host_sets, cfg, seconds: float):
    """The oracle on the host over whole input sets, in verified positions per second."""
    import oracle

    oracle._load()
    B, G = host_sets[0]["tokens"].shape
    state = {"i": 0}

    def once(threads):
        h = host_sets[state["i"] % len(host_sets)]
        state["i"] += 1
        oracle.spec_verify_ref(h["target"], h["draft"], h["tokens"], h["u_accept"], h["u_sample"],
                               cfg.temperature, cfg.top_k, nthreads=threads)

    return oracle_baseline(once, B * G, "positions/s", seconds,
                           f"full calls (B={B}, G={G}) over {len(host_sets)} input sets; the oracle stops "
                           f"reading each sequence at its first rejection")


def summarize_counters(kdir: str, cdir: str, op: str) -> None:
    """Turn rocprofv3 --pmc CSV output into the traffic summary bench.py reads.

    kdir holds the FETCH_SIZE and WRITE_SIZE runs of the benchmark, cdir those of the
    copy probe.  Counters are KiB per dispatch; each is scaled by (bytes the copy
    really moves) / (what the counter read for it): a copy of N bytes reads N and
    writes N.
    """
    import csv
    import glob

    def rows_of(d, counter):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            out += [r for r in csv.DictReader(open(f)) if r.get("Counter_Name") == counter]
        return out

    def per_dispatch(d, counter, kernel_pred):
        return [float(r["Counter_Value"]) for r in rows_of(d, counter) if kernel_pred(r)]

    # the timed workload's dispatches: the most frequent grid among the kernel's dispatches
    # (the draft-token draws that prepare the inputs launch it on another grid)
    spec = COUNTED[op]
    kernel = spec["kernel"]
    grids = [int(r.get("Grid_Size") or 0) for r in rows_of(kdir, "FETCH_SIZE") if kernel in r["Kernel_Name"]]
    main_grid = max(set(grids), key=grids.count) if grids else -1
    is_main = lambda r: kernel in r["Kernel_Name"] and int(r.get("Grid_Size") or 0) == main_grid
    is_copy = lambda r: ("copy" in r["Kernel_Name"].lower() or "elementwise" in r["Kernel_Name"].lower())
    probe = json.loads(open(os.path.join(cdir, "probe.json")).read())
    nbytes = probe["copy_probe_bytes"]
    cf = per_dispatch(cdir, "FETCH_SIZE", is_copy)
    cw = per_dispatch(cdir, "WRITE_SIZE", is_copy)
    kf = per_dispatch(kdir, "FETCH_SIZE", is_main)
    kw = per_dispatch(kdir, "WRITE_SIZE", is_main)
    copy_f = max(cf) * 1024.0
    copy_w = max(cw) * 1024.0
    f_fetch, f_write = nbytes / copy_f, nbytes / copy_w
    fetch = float(np.median(kf)) * 1024.0 * f_fetch
    write = float(np.median(kw)) * 1024.0 * f_write
    res = {"kernel": kernel, "workload": f"{spec['workload']} ({spec['desc']})",
           "dispatches": {"fetch": len(kf), "write": len(kw)},
           "fetch_kib_median": float(np.median(kf)), "write_kib_median": float(np.median(kw)),
           "copy_probe_bytes": nbytes, "copy_fetch_kib": max(cf), "copy_write_kib": max(cw),
           "scale_fetch": f_fetch, "scale_write": f_write,
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "traffic_bytes_per_launch": fetch + write,
           "algorithmic_bytes": spec["alg"],
           "source_sha256": source_sha(op),
           "note": "FETCH_SIZE and WRITE_SIZE from separate rocprofv3 --pmc runs, scaled by a plain copy"}
    counters_path(op).write_text(json.dumps(res, indent=1) + "\n")
    ratio = (fetch + write) / spec["alg"]
    md = [f"# HBM traffic of {kernel}, {spec['workload']} ({spec['desc']})", "",
          "Commands (on the MI355X machine, after `cd /tmp && export TMPDIR=/tmp`; each counter in a run of its own):", "", "```"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        md.append(f"rocprofv3 --pmc {c} --output-format csv -d <k>/{c} -o k -- python3 <repo>/bench.py --op {op} "
                  f"--steps 30 --warmup 5 --no-cpu-baseline --no-stage-events --no-probe")
    md += ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d <c>/fetch -o c -- python3 <repo>/bench.py "
           "--copy-probe 1073741824 > <c>/probe.json",
           "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <c>/write -o c -- python3 <repo>/bench.py "
           "--copy-probe 1073741824",
           f"python3 bench.py --op {op} --summarize-counters <k> <c>",
           "```", "",
           f"Calibration: a {nbytes / 2**30:g} GiB device copy reads FETCH_SIZE = {max(cf):,.1f} KiB and "
           f"WRITE_SIZE = {max(cw):,.1f} KiB, so FETCH_SIZE is scaled by {f_fetch:.5f} and WRITE_SIZE by {f_write:.5f}.",
           "",
           f"| per {kernel} launch (median of {len(kf)} dispatches on the workload's grid) | counter | scaled bytes |",
           "|---|---|---|",
           f"| FETCH_SIZE | {float(np.median(kf)):,.1f} KiB | {fetch:,.0f} |",
           f"| WRITE_SIZE | {float(np.median(kw)):,.1f} KiB | {write:,.0f} |",
           f"| total traffic | | {fetch + write:,.0f} |",
           f"| algorithmic bytes (every logit the result depends on, once) | | {spec['alg']:,} |", "",
           f"Traffic is {ratio:.2f}x the algorithmic bytes.  {spec.get('why', '')}", ""]
    counters_path(op).with_suffix(".md").write_text("\n".join(md))
    print(json.dumps(res))


def _last_line(path: str):
    line = None
    for ln in open(path):
        ln = ln.strip()
        if ln.startswith("{"):
            line = json.loads(ln)
    return line


def summarize_trace(tdir: str, line_file: str, cmd: str, ref_file: str | None = None) -> None:
    """Write the kernel-trace summary of one profiled benchmark run: rocprofv3's own
    per-dispatch durations (kernel_trace.csv) for the dispatches of the workload's main
    kernel, split into the benchmark's phases in launch order (the line's "dispatches"
    field), next to the line's own HIP-event figures from the same run."""
    import csv
    import glob

    line = _last_line(line_file)
    rows = []
    for f in glob.glob(os.path.join(tdir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    rf = line["roofline"]
    kernel = rf["kernel"]

    def grid(r):
        return int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0)

    mine = [r for r in rows if f"{kernel}<" in r["Kernel_Name"] or r["Kernel_Name"].endswith(kernel)]
    grids = [grid(r) for r in mine]
    main = max(set(grids), key=grids.count)
    d = sorted((r for r in mine if grid(r) == main), key=lambda r: int(r["Start_Timestamp"]))
    us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in d]
    ph = line["dispatches"]
    spans, o = [], 0
    for name in ("warmup", "timed_loops", "per_kernel_events", "flushed"):
        n = ph.get(name, 0)
        spans.append((name, us[o:o + n]))
        o += n
    spans.append(("after", us[o:]))  # calls made after the timing (outputs checked)
    alg = rf["algorithmic_bytes"]
    out = [f"# Kernel trace: {kernel}, {line['config']['workload']}", "",
           "Command (repository root on the MI355X machine, after `cd /tmp && export TMPDIR=/tmp`):", "",
           "```", cmd, "```", "",
           f"Dispatches of `{kernel}` on the workload's grid ({main} threads), in launch order, split into",
           "the benchmark's phases; durations from rocprofv3's kernel trace of the same run.", "",
           "| phase | dispatches | mean (us) | median (us) | min (us) | GB/s at the mean | of 8 TB/s |",
           "|---|---|---|---|---|---|---|"]
    for name, v in spans:
        if not v:
            continue
        m = float(np.mean(v))
        out.append(f"| {name} | {len(v)} | {m:.3f} | {np.median(v):.3f} | {np.min(v):.3f} | "
                   f"{alg / m / 1e3:.1f} | {alg / m / 1e3 / PEAK_HBM_GBS:.4f} |")
    ev = dict(spans).get("per_kernel_events", [])
    out += ["", f"The profiled run's own line: `{kernel}` {rf['avg_launch_us']} us from bench.py's per-dispatch HIP "
            f"events (under the profiler the events are recorded late, so they read long), event-free loop "
            f"{line['ms_per_step'] * 1e3:.2f} us per call ({line['value'] / 1e6:.3f} M {line['unit']})."]
    if ev:
        m = float(np.mean(ev))
        out.append(f"rocprofv3 over the per-kernel-event dispatches: {m:.3f} us, frac {alg / m / 1e3 / PEAK_HBM_GBS:.4f}.")
        if ref_file:
            ref = _last_line(ref_file)
            rr = ref["roofline"]
            out.append(f"The same command without the profiler, on the same machine: `{kernel}` {rr['avg_launch_us']} us from "
                       f"the events, frac {rr['frac']} ({(m / rr['avg_launch_us'] - 1) * 100:+.2f}% from rocprofv3's "
                       f"{m:.3f} us); event-free loop {ref['ms_per_step'] * 1e3:.2f} us per call "
                       f"({ref['value'] / 1e6:.3f} M {ref['unit']}).")
    others = [k.split(":", 1)[1] for k in line.get("per_kernel_us", {}) if k.split(":", 1)[1] != kernel]
    if others:
        out += ["", "The call's other kernels (rocprofv3, every dispatch on each kernel's most frequent grid; "
                "bench.py's per-dispatch events of the reference run):", "",
                "| kernel | dispatches | mean (us) | median (us) | events (us) |", "|---|---|---|---|---|"]
        ref_pk = (_last_line(ref_file) if ref_file else line).get("per_kernel_us", {})
        for name in others:
            rs = [r for r in rows if f"{name}<" in r["Kernel_Name"] or r["Kernel_Name"].endswith(name)]
            if not rs:
                continue
            gs = [grid(r) for r in rs]
            g0 = max(set(gs), key=gs.count)
            v = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs if grid(r) == g0]
            ev_us = next((val for k, val in ref_pk.items() if k.split(":", 1)[1] == name), None)
            out.append(f"| `{name}` | {len(v)} | {np.mean(v):.3f} | {np.median(v):.3f} | {ev_us} |")
        out.append("")
    src = _last_line(ref_file) if ref_file else line
    if src.get("read_probe"):
        pr = src["read_probe"]
        out.append(f"Streaming-read probe ({'the run without the profiler' if ref_file else 'the same run'}): "
                   f"{pr['GBs']} GB/s ({pr['frac_of_peak']} of 8 TB/s) over {pr['bytes_per_launch']:,} bytes per "
                   f"launch; {kernel} reaches {src['roofline'].get('frac_of_read_probe')} of it.")
    out.append("")
    path = ROOT / "profiles" / f"{kernel}_{line['config']['workload']}_kernel_trace.md"
    path.write_text("\n".join(out))
    print(path)


def run_timeline(args, dev) -> dict:
    """Where one call's time goes (B=64, G=4, V=128256 bf16), from the timeline build of the library
    (libspec_verify_timeline.so: the product sources with wall-clock stamps at fixed
    points of each sequence's path).  Per call: when the stream of partials ends, when the
    call's last token is written, and for the sequence that finishes last, each step of its
    tail.  Medians over the calls; microseconds from the grid's first stamp."""
    import ctypes
    import torch
    import rejection_sampling_verify_02_amd as sv
    from rejection_sampling_verify_02_amd import build as svb

    sv._lib = sv.load_library(svb.LIB_TIMELINE)  # every binding call now goes through it
    from rejection_sampling_verify_02_amd import workloads as wl
    cfg = wl.CONFIGS[args.config]
    B, G, V = cfg.B, cfg.G, cfg.V
    n_sets = args.sets or 8
    sets, _ = make_sets(args.config, n_sets, dev)
    words = 8 + B * 512
    stamps = torch.zeros((words,), dtype=torch.int64, device=dev)
    khz = ctypes.c_int32(0)
    rc = sv._lib.sv_timeline_stamps(ctypes.c_void_p(stamps.data_ptr()), ctypes.byref(khz))
    if rc != 0:
        raise RuntimeError(f"sv_timeline_stamps returned {rc}")
    ticks_us = khz.value / 1000.0
    ws = sv.Workspace()
    stream = torch.cuda.current_stream(dev).cuda_stream
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    C = -(-V * (2 if cfg.dtype == "bf16" else 4) // 32768)
    rps, nd = 2 * G + 1, min(C * 4, 96)

    def call(i):
        s = sets[i % n_sets]
        sv.spec_verify(s["target"], s["draft"], s["tokens"], s["u_accept"], s["u_sample"], cfg.temperature,
                       cfg.top_k, workspace=ws, stream=stream, out=(acc, out))

    for i in range(args.warmup):
        call(i)
    rec = {k: [] for k in ("stream_end", "call_end", "last_partial", "fin_parts", "fin_record", "draws_have_record",
                           "masses_out", "combiner_in", "token_out")}
    for i in range(args.steps):
        stamps.zero_()
        call(i)
        torch.cuda.synchronize(dev)
        h = stamps.cpu().numpy().astype(np.float64)
        t0 = h[0]
        us = lambda x: (x - t0) / ticks_us
        last_parts, dones = [], []
        for b in range(B):
            base = 8 + 512 * b
            fp = h[base: base + min(rps * C, 256)]
            last_parts.append(us(fp[fp > 0].max()) if np.any(fp > 0) else np.nan)
            dones.append(us(h[base + 461]) if h[base + 461] > 0 else np.nan)
        bl = int(np.nanargmax(dones))
        base = 8 + 512 * bl

        def step(k):
            return us(h[base + k]) if h[base + k] > 0 else np.nan

        def most(lo):
            v = h[base + lo: base + lo + nd]
            return us(v[v > 0].max()) if np.any(v > 0) else np.nan

        rec["stream_end"].append(np.nanmax(last_parts))
        rec["call_end"].append(np.nanmax(dones))
        rec["last_partial"].append(last_parts[bl])
        rec["fin_parts"].append(step(257))
        rec["fin_record"].append(step(258))
        rec["draws_have_record"].append(most(260))
        rec["masses_out"].append(most(360))
        rec["combiner_in"].append(step(460))
        rec["token_out"].append(step(461))
    med = {k: round(float(np.nanmedian(v)), 3) for k, v in rec.items()}
    res = {"workload": cfg.name, "calls": args.steps, "wall_clock_khz": khz.value, "median_us": med}
    cmd = (f"python3 <repo>/bench.py --timeline --steps {args.steps} --warmup {args.warmup}"
           + (f" --config {args.config}" if args.config != 3 else ""))
    names = {"stream_end": "the last partial of any sequence is out (the stream's end)",
             "call_end": "the call's last token is written",
             "last_partial": "last sequence to finish: its last partial out",
             "fin_parts": "its finisher has every partial",
             "fin_record": "its finisher has combined, scanned and published the draw's record",
             "draws_have_record": "its draw items have the record (the last of them)",
             "masses_out": "its draw items' segment masses are out (the last of them)",
             "combiner_in": "its combiner has every segment mass",
             "token_out": "its token is written"}
    lines = [f"# Timeline: k_verify, {cfg.name}", "",
             "Command (repository root on the MI355X machine; the timeline build of the library, which the build "
             "step compiles next to the product library):", "", "```", cmd, "```", "",
             f"Wall clock stamps (`wall_clock64`, {khz.value} kHz) stored by the kernels of "
             "`libspec_verify_timeline.so` at fixed points of each sequence's path (`sv_timeline_stamps`); "
             f"microseconds from the grid's first stamp, medians over {args.steps} calls after {args.warmup} "
             "warm-up calls.", "", "| point | µs |", "|---|---|"]
    for k, v in med.items():
        lines.append(f"| {names[k]} | {v} |")
    lines.append("")
    (ROOT / "profiles" / f"k_verify_{cfg.name}_timeline.md").write_text("\n".join(lines))
    return res


def copy_probe(nbytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").uniform_()
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


LOOPS = 5  # timed loops of K calls; the reported time is their median


def time_loop(call, plan, K, warmup, stream, dev, hev, stage_events, flush_calls=0):
    """Warm-up, then LOOPS loops of K calls each, timed as a caller runs them (wall clock
    and stream events; the median loop gives the throughput), then (unless disabled) K calls
    with a (start, stop) event pair on every kernel dispatch, then flush_calls single calls
    each after writing a 1 GiB scratch buffer (cold caches).  Returns a dict."""
    import torch
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize(dev)
    log(f"[bench] warmup done ({warmup} calls)")
    walls, gpus = [], []
    n = warmup
    for lp in range(LOOPS):
        loop_ev = hev.create(2)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        hev.record(loop_ev[0], stream)
        for i in range(K):
            call(n + i)
        hev.record(loop_ev[1], stream)
        torch.cuda.synchronize(dev)
        walls.append(time.perf_counter() - t0)
        gpus.append(hev.elapsed_ms(loop_ev[0], loop_ev[1]))
        hev.destroy(loop_ev)
        n += K
    log(f"[bench] {LOOPS} timed loops of {K} calls: wall " + ", ".join(f"{w * 1e3:.3f}" for w in walls) + " ms")
    # The per-dispatch event pairs add a few microseconds of gap between kernels, so the
    # loops above give the throughput and this one each kernel's own duration.
    per_kernel, wall2 = {}, None
    if stage_events:
        nl = len(plan)
        stage = [hev.create(2 * nl) for _ in range(K)]
        torch.cuda.synchronize(dev)
        t1 = time.perf_counter()
        for i in range(K):
            call(n + i, stage[i])
        torch.cuda.synchronize(dev)
        wall2 = time.perf_counter() - t1
        durs = np.array([[hev.elapsed_ms(ev[2 * j], ev[2 * j + 1]) for j in range(nl)] for ev in stage])
        for j, name in enumerate(plan):
            per_kernel[f"{j}:{name}"] = float(np.mean(durs[:, j]) * 1e3)
        for ev in stage:
            hev.destroy(ev)
        n += K
        log(f"[bench] timed {K} calls with per-kernel events: wall {wall2 * 1e3:.2f} ms")
    cold = []
    if flush_calls:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        ev = hev.create(2)
        for i in range(flush_calls):
            scratch.fill_(float(i))
            torch.cuda.synchronize(dev)
            hev.record(ev[0], stream)
            call(n + i)
            hev.record(ev[1], stream)
            cold.append(hev.elapsed_ms(ev[0], ev[1]) * 1e3)
        hev.destroy(ev)
        del scratch
        torch.cuda.synchronize(dev)
        n += flush_calls
        log(f"[bench] {flush_calls} single calls after a 1 GiB flush: median {np.median(cold):.2f} us")
    med = int(np.argsort(walls)[len(walls) // 2])
    return {"wall": walls[med], "gpu_ms": gpus[med], "walls": walls, "per_kernel": per_kernel,
            "wall2": wall2, "cold_us": cold, "calls": n}


def timing_fields(t, K, W):
    """The timing part of a result line: median loop, all loops, per-kernel durations, flushed
    latency, and how many calls each phase made (in launch order; a kernel trace of the run
    splits its dispatches by these counts)."""
    return {
        "dispatches": {"warmup": W, "timed_loops": LOOPS * K, "per_kernel_events": K if t["per_kernel"] else 0,
                       "flushed": len(t["cold_us"])},
        "timed_loops_ms": [round(w * 1e3, 4) for w in t["walls"]],
        "gpu_event_ms_per_step": round(t["gpu_ms"] / K, 5),
        "per_kernel_us": {k: round(v, 3) for k, v in t["per_kernel"].items()},
        "ms_per_step_with_kernel_events": None if t["wall2"] is None else round(t["wall2"] * 1e3 / K, 5),
        "single_call_after_flush_us": None if not t["cold_us"] else {
            "median": round(float(np.median(t["cold_us"])), 3), "min": round(float(np.min(t["cold_us"])), 3),
            "calls": len(t["cold_us"]), "flush": "1 GiB written before each call"},
    }


def read_probe(nbytes: int, n_sets: int, K: int, dev, hev):
    """The plain streaming-read probe (sv_read_probe) over n_sets buffers of nbytes each,
    rotated like the workload's input sets: mean kernel duration from per-dispatch events,
    and a checksum of one buffer against torch's sum of its words."""
    import torch
    import rejection_sampling_verify_02_amd as sv
    chunk = 32768
    nb = nbytes // chunk * chunk
    bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (nb // 4,), dtype=torch.int32, device=dev) for _ in range(n_sets)]
    out = torch.empty((nb // chunk,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    sv.read_probe(bufs[0], out, stream=stream)
    got = int(out.to(torch.int64).sum().item()) % (1 << 32)
    want = int(bufs[0].to(torch.int64).sum().item()) % (1 << 32)
    if got != want:
        raise RuntimeError(f"read probe checksum {got:#x} != {want:#x}")
    for i in range(10):
        sv.read_probe(bufs[i % n_sets], out, stream=stream)
    evs = [hev.create(2) for _ in range(K)]
    torch.cuda.synchronize(dev)
    for i in range(K):
        hev.record(evs[i][0], stream)
        sv.read_probe(bufs[i % n_sets], out, stream=stream)
        hev.record(evs[i][1], stream)
    torch.cuda.synchronize(dev)
    us = np.array([hev.elapsed_ms(a, b) * 1e3 for a, b in evs])
    for e in evs:
        hev.destroy(e)
    del bufs
    gbs = nb / (float(np.mean(us)) * 1e-6) / 1e9
    log(f"[bench] read probe: {nb / 1e6:.2f} MB per launch, {np.mean(us):.3f} us -> {gbs:.1f} GB/s")
    return {"kernel": "k_read_probe", "bytes_per_launch": nb, "avg_launch_us": round(float(np.mean(us)), 3),
            "median_launch_us": round(float(np.median(us)), 3), "GBs": round(gbs, 1),
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "launches": K, "buffers": n_sets}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_baseline(run_once, units_per_call: float, unit: str, seconds: float, sample: str):
    """The oracle as committed (fp64, unmodified), timed on the host: on every core in this
    process's affinity set and on one core, each as the median of 3 runs of about
    seconds / 6 (at least one call each).  run_once(nthreads) makes one full call."""
    try:
        all_cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        all_cores = os.cpu_count() or 1
    per_run = max(seconds / 6.0, 1e-3)

    def rate(threads):
        rates, calls_total = [], 0
        for _ in range(3):
            calls, t0 = 0, time.perf_counter()
            while True:
                run_once(threads)
                calls += 1
                el = time.perf_counter() - t0
                if el >= per_run:
                    break
            rates.append(units_per_call * calls / el)
            calls_total += calls
        return float(np.median(rates)), calls_total

    v_all, c_all = rate(all_cores)
    v_one, c_one = rate(1)
    return {"value": v_all, "unit": unit, "cores": all_cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{sample}; median of 3 runs of ~{per_run:.1f} s ({c_all} calls) on {all_cores} threads",
            "one_core": {"value": v_one, "unit": unit, "cores": 1,
                         "sample": f"median of 3 runs of ~{per_run:.1f} s ({c_one} calls) on 1 thread"}}


def roofline(per_kernel, kernel, alg_bytes, traffic):
    main_us = next((v for k, v in per_kernel.items() if k.endswith(":" + kernel)), None)
    if not main_us:
        return None
    achieved = alg_bytes / (main_us * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "algorithmic_bytes": alg_bytes, "avg_launch_us": round(main_us, 3)}


def source_sha(op: str = "verify") -> str:
    h = hashlib.sha256()
    for n in COUNTED[op]["sources"]:
        h.update((_CSRC / n).read_bytes())
    return h.hexdigest()


def run_verify(args, dev, hev):
    import torch
    import rejection_sampling_verify_02_amd as sv
    from rejection_sampling_verify_02_amd import workloads as wl

    cfg = wl.CONFIGS[args.config]
    B, G, V = cfg.B, cfg.G, cfg.V
    esz = 2 if cfg.dtype == "bf16" else 4
    greedy = cfg.temperature == 0
    rows = B * (G + 1) if greedy else B * (2 * G + 1)  # greedy reads no draft row
    alg_bytes = rows * V * esz  # one read of every logit the result depends on
    n_sets = args.sets or max(2, -(-(1 << 30) // alg_bytes))
    log(f"[bench] workload {cfg.name}: B={B} G={G} V={V} {cfg.dtype}, {alg_bytes / 1e6:.2f} MB per call, "
        f"{n_sets} input sets")
    sets, host = make_sets(args.config, n_sets, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    dtc = sv.SV_BF16 if cfg.dtype == "bf16" else sv.SV_F32
    plan = sv.sv_launch_plan(B, G, V, dtc, cfg.temperature, cfg.top_k)
    ws = sv.Workspace()
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=dev)

    def call(i, events=None):
        s = sets[i % n_sets]
        return sv.spec_verify(s["target"], s["draft"], s["tokens"], s["u_accept"], s["u_sample"],
                              cfg.temperature, cfg.top_k, workspace=ws, stream=stream,
                              out=(acc, out), events=events)

    K = args.steps
    t = time_loop(call, plan, K, args.warmup, stream, dev, hev, not args.no_stage_events, args.flush_calls)
    wall, per_kernel = t["wall"], t["per_kernel"]
    # emitted tokens for the last call of each set (accepted + 1 per valid sequence)
    emitted = torch.zeros((), dtype=torch.int64, device=dev)
    for s_i in range(min(n_sets, K)):
        call(s_i)
        emitted += (acc.clamp(min=-1) + 1).sum()
    torch.cuda.synchronize(dev)
    mean_emitted = float(emitted.item()) / min(n_sets, K)

    ms = wall * 1e3 / K
    t_call = ms / 1e3
    # the kernel that streams the logits: with the one-pass top-k threshold that is its
    # select pass (the verification then reads only chunks without a complete list)
    kernel = "k_argmax" if greedy else ("k_topk_select" if "k_topk_select" in plan else KERNEL)
    traffic, tnote = counters_traffic("verify") if args.config == 3 else (None, "counters are taken on workload 3")
    res = {
        "metric": METRIC, "value": round(B * G / t_call, 1), "unit": "positions/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "G": G, "V": V, "logits": cfg.dtype,
                   "temperature": cfg.temperature, "top_k": cfg.top_k, "input_sets": n_sets,
                   "set_bytes": alg_bytes},
        "call_GBs": round(alg_bytes / t_call / 1e9, 1),
        "call_frac_of_peak": round(alg_bytes / t_call / 1e9 / PEAK_HBM_GBS, 4),
        "emitted_tokens_per_s": round(mean_emitted / t_call, 1),
        "mean_accepted_plus_one": round(mean_emitted / B, 4),
        **timing_fields(t, K, args.warmup),
        "roofline": roofline(per_kernel, kernel, alg_bytes, traffic),
        "traffic_note": tnote,
    }
    if not args.no_probe:
        probe = read_probe(alg_bytes, n_sets, K, dev, hev)
        res["read_probe"] = probe
        if res["roofline"]:
            res["roofline"]["frac_of_read_probe"] = round(res["roofline"]["achieved"] / probe["GBs"], 4)
    if not args.no_cpu_baseline:
        log(f"[bench] oracle CPU baseline (~{args.cpu_seconds:.0f} s)")
        res["cpu_baseline"] = cpu_baseline(host, cfg, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    return res


def run_sample(args, dev, hev):
    """The batched sampler on one decode step of B rows: tokens drawn per second."""
    import torch
    import rejection_sampling_verify_02_amd as sv
    from rejection_sampling_verify_02_amd import workloads as wl

    cfg = wl.SAMPLE_CONFIGS["sample_bf16_b256"]
    B, V = cfg.B, cfg.V
    esz = 2 if cfg.dtype == "bf16" else 4
    alg_bytes = B * V * esz
    n_sets = args.sets or max(2, -(-(1 << 30) // alg_bytes))
    log(f"[bench] sampler {cfg.name}: B={B} V={V} {cfg.dtype}, {alg_bytes / 1e6:.2f} MB per call, {n_sets} sets")
    sets, host = [], []
    for s in range(n_sets):
        z, u = wl.make_sample(B, V, cfg.dtype, cfg.seed + 1000 * s)
        t = torch.from_numpy(z)
        sets.append((t.view(torch.bfloat16).to(dev) if z.dtype == np.uint16 else t.to(dev),
                     torch.from_numpy(u).to(dev)))
        host.append((z, u))
    stream = torch.cuda.current_stream(dev).cuda_stream
    dtc = sv.SV_BF16 if cfg.dtype == "bf16" else sv.SV_F32
    plan = sv.sv_launch_plan(B, 0, V, dtc, cfg.temperature, cfg.top_k)
    ws = sv.Workspace()
    tok = torch.empty((B,), dtype=torch.int32, device=dev)
    st = torch.empty((B,), dtype=torch.int32, device=dev)

    def call(i, events=None):
        z, u = sets[i % n_sets]
        return sv.spec_sample(z, u, cfg.temperature, cfg.top_k, workspace=ws, stream=stream,
                              out=(tok, st), events=events)

    K = args.steps
    t = time_loop(call, plan, K, args.warmup, stream, dev, hev, not args.no_stage_events, args.flush_calls)
    wall, per_kernel = t["wall"], t["per_kernel"]
    t_call = wall / K
    res = {
        "metric": "sampled tokens/sec and achieved HBM GB/s (% of peak), one draw per row",
        "value": round(B / t_call, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(t_call * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "V": V, "logits": cfg.dtype, "temperature": cfg.temperature,
                   "top_k": cfg.top_k, "input_sets": n_sets, "set_bytes": alg_bytes},
        "call_GBs": round(alg_bytes / t_call / 1e9, 1),
        "call_frac_of_peak": round(alg_bytes / t_call / 1e9 / PEAK_HBM_GBS, 4),
        **timing_fields(t, K, args.warmup),
        "roofline": roofline(per_kernel, KERNEL, alg_bytes, counters_traffic("sample")[0]),
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle._load()
        st = {"i": 0}

        def once(threads):
            z, u = host[st["i"] % len(host)]
            st["i"] += 1
            oracle.sample_rows(z, u, cfg.temperature, cfg.top_k, nthreads=threads)

        res["cpu_baseline"] = oracle_baseline(once, B, "tokens/s", args.cpu_seconds,
                                              f"full calls (B={B}, V={V}) over {len(host)} input sets")
    else:
        res["cpu_baseline"] = None
    return res


def run_overlap(args, dev, hev):
    """beta and tv of every drafted position of the batch B=64, G=4, V=128256
    bf16 (T=1), in the verification layout: positions per second."""
    import torch
    import rejection_sampling_verify_02_amd as sv
    from rejection_sampling_verify_02_amd import workloads as wl
    import oracle

    cfg = wl.CONFIGS[3]
    B, G, V = cfg.B, cfg.G, cfg.V
    esz = 2 if cfg.dtype == "bf16" else 4
    alg_bytes = 2 * B * G * V * esz  # one read of target row i and draft row i per position
    n_sets = args.sets or max(2, -(-(1 << 30) // alg_bytes))
    log(f"[bench] overlap on {cfg.name}: B={B} G={G} V={V} {cfg.dtype}, {alg_bytes / 1e6:.2f} MB per call, "
        f"{n_sets} input sets")
    sets, host = [], []
    for s in range(n_sets):
        target, draft = wl.zipf_gauss(B, G, V, cfg.dtype, cfg.draft_noise, cfg.seed + 1000 * s)
        conv = (lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)) if cfg.dtype == "bf16" \
            else (lambda a: torch.from_numpy(a).to(dev))
        sets.append((conv(target), conv(draft)))
        host.append((target, draft))
    stream = torch.cuda.current_stream(dev).cuda_stream
    dtc = sv.SV_BF16 if cfg.dtype == "bf16" else sv.SV_F32
    plan = sv.sv_overlap_launch_plan(B, G, V, dtc, cfg.temperature, cfg.top_k)
    ws = sv.Workspace()
    outs = (torch.empty((B, G), dtype=torch.float64, device=dev),
            torch.empty((B, G), dtype=torch.float64, device=dev),
            torch.empty((B, G), dtype=torch.int32, device=dev))

    def call(i, events=None):
        t, d = sets[i % n_sets]
        return sv.spec_overlap(t, d, cfg.temperature, cfg.top_k, workspace=ws, stream=stream, out=outs,
                               events=events)

    K = args.steps
    t = time_loop(call, plan, K, args.warmup, stream, dev, hev, not args.no_stage_events, args.flush_calls)
    wall, per_kernel = t["wall"], t["per_kernel"]
    t_call = wall / K
    res = {
        "metric": "overlap (beta, tv) positions/sec and achieved HBM GB/s (% of peak) at B=64,V=128k",
        "value": round(B * G / t_call, 1), "unit": "positions/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(t_call * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "overlap_" + cfg.name, "B": B, "G": G, "V": V, "logits": cfg.dtype,
                   "temperature": cfg.temperature, "top_k": cfg.top_k, "input_sets": n_sets,
                   "set_bytes": alg_bytes},
        "call_GBs": round(alg_bytes / t_call / 1e9, 1),
        "call_frac_of_peak": round(alg_bytes / t_call / 1e9 / PEAK_HBM_GBS, 4),
        "mean_beta": round(float(outs[0].mean().item()), 5),
        **timing_fields(t, K, args.warmup),
        "roofline": roofline(per_kernel, "k_overlap", alg_bytes, counters_traffic("overlap")[0]),
    }
    if not args.no_cpu_baseline:
        oracle._load()
        st = {"i": 0}

        def once(threads):
            t_, d_ = host[st["i"] % len(host)]
            st["i"] += 1
            oracle.overlap(t_, d_, cfg.temperature, cfg.top_k, nthreads=threads)

        res["cpu_baseline"] = oracle_baseline(once, B * G, "positions/s", args.cpu_seconds,
                                              f"full calls (B={B}, G={G}, V={V}) over {len(host)} input sets")
    else:
        res["cpu_baseline"] = None
    return res


def run_tree(args, dev, hev):
    """Verification of a batch of draft trees: drafted nodes verified per second."""
    import torch
    import rejection_sampling_verify_02_amd as sv
    from rejection_sampling_verify_02_amd import workloads as wl

    cfg = wl.TREE_CONFIGS["tree_bf16_b16_n32"]
    B, N, V, S = cfg.B, cfg.N, cfg.V, cfg.max_children
    esz = 2 if cfg.dtype == "bf16" else 4
    set_bytes = 2 * B * N * V * esz
    n_sets = args.sets or max(2, -(-(1 << 30) // set_bytes))
    log(f"[bench] trees {cfg.name}: B={B} N={N} V={V} {cfg.dtype}, max children {S}, {n_sets} input sets")
    conv = (lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)) if cfg.dtype == "bf16" \
        else (lambda a: torch.from_numpy(a).to(dev))
    sets, host, alg = [], [], []
    for s in range(n_sets):
        raw = wl.make_tree(B, N, V, cfg.dtype, cfg.seed + 1000 * s, max_children=S, draft_noise=cfg.draft_noise)
        t, d = conv(raw.target), conv(raw.draft)
        par = torch.from_numpy(raw.parent).to(dev)
        # node tokens drawn from the parent's draft distribution by the library's sampler
        rows = d[torch.arange(B, device=dev)[:, None], par[:, 1:].long()].reshape(B * (N - 1), V).contiguous()
        tk, st = sv.spec_sample(rows, torch.from_numpy(raw.u_draft[:, 1:].reshape(-1).copy()).to(dev),
                                cfg.temperature, cfg.top_k)
        tok = torch.zeros((B, N), dtype=torch.int32, device=dev)
        tok[:, 1:] = tk.reshape(B, N - 1)
        sets.append((t, d, tok, par, torch.from_numpy(raw.u_accept).to(dev), torch.from_numpy(raw.u_sample).to(dev)))
        host.append((raw, tok.cpu().numpy()))
        internal = sum(len(set(raw.parent[b, 1:].tolist())) for b in range(B))
        alg.append((B * N + internal) * V * esz)  # every target row, and the draft rows of nodes with children
    torch.cuda.synchronize(dev)
    alg_bytes = int(np.mean(alg))
    stream = torch.cuda.current_stream(dev).cuda_stream
    dtc = sv.SV_BF16 if cfg.dtype == "bf16" else sv.SV_F32
    plan = sv.sv_tree_launch_plan(B, N, V, S, dtc, cfg.temperature, cfg.top_k)
    ws = sv.Workspace()
    outs = (torch.empty((B,), dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev),
            torch.empty((B, N), dtype=torch.int32, device=dev))

    def call(i, events=None):
        t, d, tok, par, ua, us = sets[i % n_sets]
        return sv.spec_tree_verify(t, d, tok, par, ua, us, cfg.temperature, cfg.top_k, max_children=S,
                                   workspace=ws, stream=stream, out=outs, events=events)

    K = args.steps
    t = time_loop(call, plan, K, args.warmup, stream, dev, hev, not args.no_stage_events, args.flush_calls)
    wall, per_kernel = t["wall"], t["per_kernel"]
    t_call = wall / K
    depth = []
    for i in range(n_sets):
        call(i)
        depth.append(float(outs[0].float().mean().item()))
    res = {
        "metric": "verified draft-tree nodes/sec and achieved HBM GB/s (% of peak)",
        "value": round(B * (N - 1) / t_call, 1), "unit": "nodes/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(t_call * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "N": N, "V": V, "logits": cfg.dtype, "max_children": S,
                   "temperature": cfg.temperature, "top_k": cfg.top_k, "input_sets": n_sets,
                   "set_bytes": set_bytes, "algorithmic_bytes": alg_bytes},
        "call_GBs": round(alg_bytes / t_call / 1e9, 1),
        "call_frac_of_peak": round(alg_bytes / t_call / 1e9 / PEAK_HBM_GBS, 4),
        "emitted_tokens_per_s": round(B * (float(np.mean(depth)) + 1) / t_call, 1),
        "mean_accepted_depth": round(float(np.mean(depth)), 4),
        **timing_fields(t, K, args.warmup),
        "roofline": roofline(per_kernel, "k_tree_rows", alg_bytes, counters_traffic("tree")[0]),
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle._load()
        st = {"i": 0}

        def once(threads):
            raw, tok = host[st["i"] % len(host)]
            st["i"] += 1
            oracle.tree_verify(raw.target, raw.draft, tok, raw.parent, raw.u_accept, raw.u_sample,
                               cfg.temperature, cfg.top_k, nthreads=threads)

        res["cpu_baseline"] = oracle_baseline(once, B * (N - 1), "nodes/s", args.cpu_seconds,
                                              f"full calls (B={B}, N={N}, V={V}) over {len(host)} input sets")
    else:
        res["cpu_baseline"] = None
    return res


def run_typical(args, dev, hev):
    """Typical acceptance of the batch B=64, G=4, V=128256 bf16 (T=1, eps = 0.1,
    delta = 0.3): positions per second."""
    import torch
    import rejection_sampling_verify_02_amd as sv
    from rejection_sampling_verify_02_amd import workloads as wl

    cfg = wl.CONFIGS[3]
    B, G, V = cfg.B, cfg.G, cfg.V
    eps, delta = 0.1, 0.3
    esz = 2 if cfg.dtype == "bf16" else 4
    alg_bytes = B * (G + 1) * V * esz  # one read of every target row
    n_sets = args.sets or max(2, -(-(1 << 30) // alg_bytes))
    log(f"[bench] typical acceptance on {cfg.name}: {alg_bytes / 1e6:.2f} MB per call, {n_sets} input sets")
    sets, host = make_sets(3, n_sets, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    dtc = sv.SV_BF16 if cfg.dtype == "bf16" else sv.SV_F32
    plan = sv.sv_typical_launch_plan(B, G, V, dtc, cfg.temperature, cfg.top_k)
    ws = sv.Workspace()
    outs = (torch.empty((B,), dtype=torch.int32, device=dev), torch.empty((B, G + 1), dtype=torch.int32, device=dev))

    def call(i, events=None):
        s = sets[i % n_sets]
        return sv.spec_typical_verify(s["target"], s["tokens"], cfg.temperature, eps, delta, cfg.top_k,
                                      workspace=ws, stream=stream, out=outs, events=events)

    K = args.steps
    t = time_loop(call, plan, K, args.warmup, stream, dev, hev, not args.no_stage_events, args.flush_calls)
    wall, per_kernel = t["wall"], t["per_kernel"]
    t_call = wall / K
    acc = []
    for i in range(min(n_sets, 8)):
        call(i)
        acc.append(float(outs[0].float().mean().item()))
    res = {
        "metric": "typical-acceptance positions/sec and achieved HBM GB/s (% of peak) at B=64,V=128k",
        "value": round(B * G / t_call, 1), "unit": "positions/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(t_call * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "typical_" + cfg.name, "B": B, "G": G, "V": V, "logits": cfg.dtype,
                   "temperature": cfg.temperature, "top_k": cfg.top_k, "epsilon": eps, "delta": delta,
                   "input_sets": n_sets, "set_bytes": alg_bytes},
        "call_GBs": round(alg_bytes / t_call / 1e9, 1),
        "call_frac_of_peak": round(alg_bytes / t_call / 1e9 / PEAK_HBM_GBS, 4),
        "mean_accepted": round(float(np.mean(acc)), 4),
        **timing_fields(t, K, args.warmup),
        "roofline": roofline(per_kernel, "k_typical", alg_bytes, counters_traffic("typical")[0]),
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle._load()
        st = {"i": 0}

        def once(threads):
            h = host[st["i"] % len(host)]
            st["i"] += 1
            oracle.typical_verify(h["target"], h["tokens"], cfg.temperature, eps, delta, cfg.top_k, nthreads=threads)

        res["cpu_baseline"] = oracle_baseline(once, B * G, "positions/s", args.cpu_seconds,
                                              f"full calls (B={B}, G={G}, V={V}) over {len(host)} input sets")
    else:
        res["cpu_baseline"] = None
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--op", default="verify", choices=["verify", "sample", "overlap", "tree", "typical"],
                    help="verify (the default: B=64, G=4, V=128256 bf16), the batched sampler, the per-position overlap, "
                         "tree verification, or typical acceptance")
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5],
                    help="verification workload (3, the default, is B=64, G=4, V=128256 bf16; 4 greedy and 5 top-k "
                         "are timed for the design notes)")
    ap.add_argument("--sets", type=int, default=0, help="input sets to rotate (default: >= 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="wall time of the oracle baseline (half on every core, half on one core)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--flush-calls", type=int, default=20,
                    help="single calls timed after a 1 GiB flush each (0: none)")
    ap.add_argument("--no-stage-events", action="store_true",
                    help="time the loop without per-kernel events")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("BENCH_DIR", "COPY_DIR"),
                    help="write the traffic summary of --op from rocprofv3 --pmc CSV directories")
    ap.add_argument("--timeline", action="store_true",
                    help="where a call's time goes, from the timeline build of the library (writes profiles/)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DIR", "LINE_FILE", "COMMAND"),
                    help="write the kernel-trace summary of a rocprofv3 --kernel-trace run of this "
                         "script (its output line in LINE_FILE; COMMAND is quoted in the summary)")
    ap.add_argument("--trace-reference", metavar="LINE_FILE",
                    help="with --summarize-trace: the line of the same command run without the profiler")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU; spec_verify has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2
    if args.copy_probe:
        copy_probe(args.copy_probe, 10)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.op)
        return 0
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, ref_file=args.trace_reference)
        return 0

    import torch
    import rejection_sampling_verify_02_amd as sv

    if args.timeline:
        print(json.dumps(run_timeline(args, torch.device("cuda:0"))), flush=True)
        return 0
    sv.load_library()  # raises if the HIP library is not built
    dev = torch.device("cuda:0")
    hev = HipEvents()
    run = {"sample": run_sample, "overlap": run_overlap, "tree": run_tree,
           "typical": run_typical}.get(args.op, run_verify)
    res = run(args, dev, hev)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
