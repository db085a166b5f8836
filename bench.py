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
                   alg=147750912, sources=("spec_verify.hip",) + _SHARED),
    "overlap": dict(kernel="k_overlap", workload="overlap_zipf_bf16_b64", desc="B=64, G=4, V=128256, bf16",
                    alg=131334144, sources=("spec_overlap.hip",) + _SHARED),
    "sample": dict(kernel="k_verify", workload="sample_bf16_b256", desc="B=256, V=128256, bf16",
                   alg=65667072, sources=("spec_verify.hip",) + _SHARED),
    "tree": dict(kernel="k_tree_rows", workload="tree_bf16_b16_n32", desc="16 trees of 32 nodes, V=128256, bf16",
                 alg=210698956, sources=("spec_tree.hip", "sv_draw.h") + _SHARED),
    "typical": dict(kernel="k_typical", workload="typical_zipf_bf16_b64", desc="B=64, G=4, V=128256, bf16",
                    alg=82083840, sources=("spec_typical.hip",) + _SHARED),
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
    """The oracle (fp64, unmodified) on the host cores over whole input sets, for a bounded
    wall time; its value is verified positions per second like the GPU's."""
    import oracle

    oracle._load()
    threads = oracle.default_threads()
    calls, t0 = 0, time.perf_counter()
    while True:
        h = host_sets[calls % len(host_sets)]
        oracle.spec_verify_ref(h["target"], h["draft"], h["tokens"], h["u_accept"], h["u_sample"],
                               cfg.temperature, cfg.top_k, nthreads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    B, G = host_sets[0]["tokens"].shape
    return {"value": B * G * calls / el, "unit": "positions/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} full calls (B={B}, G={G}) over {min(calls, len(host_sets))} input sets, "
                      f"{el:.1f} s; the oracle stops reading each sequence at its first rejection"}


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
    print(json.dumps(res))


def copy_probe(nbytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").uniform_()
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


def time_loop(call, plan, K, warmup, stream, dev, hev, stage_events):
    """Warm-up, then K calls timed as a caller runs them (wall clock and stream events),
    then (unless disabled) the same K calls with a (start, stop) event pair on every kernel
    dispatch.  Returns (wall_s, gpu_ms, per_kernel_us, wall2_s)."""
    import torch
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize(dev)
    log(f"[bench] warmup done ({warmup} calls)")
    loop_ev = hev.create(2)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    hev.record(loop_ev[0], stream)
    for i in range(K):
        call(warmup + i)
    hev.record(loop_ev[1], stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    gpu_ms = hev.elapsed_ms(loop_ev[0], loop_ev[1])
    hev.destroy(loop_ev)
    log(f"[bench] timed {K} calls: wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms")
    # The per-dispatch event pairs add a few microseconds of gap between kernels, so the
    # first loop gives the throughput and this one each kernel's own duration.
    per_kernel, wall2 = {}, None
    if stage_events:
        nl = len(plan)
        stage = [hev.create(2 * nl) for _ in range(K)]
        torch.cuda.synchronize(dev)
        t1 = time.perf_counter()
        for i in range(K):
            call(warmup + i, stage[i])
        torch.cuda.synchronize(dev)
        wall2 = time.perf_counter() - t1
        durs = np.array([[hev.elapsed_ms(ev[2 * j], ev[2 * j + 1]) for j in range(nl)] for ev in stage])
        for j, name in enumerate(plan):
            per_kernel[f"{j}:{name}"] = float(np.mean(durs[:, j]) * 1e3)
        for ev in stage:
            hev.destroy(ev)
        log(f"[bench] timed {K} calls with per-kernel events: wall {wall2 * 1e3:.2f} ms")
    return wall, gpu_ms, per_kernel, wall2


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
    wall, gpu_ms, per_kernel, wall2 = time_loop(call, plan, K, args.warmup, stream, dev, hev,
                                                not args.no_stage_events)
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
        "gpu_event_ms_per_step": round(gpu_ms / K, 5),
        "per_kernel_us": {k: round(v, 3) for k, v in per_kernel.items()},
        "ms_per_step_with_kernel_events": None if wall2 is None else round(wall2 * 1e3 / K, 5),
        "roofline": roofline(per_kernel, kernel, alg_bytes, traffic),
        "traffic_note": tnote,
    }
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
    wall, gpu_ms, per_kernel, wall2 = time_loop(call, plan, K, args.warmup, stream, dev, hev,
                                                not args.no_stage_events)
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
        "gpu_event_ms_per_step": round(gpu_ms / K, 5),
        "per_kernel_us": {k: round(v, 3) for k, v in per_kernel.items()},
        "ms_per_step_with_kernel_events": None if wall2 is None else round(wall2 * 1e3 / K, 5),
        "roofline": roofline(per_kernel, KERNEL, alg_bytes, counters_traffic("sample")[0]),
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle._load()
        threads = oracle.default_threads()
        calls, t0 = 0, time.perf_counter()
        while True:
            z, u = host[calls % len(host)]
            oracle.sample_rows(z, u, cfg.temperature, cfg.top_k, nthreads=threads)
            calls += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": B * calls / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"{calls} full calls (B={B}, V={V}) over {min(calls, len(host))} "
                                         f"input sets, {el:.1f} s"}
    else:
        res["cpu_baseline"] = None
    return res


def run_overlap(args, dev, hev):
    """beta and tv of every drafted position of the headline batch (B=64, G=4, V=128256
    bf16, T=1), in the verification layout: positions per second."""
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
    wall, gpu_ms, per_kernel, wall2 = time_loop(call, plan, K, args.warmup, stream, dev, hev,
                                                not args.no_stage_events)
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
        "gpu_event_ms_per_step": round(gpu_ms / K, 5),
        "per_kernel_us": {k: round(v, 3) for k, v in per_kernel.items()},
        "ms_per_step_with_kernel_events": None if wall2 is None else round(wall2 * 1e3 / K, 5),
        "roofline": roofline(per_kernel, "k_overlap", alg_bytes, counters_traffic("overlap")[0]),
    }
    if not args.no_cpu_baseline:
        oracle._load()
        threads = oracle.default_threads()
        calls, t0 = 0, time.perf_counter()
        while True:
            t, d = host[calls % len(host)]
            oracle.overlap(t, d, cfg.temperature, cfg.top_k, nthreads=threads)
            calls += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": B * G * calls / el, "unit": "positions/s", "cores": threads,
                               "kind": "oracle", "sample": f"{calls} full calls (B={B}, G={G}, V={V}) over "
                                                           f"{min(calls, len(host))} input sets, {el:.1f} s"}
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
    wall, gpu_ms, per_kernel, wall2 = time_loop(call, plan, K, args.warmup, stream, dev, hev,
                                                not args.no_stage_events)
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
        "gpu_event_ms_per_step": round(gpu_ms / K, 5),
        "per_kernel_us": {k: round(v, 3) for k, v in per_kernel.items()},
        "ms_per_step_with_kernel_events": None if wall2 is None else round(wall2 * 1e3 / K, 5),
        "roofline": roofline(per_kernel, "k_tree_rows", alg_bytes, counters_traffic("tree")[0]),
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle._load()
        threads = oracle.default_threads()
        calls, t0 = 0, time.perf_counter()
        while True:
            raw, tok = host[calls % len(host)]
            oracle.tree_verify(raw.target, raw.draft, tok, raw.parent, raw.u_accept, raw.u_sample,
                               cfg.temperature, cfg.top_k, nthreads=threads)
            calls += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": B * (N - 1) * calls / el, "unit": "nodes/s", "cores": threads,
                               "kind": "oracle", "sample": f"{calls} full calls (B={B}, N={N}, V={V}) over "
                                                           f"{min(calls, len(host))} input sets, {el:.1f} s"}
    else:
        res["cpu_baseline"] = None
    return res


def run_typical(args, dev, hev):
    """Typical acceptance of the headline batch (B=64, G=4, V=128256 bf16, T=1, eps = 0.1,
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
    wall, gpu_ms, per_kernel, wall2 = time_loop(call, plan, K, args.warmup, stream, dev, hev,
                                                not args.no_stage_events)
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
        "gpu_event_ms_per_step": round(gpu_ms / K, 5),
        "per_kernel_us": {k: round(v, 3) for k, v in per_kernel.items()},
        "ms_per_step_with_kernel_events": None if wall2 is None else round(wall2 * 1e3 / K, 5),
        "roofline": roofline(per_kernel, "k_typical", alg_bytes, counters_traffic("typical")[0]),
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle._load()
        threads = oracle.default_threads()
        calls, t0 = 0, time.perf_counter()
        while True:
            h = host[calls % len(host)]
            oracle.typical_verify(h["target"], h["tokens"], cfg.temperature, eps, delta, cfg.top_k, nthreads=threads)
            calls += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": B * G * calls / el, "unit": "positions/s", "cores": threads,
                               "kind": "oracle", "sample": f"{calls} full calls (B={B}, G={G}, V={V}) over "
                                                           f"{min(calls, len(host))} input sets, {el:.1f} s"}
    else:
        res["cpu_baseline"] = None
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--op", default="verify", choices=["verify", "sample", "overlap", "tree", "typical"],
                    help="verify (the default, the headline), the batched sampler, the per-position overlap, "
                         "tree verification, or typical acceptance")
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5],
                    help="verification workload (3, the default, is the headline; 4 greedy and 5 top-k "
                         "are timed for the design notes)")
    ap.add_argument("--sets", type=int, default=0, help="input sets to rotate (default: >= 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stage-events", action="store_true",
                    help="time the loop without per-kernel events")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("BENCH_DIR", "COPY_DIR"),
                    help="write the traffic summary of --op from rocprofv3 --pmc CSV directories")
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

    import torch
    import rejection_sampling_verify_02_amd as sv

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
