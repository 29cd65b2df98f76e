#!/usr/bin/env python3
"""Throughput of the LoRA-linear training step on one MI355X.

One step = one optimizer update of every adapter slot: for each of the G
accumulation chunks, forward and backward of every adapted linear (all
layers, all projections; the layers' calls spread over `--streams` HIP
streams), then gradient preparation, AdamW and (DoRA) the row-norm refresh.  Inputs are seeded synthetic tensors already resident in
HBM; the timed region contains exactly `--steps` updates.

Prints one JSON line: tokens/s for the whole job, the roofline position of
the kernel that takes most of the time (its average duration measured with
HIP events on its launch stream during a second, instrumented pass of the
same steps), a per-kernel breakdown, and the CPU oracle timed on a bounded
sample of the same workload on this host.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA-linear fwd+bwd+step tokens/sec; % MFMA peak (GEMM), % HBM peak (rest)"
PEAK = {"hbm": 8000.0, "f32": 157.3, "bf16": 2516.6}   # GB/s; TFLOP/s dense MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Block-quantized frozen W for the bf16 workloads: one format for every
# projection, or "q4_k_m", a mix in the manner of the pages' Q4_K_M base
# (wv and wdown in Q6_K, the other projections in Q4_K).
W_FORMATS = ("q8_0", "q4_0", "q4_k", "q6_k", "q4_k_m")


def projection_format(w_format, proj):
    if w_format == "q4_k_m":
        return "q6_k" if proj.name in ("wv", "wdown") else "q4_k"
    return w_format


def build_workload(cfg, device, layers=None, tokens=None, chunks=None, streams=4):
    """Frozen model, slots and per-slot chunk inputs, all seeded.  A
    workload whose w_dtype names a block-quantized format gets W drawn as
    that format's planes."""
    import torch
    from bwd_adamw_amd import lora as L
    from bwd_adamw_amd import step as S
    from bwd_adamw_amd import workloads as WL

    layers = cfg.layers if layers is None else layers
    T = cfg.tokens if tokens is None else tokens
    G = cfg.chunks if chunks is None else chunks
    Wq = {}
    for l in range(layers):
        for pj in cfg.projections:
            if cfg.w_dtype in W_FORMATS:
                fmt = projection_format(cfg.w_dtype, pj)
                planes = WL.qweight_planes(fmt, pj.out_dim, pj.in_dim,
                                           (cfg.number, 0, l, pj.ordinal), device=device)
                Wq[(l, pj.ordinal)] = L.qweight_pack(fmt, pj.out_dim, pj.in_dim, planes, device)
                continue
            inp = WL.linear_inputs(cfg, l, pj, chunks=0, tokens=T, device=device)
            Wq[(l, pj.ordinal)] = inp.get("W_bf16", inp["W"])
    model = S.FrozenModel(cfg, Wq)
    trainer = S.Trainer(cfg, model, tokens=T, device=device, slots=cfg.slots, streams=streams)
    slots, inputs = [], []
    for si in range(cfg.slots):
        A, B = {}, {}
        chunk_list = [dict() for _ in range(G)]
        xcache = {}
        for l in range(layers):
            for pj in cfg.projections:
                key = (l, pj.ordinal)
                n = cfg.number
                A[key] = WL.draw((cfg.rank, pj.in_dim), (n, si, l, pj.ordinal, 0, "A"), "uniform",
                                 1.0 / pj.in_dim ** 0.5, device)
                B[key] = WL.draw((pj.out_dim, cfg.rank), (n, si, l, pj.ordinal, 0, "B"), "normal",
                                 cfg.b_std, device)
                for g in range(G):
                    xk = (l, pj.x_group, g)
                    if xk not in xcache:
                        xcache[xk] = WL.draw((T, pj.in_dim), (n, si, l, 100 + pj.x_group, g, "X"),
                                             "normal", cfg.x_std, device)
                    dY = WL.draw((T, pj.out_dim), (n, si, l, pj.ordinal, g, "dY"), "normal",
                                 cfg.dy_std, device)
                    chunk_list[g][key] = (xcache[xk], dY)
        slot = S.Slot(cfg, model, A, B, cfg.seeds[si], device=device)
        if cfg.dora:
            trainer.init_dora(slot)
        slots.append(slot)
        inputs.append(chunk_list)
    return model, trainer, slots, inputs


def run_steps(trainer, slots, inputs, n):
    for _ in range(n):
        for st in trainer.step_slots(slots, inputs):
            if st.vetoed:
                raise RuntimeError("non-finite gradient in a synthetic run")


TRAFFIC_FILE = os.path.join(ROOT, "bwd_adamw_amd", "traffic.json")


def kernel_source_digest():
    """SHA-256 over the HIP sources; stored counter readings are valid only
    for the kernels they were taken from."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "bwd_adamw_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(src, name), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel, shape):
    """HBM bytes per launch of (kernel, shape) from the stored FETCH_SIZE and
    WRITE_SIZE readings, each scaled by the factor a plain copy of known size
    gave for the same counter; None when absent or taken on other sources."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_digest():
        return None
    k = rec.get("kernels", {}).get(f"{kernel} {shape[0]}x{shape[1]}x{shape[2]}")
    if not k:
        return None
    return k["fetch_kib"] * 1024.0 * rec["copy_factor_fetch"] + \
        k["write_kib"] * 1024.0 * rec["copy_factor_write"]


def copy_calibration(mib):
    """A plain device copy of `mib` MiB, five times: the reference dispatch
    whose FETCH_SIZE / WRITE_SIZE readings convert the counters to bytes."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n,
                                           "dispatches": 5}}), flush=True)


def stream_copy_gbps(mib=1024, reps=5):
    """Bytes moved (read + write) per second by a plain device copy of `mib`
    MiB: the attainable HBM rate reported beside the published peak."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbps = 2.0 * 4 * n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return gbps


def roofline_of(entries, cfg):
    """Dominant kernel (largest summed time) and its place on the roofline."""
    dom = max(entries, key=lambda e: e["total_ms"])
    sec = dom["avg_ms"] / 1e3
    if dom["kernel"].startswith("gemm"):
        peak = PEAK["f32" if "f32" in dom["kernel"] else "bf16"]
        achieved = dom["flops"] / sec / 1e12
        rl = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s"}
    else:
        achieved = dom["bytes"] / sec / 1e9
        rl = {"bound": "hbm", "achieved": achieved, "peak": PEAK["hbm"], "unit": "GB/s"}
    rl["frac"] = rl["achieved"] / rl["peak"]
    rl["traffic"] = measured_traffic(dom["kernel"], [dom["M"], dom["N"], dom["K"]])
    rl["kernel"] = dom["kernel"]
    rl["shape"] = [dom["M"], dom["N"], dom["K"]]
    rl["avg_us"] = dom["avg_ms"] * 1e3
    rl["launches"] = dom["launches"]
    return rl


def kernel_table(entries, total_ms):
    rows = []
    for e in sorted(entries, key=lambda e: -e["total_ms"])[:16]:
        sec = e["avg_ms"] / 1e3
        row = {"kernel": e["kernel"], "shape": [e["M"], e["N"], e["K"]], "launches": e["launches"],
               "avg_us": round(e["avg_ms"] * 1e3, 3), "share": round(e["total_ms"] / total_ms, 4)}
        if e["kernel"].startswith("gemm"):
            peak = PEAK["f32" if "f32" in e["kernel"] else "bf16"]
            row["tflops"] = round(e["flops"] / sec / 1e12, 2)
            row["frac_mfma"] = round(e["flops"] / sec / 1e12 / peak, 4)
        else:
            row["gbps"] = round(e["bytes"] / sec / 1e9, 1)
            row["frac_hbm"] = round(e["bytes"] / sec / 1e9 / PEAK["hbm"], 4)
        rows.append(row)
    return rows


def per_label_ms(entries, steps):
    """Kernel time per step of each launch label (all shapes together),
    largest first."""
    tot = {}
    for e in entries:
        tot[e["kernel"]] = tot.get(e["kernel"], 0.0) + e["total_ms"] / steps
    return {k: round(v, 3) for k, v in sorted(tot.items(), key=lambda kv: -kv[1])}


def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(cfg, budget_s, threads=None):
    """The oracle's whole step on a bounded sample: the full per-layer step
    (all projections, all G chunks, one slot) layer after layer, wrapping
    round to layer 0 again, until about `budget_s` of work; the per-layer
    time is scaled to the whole workload (extrapolated when the sample is
    not the whole step).  threads: BLAS thread limit (None = all)."""
    if threads is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=int(threads)):
            return cpu_baseline(cfg, budget_s)
    import numpy as np
    import oracle as O
    from bwd_adamw_amd import workloads as WL
    cores = blas_threads()
    s = O.scaling(cfg.alpha, cfg.rank, cfg.scaling)
    f64 = lambda t: t.double().numpy()
    def layer_inputs(l):
        lin, params, chunks = {}, {}, [dict() for _ in range(cfg.chunks)]
        for pj in cfg.projections:
            inp = WL.linear_inputs(cfg, l, pj)
            key = (l, pj.ordinal)
            if cfg.w_dtype in W_FORMATS:
                from oracle import quant as Q
                fmt = projection_format(cfg.w_dtype, pj)
                planes = WL.qweight_planes(fmt, pj.out_dim, pj.in_dim, (cfg.number, 0, l, pj.ordinal))
                lin[key] = Q.dequantize(fmt, {k: v.numpy() for k, v in planes.items()})
            else:
                lin[key] = f64(inp["W"])
            params[key] = {"A": f64(inp["A"]), "B": f64(inp["B"])}
            if cfg.dora:
                params[key]["mag"] = O.dora_row_norms(lin[key])
            for g in range(cfg.chunks):
                chunks[g][key] = (f64(inp["X"][g]), f64(inp["dY"][g]))
        return lin, params, chunks

    # Layers are generated once and kept while they fit in about 2 GB; the
    # timed loop then cycles over the kept layers.
    cache, cache_bytes = [], 0
    elapsed_total, layers_done = 0.0, 0
    while elapsed_total < budget_s:
        l = layers_done % cfg.layers
        if l < len(cache):
            lin, params0, chunks = cache[l]
        elif cache_bytes < 2e9 or not cache:
            lin, params0, chunks = layer_inputs(l)
            cache.append((lin, params0, chunks))
            cache_bytes += sum(w.nbytes for w in lin.values()) + \
                sum(x.nbytes + d.nbytes for c in chunks for x, d in c.values())
        else:
            lin, params0, chunks = cache[layers_done % len(cache)]
        params = {k: {n: a.copy() for n, a in v.items()} for k, v in params0.items()}
        st = O.SlotState(params=params)
        if cfg.dora:
            for key in lin:
                st.norms[key] = O.dora_row_norms(lin[key], params[key]["A"], params[key]["B"], s)
        hp = dict(s=s, p=cfg.dropout, seed=cfg.seeds[0], n_pred=cfg.tokens * cfg.chunks,
                  max_norm=cfg.max_norm, lr=cfg.lr, weight_decay=cfg.weight_decay,
                  plus_ratio=cfg.plus_ratio, dora=cfg.dora)
        t0 = time.perf_counter()
        O.train_step(st, lin, chunks, hp)
        elapsed_total += time.perf_counter() - t0
        layers_done += 1
    # whole-step time of the full workload, scaled from the sampled layers
    step_s = elapsed_total / layers_done * cfg.layers * cfg.slots
    value = cfg.tokens_per_step / step_s
    whole = layers_done >= cfg.layers and cfg.slots == 1
    sample = (f"oracle train_step, one layer at a time (all projections, {cfg.chunks} chunk(s) of "
              f"{cfg.tokens} tokens, slot 0): {layers_done} layer-steps over the {cfg.layers} "
              f"layers in {elapsed_total:.1f} s, scaled to the full {cfg.layers}-layer x "
              f"{cfg.slots}-slot step")
    return {"value": value, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "extrapolated": not whole, "cpu_model": cpu_model(),
            "workload": cfg.name}


# ---------------------------------------------------------------------------
# Summaries of rocprofv3 CSV output (no GPU needed): the tables committed
# under profiles/ are printed by these, from the directory a run wrote.
def _rocprof_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _field(row, name):
    if name in row:
        return row[name]
    for k, v in row.items():
        if k.lower() == name.lower():
            return v
    raise KeyError(name)


def _short(name, width=110):
    return name if len(name) <= width else name[:width - 3] + "..."


def summarize_trace(directory, top=30):
    """Kernel-trace table: dispatches grouped by kernel, grid (workgroups)
    and workgroup size, with durations from the trace's timestamps (ns)."""
    groups = {}
    for r in _rocprof_rows(directory, "kernel_trace.csv"):
        wgs = [int(_field(r, f"Workgroup_Size_{a}")) for a in "XYZ"]
        grid = [int(_field(r, f"Grid_Size_{a}")) for a in "XYZ"]
        blocks = "x".join(str(g // max(w, 1)) for g, w in zip(grid, wgs))
        key = (_field(r, "Kernel_Name"), blocks, wgs[0] * wgs[1] * wgs[2])
        dur = (int(_field(r, "End_Timestamp")) - int(_field(r, "Start_Timestamp"))) / 1e3
        groups.setdefault(key, []).append(dur)
    total = sum(sum(v) for v in groups.values()) or 1.0
    out = ["| kernel | grid | threads | calls | total ms | avg us | min us | max us | % |",
           "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (name, blocks, nt), d in sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]:
        out.append(f"| `{_short(name)}` | {blocks} | {nt} | {len(d)} | {sum(d) / 1e3:.3f} | "
                   f"{sum(d) / len(d):.2f} | {min(d):.2f} | {max(d):.2f} | "
                   f"{100.0 * sum(d) / total:.2f} |")
    return "\n".join(out)


def summarize_pmc(directory, top=30):
    """Counter table: per (kernel, grid threads), each counter's value per
    dispatch (summed over a dispatch's rows, averaged over dispatches)."""
    per_dispatch = {}
    for r in _rocprof_rows(directory, "counter_collection.csv"):
        key = (_field(r, "Kernel_Name"), int(_field(r, "Grid_Size")))
        d = per_dispatch.setdefault(key, {}).setdefault(_field(r, "Dispatch_Id"), {})
        c = _field(r, "Counter_Name")
        d[c] = d.get(c, 0.0) + float(_field(r, "Counter_Value"))
    counters = sorted({c for disp in per_dispatch.values() for d in disp.values() for c in d})
    out = ["| kernel | grid threads | dispatches | " + " | ".join(counters) + " |",
           "|---|---:|---:|" + "---:|" * len(counters)]
    rank = sorted(per_dispatch.items(),
                  key=lambda kv: -sum(sum(d.values()) for d in kv[1].values()))
    for (name, grid), disp in rank[:top]:
        means = [sum(d.get(c, 0.0) for d in disp.values()) / len(disp) for c in counters]
        out.append(f"| `{_short(name)}` | {grid} | {len(disp)} | " +
                   " | ".join(f"{m:.1f}" for m in means) + " |")
    return "\n".join(out)


def frozen_flops_per_step(cfg):
    """Algorithmic flops of the frozen products in one step: forward and dX,
    2*T*N*K each, for every linear, chunk and slot."""
    per_token = sum(2 * 2 * p.in_dim * p.out_dim for p in cfg.projections) * cfg.layers
    return per_token * cfg.tokens_per_step


def one_stream(trainer):
    """Context: the trainer's calls all on the current stream (its side
    streams and their workspaces set aside), for the instrumented pass."""
    import contextlib

    @contextlib.contextmanager
    def ctx():
        side, side_ws = trainer.side, trainer.side_ws
        trainer.side, trainer.side_ws = [], []
        try:
            yield
        finally:
            trainer.side, trainer.side_ws = side, side_ws
    return ctx()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5,
                    help="workload number (default 5: DoRA on the Qwen3-4B-shaped all-linear "
                         "layers, two slots, the largest single-GPU workload)")
    ap.add_argument("--w-format", choices=W_FORMATS, default=None,
                    help="block-quantized frozen W for a bf16 workload (default: its bf16 W)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--cpu-others", type=float, default=3.0,
                    help="seconds of oracle work per extra CPU figure (the small float32 "
                         "workloads at all threads and at one thread; 0 = skip)")
    ap.add_argument("--streams", type=int, default=4,
                    help="HIP streams the layers' calls are spread over in the timed pass "
                         "(default 4; at most one per layer group)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--no-profile-pass", action="store_true",
                    help="skip the instrumented pass (per-launch HIP events); the line then "
                         "has no roofline or kernel table (for counter-collection runs)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="only print the kernel-trace table of a rocprofv3 --kernel-trace "
                         "CSV run under DIR (no GPU)")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="only print the counter table of a rocprofv3 --pmc CSV run under DIR "
                         "(no GPU)")
    args = ap.parse_args()
    if args.summarize_trace or args.summarize_pmc:
        if args.summarize_trace:
            print(summarize_trace(args.summarize_trace))
        if args.summarize_pmc:
            print(summarize_pmc(args.summarize_pmc))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py: only --gpus 1 is supported (the path is built and measured on one GPU)")
        sys.exit(2)

    import torch
    from bwd_adamw_amd import lora as L
    from bwd_adamw_amd import workloads as WL

    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        sys.exit(1)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    L.lib()
    cfg = WL.get_config(args.config)
    if args.w_format:
        if cfg.w_dtype != "bf16":
            log("bench.py: --w-format applies to the bf16 workloads")
            sys.exit(2)
        import dataclasses
        cfg = dataclasses.replace(cfg, w_dtype=args.w_format,
                                  name=cfg.name.replace("-bf16-", f"-{args.w_format}-"))
    dev = "cuda"
    t0 = time.perf_counter()
    model, trainer, slots, inputs = build_workload(cfg, dev, streams=args.streams)
    torch.cuda.synchronize()
    log(f"setup {cfg.name}: {time.perf_counter() - t0:.1f} s")

    run_steps(trainer, slots, inputs, args.warmup)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(trainer, slots, inputs, args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3
    value = cfg.tokens_per_step * args.steps / elapsed
    log(f"timed {args.steps} steps on {1 + len(trainer.side)} stream(s): {ms:.3f} ms/step, "
        f"{value:.1f} tokens/s")

    if args.no_profile_pass:
        print(json.dumps({"metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
                          "higher_is_better": True, "config": {"workload": cfg.name,
                          "streams": 1 + len(trainer.side)}, "roofline": None}), flush=True)
        return
    # Instrumented pass over the same number of steps, every call on one
    # stream so that a launch's duration is its own and not shared with
    # other layers' launches: per-kernel HIP events on the launch stream.
    with one_stream(trainer):
        run_steps(trainer, slots, inputs, 1)
        torch.cuda.synchronize()
        L.lora_profile_begin(200000)
        t1 = time.perf_counter()
        run_steps(trainer, slots, inputs, args.steps)
        entries = L.lora_profile_end()
        prof_ms = (time.perf_counter() - t1) / args.steps * 1e3
    kernel_ms = sum(e["total_ms"] for e in entries) / args.steps
    log(f"profiled pass (one stream): {prof_ms:.3f} ms/step, kernel time {kernel_ms:.3f} ms/step")

    rl = roofline_of(entries, cfg)
    rl["streams"] = 1
    rl["stream_copy_gbps"] = stream_copy_gbps()
    # chip level: the frozen products' flops of a step over the timed step
    peak = PEAK["f32" if cfg.w_dtype == "f32" else "bf16"]
    fl = frozen_flops_per_step(cfg)
    rl["step"] = {"frozen_flops": fl, "achieved": fl / (ms * 1e-3) / 1e12, "peak": peak,
                  "unit": "TFLOP/s", "frac": fl / (ms * 1e-3) / 1e12 / peak}
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.w_dtype == "f32" else "bf16",
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {
            "workload": cfg.name, "layers": cfg.layers,
            "projections": [f"{p.name} {p.in_dim}->{p.out_dim}" for p in cfg.projections],
            "tokens_per_chunk": cfg.tokens, "chunks": cfg.chunks, "slots": cfg.slots,
            "tokens_per_step": cfg.tokens_per_step, "rank": cfg.rank, "w_dtype": cfg.w_dtype,
            "dropout": cfg.dropout, "dora": cfg.dora, "parallelism": "single GPU",
            "streams": 1 + len(trainer.side),
        },
        "roofline": rl,
        "kernels": {"streams": 1, "ms_per_step": prof_ms, "sum_kernel_ms_per_step": kernel_ms,
                    "table": kernel_table(entries, kernel_ms * args.steps),
                    "per_label_ms": per_label_ms(entries, args.steps)},
    }
    del model, trainer, slots, inputs
    torch.cuda.empty_cache()
    if args.cpu_budget > 0:
        t2 = time.perf_counter()
        cb = cpu_baseline(cfg, args.cpu_budget)
        if args.cpu_others > 0:
            # the small float32 workloads, at all threads and at one
            cb["others"] = []
            for n in (1, 2, 3):
                for th in (None, 1):
                    o = cpu_baseline(WL.get_config(n), args.cpu_others, threads=th)
                    cb["others"].append({k: o[k] for k in ("workload", "value", "unit", "cores",
                                                           "extrapolated")})
        out["cpu_baseline"] = cb
        log(f"cpu baseline: {time.perf_counter() - t2:.1f} s")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
