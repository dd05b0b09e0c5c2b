#!/usr/bin/env python3
"""Benchmark: one step = the whole hot path over the 32-layer, 32K-context,
batch-4 Llama-3-8B-shaped workload with per-layer bounded budgets:

  window score (all layers, one call) -> top-B select (all layers, one call)
  -> gather-compact (all layers, one call) -> one decode step through all 32
  layers over the compacted caches (one call per layer), plus the host-side
  per-layer budget computation.  The same compression step issued one layer
  at a time is timed too and reported beside it.

Inputs are synthetic (seeded generator), resident in HBM before timing.  Each
phase is captured once as a HIP graph of the library's launches and replayed
between two HIP events, so per-layer stage times carry no host launch gaps;
the reported value is the decode attention's algorithmic HBM bandwidth.
Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "compacted decode-attn HBM GB/s (% peak) + select-and-compact µs/layer, 32K ctx"
COUNTERS = os.path.join(ROOT, "profiles", "decode_c2_counters.json")
CSRC = os.path.join(ROOT, "sparse_decode_attention_window_amd", "csrc")
DECODE_SRCS = [os.path.join(CSRC, f) for f in ("decode.hip", "kvsel_internal.h")]
DECODE_KERNELS = ("decode_split_kernel", "decode_combine_head_kernel")
COPY_BYTES = 1 << 30           # plain device copy used as HBM reference and counter calibration


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(paths) -> str:
    """Hash of the code in `paths`: comments, blank lines and trailing spaces
    are dropped first, so that only a change to the code itself marks the
    stored counters as stale."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def copy_reference(torch, reps: int = 5) -> float:
    """GB/s (read + write) of a plain 1 GiB device-to-device copy on this GPU."""
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) / reps * 1e-3
    del src, dst
    return 2 * COPY_BYTES / t / 1e9


def stream_ceiling(torch, probe, mode: int, moved: int, nb: int = 4, calls: int = 8) -> float:
    """GB/s of the benchmark's non-temporal HBM stream (libkvsel_probe.so) at one
    call's size: `moved` bytes per call (read, or read + write for a copy), in
    a graph of `calls` back-to-back calls over `nb` rotating buffers."""
    per = (moved if mode == probe.PROBE_READ else moved // 2) // 16 * 16
    srcs = [torch.ones(per // 2, dtype=torch.bfloat16, device="cuda") for _ in range(nb)]
    dst_bytes = probe.PROBE_BLOCKS * 16 if mode == probe.PROBE_READ else per
    dsts = [torch.empty(dst_bytes, dtype=torch.uint8, device="cuda") for _ in range(nb)]

    def run():
        for i in range(calls):
            probe.probe_stream(mode, srcs[i % nb], dsts[i % nb], per)
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(10):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        g.replay()
        e[1].record()
        torch.cuda.synchronize()
        ts.append(e[0].elapsed_time(e[1]) * 1e-3 / calls)
    del g, srcs, dsts
    ts.sort()
    moved_per = per if mode == probe.PROBE_READ else 2 * per
    return moved_per / ts[len(ts) // 2] / 1e9


def serving_loop_us(torch, pipeline, kvsynth, cfg, budgets, layers: int = 4,
                    graphs: int = 4) -> float:
    """Decode-time loop on `layers` C2 layers (pipeline.ServingLoop): every step
    appends the new token to the full and the compacted cache and decodes; every
    w steps the window score over the resident full cache, the top-B selection
    and the compaction are redone.  Each graph holds w steps of every layer (one
    re-selection each); the first is a warm-up.  Returns µs per layer per step."""
    W = cfg.w
    loops = []
    for l in range(layers):
        run = pipeline.build_layer(cfg, kvsynth.layer_inputs(cfg, l), budget=budgets[l], slack=W)
        run.score()
        run.select()
        run.compact()
        loops.append(pipeline.ServingLoop.start(run, run.k, run.v, cfg.n, graphs * W))
    toks = [kvsynth.step_inputs(cfg, 0, t) for t in range(W)]
    dev = [tuple(pipeline.device_tensor(tk[name]) for name in ("k_new", "v_new", "q"))
           for tk in toks]
    gs = []
    for _ in range(graphs):   # positions advance from one captured graph to the next
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t in range(W):
                for lp in loops:
                    lp.step(*dev[t])
        gs.append(g)
    assert all(lp.reselections == graphs for lp in loops)
    torch.cuda.synchronize()
    gs[0].replay()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    for g in gs[1:]:
        g.replay()
    e[1].record()
    torch.cuda.synchronize()
    us = e[0].elapsed_time(e[1]) * 1e3 / ((graphs - 1) * W) / layers
    del gs, loops
    return us


def model_serving_loop_us(torch, pipeline, kvsynth, cfg, budgets, layers: int = 4,
                          graphs: int = 4) -> float:
    """The same decode-time loop on `layers` C2 layers with every layer's
    re-selection batched (pipeline.ModelServingLoop: one score, one select
    and one compact call over all layers' segments every w steps).  Each graph
    holds w steps of every layer; the first is a warm-up.  Returns µs per
    layer per step."""
    W = cfg.w
    ins = [kvsynth.layer_inputs(cfg, l) for l in range(layers)]
    k = torch.cat([pipeline.device_tensor(x["K"]) for x in ins])
    v = torch.cat([pipeline.device_tensor(x["V"]) for x in ins])
    q_win = torch.cat([pipeline.device_tensor(x["q_win"]) for x in ins])
    del ins
    mc = kvsynth.get_config(cfg.cid, layers=layers)
    ml = pipeline.ModelServingLoop.start(mc, budgets[:layers], k, v, q_win, graphs * W)
    del k, v, q_win
    toks = [kvsynth.step_inputs(cfg, 0, t) for t in range(W)]
    dev = [tuple(pipeline.device_tensor(tk[name]) for name in ("k_new", "v_new", "q"))
           for tk in toks]
    gs = []
    for _ in range(graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t in range(W):
                for l in range(layers):
                    ml.step_layer(l, *dev[t])
                ml.end_step()
        gs.append(g)
    assert ml.reselections == graphs
    torch.cuda.synchronize()
    gs[0].replay()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    for g in gs[1:]:
        g.replay()
    e[1].record()
    torch.cuda.synchronize()
    us = e[0].elapsed_time(e[1]) * 1e3 / ((graphs - 1) * W) / layers
    del gs, ml
    return us


def summarize_counters(fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes per decode launch from two rocprofv3 --pmc runs of this
    script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by the
    same counter's reading on the 1 GiB reference copy (known bytes)."""
    import csv

    def rows(path, counter):
        with open(path) as f:
            rs = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        rs.sort(key=lambda r: int(r["Dispatch_Id"]))
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rs]

    def reference_copy(rs):
        # copy_reference(): a bf16 fill of the source, then the first device copy after it
        fill = next(i for i, (k, _) in enumerate(rs) if "FillFunctor<c10::BFloat16>" in k)
        return next(v for k, v in rs[fill + 1:] if "copy" in k.lower())

    out = {"source_sha256_16": src_hash(DECODE_SRCS), "copy_bytes": COPY_BYTES}
    per_launch = 0.0
    for counter, path, known in (("FETCH_SIZE", fetch_csv, COPY_BYTES),
                                 ("WRITE_SIZE", write_csv, COPY_BYTES)):
        rs = rows(path, counter)
        copies = [reference_copy(rs)]
        factor = known / (copies[0] * 1024)
        # the C2 step's decode dispatches all come before the first extra
        # workload (LMBA opens them); the C3 / C4 extras reuse the decode kernels
        end = next((i for i, (k, _) in enumerate(rs) if "lmba_row_kernel" in k), len(rs))
        kern = {}
        for name in DECODE_KERNELS:
            vals = [v for k, v in rs[:end] if name in k]
            assert vals, f"no {name} dispatch in {path}"
            kern[name] = {"dispatches": len(vals), "mean_KiB": sum(vals) / len(vals)}
        launch_kib = sum(k["mean_KiB"] for k in kern.values())
        out[counter] = {"copy_KiB": max(copies), "scale_factor": factor, "kernels": kern,
                        "raw_KiB_per_launch": launch_kib,
                        "bytes_per_launch": launch_kib * 1024 * factor}
        per_launch += launch_kib * 1024 * factor
    out["hbm_bytes_per_launch"] = int(per_launch)
    out["_table"] = traffic_table(fetch_csv, write_csv,
                                  {k: out[k]["scale_factor"] for k in ("FETCH_SIZE", "WRITE_SIZE")})
    return out


def _kernel_key(name: str, grid: str) -> str:
    import re
    m = re.search(r"\(anonymous namespace\)::(\w+)(<[^()]*>)?", name)
    short = (m.group(1) + (m.group(2) or "")) if m else name[:40]
    return f"`{short}` (grid {grid})"


def _extras_start(names) -> int:
    """Index of the first dispatch of the extras in a dispatch-ordered list of
    kernel names: the first LMBA call opens them with its own statistics pass
    (`score_stats_reg_kernel`, `score_reduce_kernel`) before the kernels only
    LMBA runs (the probability-writing final pass, the mask, the row select)."""
    names = list(names)
    only = ("lmba_row_kernel", "keep_mask_kernel", "score_stats_kernel<", "score_final_kernel<")
    end = next((i for i, k in enumerate(names) if any(x in k for x in only)), len(names))
    for prev in ("score_reduce_kernel", "score_stats_reg_kernel<"):
        if end > 0 and prev in names[end - 1]:
            end -= 1
    return end


def _dispatches(path: str):
    """Per-dispatch counter values of a rocprofv3 --pmc CSV: [(kernel key,
    kernel name, {counter: value})] in dispatch order (values summed over
    the counter's instances)."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = out.setdefault(int(r["Dispatch_Id"]), [_kernel_key(r["Kernel_Name"],
                                                                   r.get("Grid_Size", "?")),
                                                      r["Kernel_Name"], {}])
            d[2][r["Counter_Name"]] = d[2].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if "Start_Timestamp" in r:
                d[2]["_dur_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    return [tuple(out[k]) for k in sorted(out)]


def traffic_table(fetch_csv: str, write_csv: str, factors: dict) -> str:
    """Markdown table: mean FETCH / WRITE MB per dispatch of every library
    kernel, separately for the C2 step (before the first LMBA dispatch) and
    for the extras measured after it."""
    import re
    rows = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        ds = _dispatches(path)
        # the extras open with the LMBA calls (attention rows, masks, row selects)
        end = _extras_start(d[1] for d in ds)
        for i, (key, name, c) in enumerate(ds):
            if "kvsel" not in name and "probe" not in name:
                continue
            phase = "C2 step" if i < end else "after"
            if phase == "C2 step":   # per-layer launches differ only in grid size
                key = re.sub(r" \(grid \d+\)$", "", key)
            r = rows.setdefault((phase, key), {"n": 0})
            r[counter] = r.get(counter, 0.0) + c[counter] * 1024 * factors[counter] / 1e6
            if counter == "FETCH_SIZE":
                r["n"] += 1
    lines = ["| phase | kernel | dispatches | fetch MB | write MB |", "|---|---|---|---|---|"]
    for (phase, key), r in sorted(rows.items(), key=lambda kv: (kv[0][0] != "C2 step", kv[0][1])):
        n = max(r["n"], 1)
        lines.append(f"| {phase} | {key} | {r['n']} | {r.get('FETCH_SIZE', 0) / n:.2f} | "
                     f"{r.get('WRITE_SIZE', 0) / n:.2f} |")
    return "\n".join(lines)


def sq_table(path: str) -> str:
    """Markdown table from one rocprofv3 --pmc pass of SQ counters (with
    GRBM_GUI_ACTIVE): per library kernel, the launch's cycles, the waves
    resident per SIMD, the share of cycles the matrix cores are busy, the VALU
    issues, both at once, and instructions per wave.  Instance sums are
    divided by the 8 XCDs (cycles) and the 1024 SIMDs (per-SIMD shares);
    SQ_WAVE_CYCLES and SQ_ACTIVE_INST_VALU count in units of four cycles.  The
    clock column is the launch's cycles over its duration; for dispatches of a
    few microseconds the counter window is wider than the kernel and it reads
    high."""
    agg = {}
    for key, name, c in _dispatches(path):
        if "kvsel" not in name:
            continue
        a = agg.setdefault(key, {"n": 0})
        a["n"] += 1
        for k, v in c.items():
            a[k] = a.get(k, 0.0) + v
    lines = ["| kernel | dispatches | cycles per dispatch | µs per dispatch | clock GHz | "
             "waves per SIMD | MFMA busy | VALU issuing | both | VALU insts per wave | "
             "MFMA insts per wave |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for key, a in agg.items():
        n = a["n"]
        cyc = a.get("GRBM_GUI_ACTIVE", 0.0) / n / 8
        simd = max(cyc, 1.0) * 1024
        waves = max(a.get("SQ_WAVES", 0.0) / n, 1.0)
        dur = a.get("_dur_us", 0.0) / n
        ghz = f"{cyc / dur / 1e3:.2f}" if dur > 0 else "?"
        lines.append(
            f"| {key} | {n} | {cyc:.0f} | {dur:.1f} | {ghz} | "
            f"{4 * a.get('SQ_WAVE_CYCLES', 0) / n / simd:.2f} | "
            f"{a.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / n / simd:.2f} | "
            f"{4 * a.get('SQ_ACTIVE_INST_VALU', 0) / n / simd:.2f} | "
            f"{a.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0) / n / simd:.2f} | "
            f"{a.get('SQ_INSTS_VALU', 0) / n / waves:.0f} | {a.get('SQ_INSTS_MFMA', 0) / n / waves:.0f} |")
    return "\n".join(lines)


def trace_tables(trace_csv: str, layers: int = 32) -> str:
    """Markdown tables from a rocprofv3 --kernel-trace CSV of this script:
    every library kernel over the whole run (dispatches, mean / min / max µs),
    then the C2 step alone -- the dispatches before the first LMBA call, of
    which the last replay of each phase's graph is averaged (the step runs
    score, select and compact once for all layers and decode once per layer)."""
    import csv
    import re
    ds = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            m = re.search(r"\(anonymous namespace\)::(\w+)(<[^()]*>)?", r["Kernel_Name"])
            if not m or ("kvsel" not in r["Kernel_Name"] and "probe" not in r["Kernel_Name"]):
                continue
            ds.append((int(r["Start_Timestamp"]), m.group(1) + (m.group(2) or ""),
                       (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    ds.sort()
    agg = {}
    for _, k, us in ds:
        agg.setdefault(k, []).append(us)
    out = ["| kernel | dispatches | mean µs | min µs | max µs |", "|---|---|---|---|---|"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{k}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    end = _extras_start(d[1] for d in ds)
    step = ds[:end]
    out += ["", "C2 step, last graph replay of each phase (µs per dispatch; per layer for the "
            "calls that cover all layers):", "",
            "| kernel | dispatches in the replay | µs per dispatch | µs per layer |",
            "|---|---|---|---|"]
    last = {}
    for k in dict.fromkeys(d[1] for d in step):
        us = [d[2] for d in step if d[1] == k]
        per_step = layers if k.startswith("decode") else 1
        rep = us[-per_step:]
        mean = sum(rep) / len(rep)
        per_layer = mean if per_step == layers else mean / layers
        last[k] = per_layer
        out.append(f"| `{k}` | {len(rep)} | {mean:.2f} | {per_layer:.2f} |")
    dec = sum(v for k, v in last.items() if k.startswith("decode"))
    out += ["", f"Decode launch (split + combine) in the last replay: {dec:.2f} µs per layer."]
    return "\n".join(out)


def pu_host(t):
    """Device tensor -> numpy (int / float tensors only)."""
    return t.detach().cpu().numpy()


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return 1


def cpu_baseline(cfg, budgets, seconds: float) -> dict:
    """The oracle, as it is, on whole segments of layer 0 until `seconds` pass."""
    import kvsynth
    import oracle
    G, w, d, n = cfg.G, cfg.w, cfg.d, cfg.n
    t_stage = {"score": 0.0, "select": 0.0, "compact": 0.0, "decode": 0.0}
    dec_bytes = 0
    segs = 0
    t_start = time.perf_counter()
    for s in range(cfg.batch * cfg.hkv):
        b, kvh = divmod(s, cfg.hkv)
        x = kvsynth.segment_inputs(cfg, 0, b, kvh)
        B = int(budgets[0])
        t = time.perf_counter()
        sc = oracle.window_scores(oracle.to_f64(x["q_win"]), oracle.to_f64(x["K"]), cfg.scale,
                                  n - w)
        t_stage["score"] += time.perf_counter() - t
        t = time.perf_counter()
        keep = oracle.select_topb(sc, B)
        t_stage["select"] += time.perf_counter() - t
        t = time.perf_counter()
        Kc, Vc = oracle.compact(x["K"], x["V"], keep)
        t_stage["compact"] += time.perf_counter() - t
        t = time.perf_counter()
        Kc64, Vc64 = oracle.to_f64(Kc), oracle.to_f64(Vc)
        qd = oracle.to_f64(x["q_dec"])
        for g in range(G):
            oracle.decode_attention(qd[g], Kc64, Vc64, cfg.scale)
        t_stage["decode"] += time.perf_counter() - t
        dec_bytes += keep.size * d * cfg.es * 2 + G * d * (cfg.es + 4)
        segs += 1
        if time.perf_counter() - t_start >= seconds:
            break
    segs_per_layer = cfg.batch * cfg.hkv
    return {
        "value": dec_bytes / t_stage["decode"] / 1e9,
        "unit": "GB/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle on {segs} whole (batch, KV head) segment(s) of layer 0 "
                   f"(score, select, compact, decode of {G} query heads each); decode GB/s over "
                   f"the same algorithmic bytes as the GPU; host os.cpu_count()={os.cpu_count()}"),
        "select_and_compact_us_per_layer_est": (t_stage["select"] + t_stage["compact"]) / segs
        * segs_per_layer * 1e6,
        "stage_s_per_segment": {k: v / segs for k, v in t_stage.items()},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layerwise", action="store_true",
                    help="skip the one-call-per-layer comparison of the compression step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="print kernel-time tables from a rocprofv3 --kernel-trace CSV and exit")
    ap.add_argument("--summarize-sq", metavar="PMC_CSV",
                    help="print a table of SQ counters per library kernel from one "
                         "rocprofv3 --pmc pass and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the decode traffic file from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        res = summarize_counters(*args.summarize_counters)
        table = res.pop("_table")
        with open(COUNTERS, "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res, indent=1))
        print(table)
        return 0
    if args.summarize_sq:
        print(sq_table(args.summarize_sq))
        return 0
    if args.summarize_trace:
        print(trace_tables(args.summarize_trace))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU and needs no collective)", file=sys.stderr)
        return 2

    import torch

    import kvsynth
    import sparse_decode_attention_window_amd as kvsel
    from sparse_decode_attention_window_amd import pipeline

    kvsel.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    copy_gbs = copy_reference(torch)
    log(f"[bench] reference 1 GiB device copy: {copy_gbs:.0f} GB/s (read + write)")
    cfg = kvsynth.get_config(2)
    L = cfg.layers
    profile = kvsynth.zigzag_profile(cfg)
    budgets = kvsel.kvsel_zigzag_budgets(profile, cfg.n, cfg.avg_budget, cfg.floor_budget)

    log(f"[bench] generating {cfg.name}: {L} layers x batch {cfg.batch} x {cfg.hkv} KV heads "
        f"x {cfg.n} tokens x d {cfg.d} ({cfg.dtype})")
    t0 = time.perf_counter()

    def progress(l):
        if l % 4 == 3:
            log(f"[bench] layer {l + 1}/{L} resident ({time.perf_counter() - t0:.1f} s)")
    mr = pipeline.ModelRun.build(cfg, budgets, lambda l: kvsynth.layer_inputs(cfg, l),
                                 log=progress)
    torch.cuda.synchronize()
    S = cfg.batch * cfg.hkv

    # One step = the compression step over the whole model (score, select,
    # compact: one call each for all L layers' segments) and one decode step
    # through the L layers (one call per layer, as a model runs them).  Each
    # phase is captured once as a HIP graph (the kernels are the eager ones;
    # the graph only removes host launch gaps).
    phases = {
        "score": mr.score,
        "select": mr.select,
        "compact": mr.compact,
        "decode": lambda: [mr.decode(l) for l in range(L)],
    }
    for fn in phases.values():   # eager warm-up before capture
        fn()
    torch.cuda.synchronize()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g
    graphs = {name: capture(fn) for name, fn in phases.items()}
    torch.cuda.synchronize()

    def step(ev):
        bud = kvsel.kvsel_zigzag_budgets(profile, cfg.n, cfg.avg_budget, cfg.floor_budget)
        assert bud == budgets
        ev[0].record()
        for i, name in enumerate(phases):
            graphs[name].replay()
            ev[i + 1].record()

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]

    for i in range(args.warmup):
        step(events())
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {wall:.3f} s")

    # per-phase GPU time averaged over steps, per layer
    st = {name: 0.0 for name in phases}
    for ev in evs:
        for i, name in enumerate(phases):
            st[name] += ev[i].elapsed_time(ev[i + 1])
    us = {k: v / (args.steps * L) * 1e3 for k, v in st.items()}       # µs per layer

    # the same compression step issued one layer at a time (for comparison)
    def timed(fn, reps=3):
        g = capture(fn)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        g.replay()
        e[0].record()
        for _ in range(reps):
            g.replay()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / (reps * L) * 1e3
    us_layerwise = {}
    if not args.no_layerwise:
        us_layerwise = {
            "score": timed(lambda: [mr.score_layer(l) for l in range(L)]),
            "select": timed(lambda: [mr.select_layer(l) for l in range(L)]),
            "compact": timed(lambda: [mr.compact_layer(l) for l in range(L)]),
        }
        mr.score(); mr.select(); mr.compact()
        torch.cuda.synchronize()

    # calibration extra, outside the timed steps: per-row LMBA of every layer
    # (ZigZagkv Eq. 3) and the attention the layer's top-B selection keeps
    # (Table 3's attention loss is max(0, 0.9 - kept)); one workspace serves
    # every layer since the launches are ordered on one stream
    R = cfg.G * cfg.w
    B = cfg.batch
    ls = mr.layer_shape
    lm_ws = torch.empty(kvsel.kvsel_lmba_workspace(ls, cfg.w), dtype=torch.uint8, device="cuda")
    lm = torch.empty(L, S * R, dtype=torch.int32, device="cuda")
    km = torch.empty(L, S * R, dtype=torch.float32, device="cuda")

    def lmba_all():
        for l in range(L):
            rows = slice(l * S, (l + 1) * S)
            kvsel.kvsel_lmba(ls, cfg.w, cfg.n - cfg.w, mr.q_win[l * B:(l + 1) * B],
                             mr.k[l * B:(l + 1) * B], lm[l], lm_ws, mr.seg_off[rows],
                             mr.seg_len[rows], mr.idx, mr.r_cap, km[l])
    lmba_all()
    torch.cuda.synchronize()
    g_lm = capture(lmba_all)
    l_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    l_ev[0].record()
    for _ in range(2):
        g_lm.replay()
    l_ev[1].record()
    torch.cuda.synchronize()
    lmba_us = l_ev[0].elapsed_time(l_ev[1]) / (2 * L) * 1e3
    layer_lmba = lm.float().mean(dim=1).cpu().tolist()
    att_loss = (0.9 - km).clamp_min(0).mean(dim=1).cpu().tolist()
    del lm_ws
    log(f"[bench] LMBA + kept mass: {lmba_us:.1f} us per layer; mean LMBA "
        f"{sum(layer_lmba) / L:.0f} tokens, mean attention loss {sum(att_loss) / L:.4f}")

    # serving-loop extra, outside the timed steps: one decoded token joins
    # every segment of every layer (segments are full, so each append
    # replaces the oldest token: the sliding-window path)
    step_tok = kvsynth.step_inputs(cfg, 0, 0)
    kn = pipeline.device_tensor(step_tok["k_new"])
    vn = pipeline.device_tensor(step_tok["v_new"])

    def append_all():
        for l in range(L):
            mr.append_layer(l, kn, vn, step_tok["pos"])
    append_all()
    torch.cuda.synchronize()
    g_app = capture(append_all)
    a_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    a_ev[0].record()
    for _ in range(5):
        g_app.replay()
    a_ev[1].record()
    torch.cuda.synchronize()
    append_us = a_ev[0].elapsed_time(a_ev[1]) / (5 * L) * 1e3

    def rate(fn, reps):
        g = capture(fn)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        g.replay()
        e[0].record()
        for _ in range(reps):
            g.replay()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / reps * 1e3

    # C3 and C4 extras, outside the timed steps.  Each is timed over ROT
    # independently seeded layers replayed back to back (one call per layer),
    # so a call never finds its own rows in the 256 MB memory-side cache: C3
    # decodes 4 x 207 MB, C4 4 x 258 MB.
    ROT = 4

    def rotated(c, stages):
        runs = [pipeline.build_layer(c, kvsynth.layer_inputs(c, l)) for l in range(ROT)]
        for r in runs:
            r.run()
        torch.cuda.synchronize()
        rows = [int(pu_host(r.seg_len).sum()) for r in runs]
        t = {k: rate(lambda k=k: [getattr(r, k)() for r in runs], 3) / ROT for k in stages}
        del runs
        torch.cuda.empty_cache()
        return t, sum(rows) / ROT

    # C3: FastGen head policies over RAP pair-pruned keys (d = 88): ragged
    # segments of 32768 / 2048 / 656 rows; its compact and decode rates beside C2's
    c3 = kvsynth.get_config(3)
    c3_us, rows3 = rotated(c3, ("compact", "decode"))
    c3_dec_us, c3_cmp_us = c3_us["decode"], c3_us["compact"]
    c3_dec_bytes = rows3 * c3.d * c3.es * 2 + c3.batch * c3.hq * c3.d * (c3.es + 4)
    c3_cmp_bytes = rows3 * (c3.d * c3.es * 4 + 4)
    log(f"[bench] C3 ({ROT} layers rotated): decode {c3_dec_us:.1f} us "
        f"({c3_dec_bytes / c3_dec_us / 1e3:.0f} GB/s), compact {c3_cmp_us:.1f} us "
        f"({c3_cmp_bytes / c3_cmp_us / 1e3:.0f} GB/s)")

    # C4: ChunkLLM at 128K context: chunk scores (w = 1 over the compressed
    # chunk keys), chunk select to 48 % of the tokens, compact, decode
    c4 = kvsynth.get_config(4)
    c4_us, rows4 = rotated(c4, ("score", "select", "compact", "decode"))
    c4_dec_bytes = rows4 * c4.d * c4.es * 2 + c4.batch * c4.hq * c4.d * (c4.es + 4)
    c4_cmp_bytes = rows4 * (c4.d * c4.es * 4 + 4)
    log(f"[bench] C4 ({ROT} layers rotated): score {c4_us['score']:.1f} select "
        f"{c4_us['select']:.1f} compact {c4_us['compact']:.1f} decode {c4_us['decode']:.1f} us")

    # serving-loop extra (f3): decode steps with periodic re-selection
    # the decode phase replayed back to back on its own, outside the timed
    # steps (after the extras whose decode dispatches the counter cut leaves
    # out): inside a step it follows the compaction, and the lines that
    # compaction left dirty in the caches are written back while it reads;
    # here the first (untimed) replay has already paid for them
    dec_alone_us = timed(phases["decode"], reps=4)
    serve_layer_us = serving_loop_us(torch, pipeline, kvsynth, cfg, budgets)
    torch.cuda.empty_cache()
    serve_us = model_serving_loop_us(torch, pipeline, kvsynth, cfg, budgets)
    log(f"[bench] serving loop: {serve_us:.1f} us per layer per step with the 4 layers' "
        f"re-selection batched, {serve_layer_us:.1f} with one loop per layer (re-selection "
        f"every {cfg.w} steps)")

    es, d, hq, hkv, n = cfg.es, cfg.d, cfg.hq, cfg.hkv, cfg.n
    lens = pu_host(mr.seg_len).reshape(L, S)
    rows = [int(lens[l].sum()) for l in range(L)]
    assert rows == [S * b for b in budgets]
    mean_rows = sum(rows) / L
    dec_bytes = mean_rows * d * es * 2 + B * hq * d * (es + 4)
    cmp_bytes = mean_rows * (d * es * 4 + 4)
    sc_bytes = B * hkv * n * d * es + B * hq * cfg.w * d * es + B * hkv * n * 4
    sel_bytes = B * hkv * n * 4 + mean_rows * 4
    sc_flops_alg = 2.0 * B * hq * cfg.w * n * d
    gbs = lambda b, t_us: b / (t_us * 1e-6) / 1e9

    dec_gbs = gbs(dec_bytes, us["decode"])
    cmp_gbs = gbs(cmp_bytes, us["compact"])
    # what a plain non-temporal stream of the same size per call reaches here
    from sparse_decode_attention_window_amd import _probe as probe
    read_ceiling = stream_ceiling(torch, probe, probe.PROBE_READ, int(dec_bytes))
    copy_ceiling = stream_ceiling(torch, probe, probe.PROBE_COPY, int(cmp_bytes))
    # the step compacts all L layers in one call: the same bytes as one long copy
    copy_ceiling_all = stream_ceiling(torch, probe, probe.PROBE_COPY, int(cmp_bytes * L),
                                      nb=2, calls=2)
    log(f"[bench] stream ceilings at the call sizes: read {read_ceiling:.0f} GB/s, "
        f"copy {copy_ceiling:.0f} GB/s (one layer's bytes per call), "
        f"{copy_ceiling_all:.0f} GB/s (all layers' bytes in one call)")
    traffic = None
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as f:
            cnt = json.load(f)
        if cnt.get("source_sha256_16") == src_hash(DECODE_SRCS):
            traffic = cnt.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator: planted sink + per-layer heavy hitters + recency; "
                "lognormal(0,0.5) layer-uncertainty profile)",
        "config": {"workload": cfg.name, "layers": L, "batch": B, "hq": hq, "hkv": hkv,
                   "head_dim": d, "context": n, "window": cfg.w,
                   "avg_budget": cfg.avg_budget, "floor_budget": cfg.floor_budget,
                   "parallelism": "single GPU",
                   "compression_calls": "one score, select and compact call for all layers; "
                                        "one decode call per layer"},
        "pct_peak_hbm": round(100 * dec_gbs / PEAK_HBM_GBS, 1),
        "select_and_compact_us_per_layer": round(us["select"] + us["compact"], 2),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic,
                     "kernel": "kvsel_decode_attn (decode_split_kernel + decode_combine_head_kernel)",
                     "algorithmic_bytes_per_launch": int(dec_bytes),
                     "avg_launch_us": round(us["decode"], 3)},
        "stages_us_per_layer": {k: round(v, 3) for k, v in us.items()},
        "stages_us_per_layer_one_call_per_layer": {k: round(v, 3) for k, v in us_layerwise.items()},
        "select_and_compact_us_per_layer_one_call_per_layer":
            round(us_layerwise["select"] + us_layerwise["compact"], 2) if us_layerwise else None,
        "hbm_copy_reference_GBps": round(copy_gbs, 1),
        "extras": {"append_us_per_layer": round(append_us, 3),
                   "append_note": "kvsel_append of one decoded token into all 32 full "
                                  "segments of a layer (oldest-token replacement), "
                                  "outside the timed step",
                   "lmba_us_per_layer": round(lmba_us, 1),
                   "lmba_note": "kvsel_lmba over the 128 window-attention rows of each of the "
                                "32 segments of a layer (rows materialised, 90 %-mass radix "
                                "select per row, kept mass of the top-B selection), outside "
                                "the timed step",
                   "c3_policy_d88": {
                       "rows": rows3,
                       "decode_us": round(c3_dec_us, 2),
                       "decode_GBps": round(c3_dec_bytes / c3_dec_us / 1e3, 1),
                       "decode_frac": round(c3_dec_bytes / c3_dec_us / 1e3 / PEAK_HBM_GBS, 4),
                       "compact_us": round(c3_cmp_us, 2),
                       "compact_GBps": round(c3_cmp_bytes / c3_cmp_us / 1e3, 1),
                       "compact_frac": round(c3_cmp_bytes / c3_cmp_us / 1e3 / PEAK_HBM_GBS, 4),
                       "layers_rotated": ROT,
                       "note": "C3 layers (batch 8, FastGen local / special / global heads, "
                               "RAP pair-pruned d = 88), per layer over 4 independently "
                               "seeded layers replayed back to back (rotated past the 256 MB "
                               "memory-side cache), outside the timed step"},
                   "c4_chunk_128k": {
                       "rows": rows4,
                       "stages_us": {k: round(v, 2) for k, v in c4_us.items()},
                       "decode_GBps": round(c4_dec_bytes / c4_us["decode"] / 1e3, 1),
                       "decode_frac": round(c4_dec_bytes / c4_us["decode"] / 1e3 / PEAK_HBM_GBS, 4),
                       "compact_GBps": round(c4_cmp_bytes / c4_us["compact"] / 1e3, 1),
                       "compact_frac": round(c4_cmp_bytes / c4_us["compact"] / 1e3 / PEAK_HBM_GBS,
                                             4),
                       "layers_rotated": ROT,
                       "note": "C4 layers (batch 1, 131072 tokens, chunk keys of 64 dims, "
                               "chunks kept to 48 % of the tokens), per layer over 4 "
                               "independently seeded layers replayed back to back, outside "
                               "the timed step"},
                   "decode_phase_alone": {
                       "us_per_layer": round(dec_alone_us, 3),
                       "GBps": round(gbs(dec_bytes, dec_alone_us), 1),
                       "note": "the same 32-layer decode graph replayed back to back, outside "
                               "the timed step; inside the step the decode follows the "
                               "compaction, whose non-temporal stores leave no dirty lines "
                               "for it to write back"},
                   "serving_loop_c2": {
                       "us_per_layer_step": round(serve_us, 2),
                       "us_per_layer_step_one_loop_per_layer": round(serve_layer_us, 2),
                       "note": "pipeline.ModelServingLoop on 4 C2 layers: every step appends "
                               "the new token to each layer's full and compacted cache and "
                               "decodes it, layer by layer; every 32 steps score, select and "
                               "compact are redone over the resident full caches, one call "
                               "each for all 4 layers (HIP graphs of 32 steps); beside it the "
                               "same loop as one pipeline.ServingLoop per layer; outside the "
                               "timed step"},
                   "layer_lmba_mean_tokens": [round(x, 1) for x in layer_lmba],
                   "attention_loss_topb_per_layer": [round(x, 5) for x in att_loss]},
        "decode_frac_of_copy_reference": round(dec_gbs / copy_gbs, 4),
        "compact_frac_of_copy_reference": round(cmp_gbs / copy_gbs, 4),
        "hbm_stream_ceilings": {
            "read_GBps": round(read_ceiling, 1), "read_bytes_per_call": int(dec_bytes),
            "copy_GBps": round(copy_ceiling, 1), "copy_bytes_per_call": int(cmp_bytes),
            "copy_GBps_all_layers_one_call": round(copy_ceiling_all, 1),
            "copy_bytes_all_layers_one_call": int(cmp_bytes * L),
            "method": "libkvsel_probe.so non-temporal read / copy streams at the decode and "
                      "compact call sizes, graph of 8 back-to-back calls over 4 rotating "
                      "buffers; the all-layers copy (the step's compaction is one call for "
                      "every layer) as 2 calls over 2 buffers"},
        "decode_frac_of_read_ceiling": round(dec_gbs / read_ceiling, 4),
        "compact_frac_of_copy_ceiling": round(cmp_gbs / copy_ceiling, 4),
        "compact_frac_of_copy_ceiling_all_layers_one_call": round(cmp_gbs / copy_ceiling_all, 4),
        "stages_roofline": {
            "score": {"bound": "hbm", "GB/s": round(gbs(sc_bytes, us["score"]), 1),
                      "frac": round(gbs(sc_bytes, us["score"]) / PEAK_HBM_GBS, 4),
                      "mfma_TFLOP/s_2pass": round(2 * sc_flops_alg / (us["score"] * 1e-6) / 1e12, 1),
                      "mfma_frac_2pass": round(2 * sc_flops_alg / (us["score"] * 1e-6) / 1e12
                                               / PEAK_BF16_TFLOPS, 4),
                      "algorithmic_bytes": int(sc_bytes)},
            "select": {"GB/s": round(gbs(sel_bytes, us["select"]), 1),
                       "algorithmic_bytes": int(sel_bytes)},
            "compact": {"bound": "hbm", "GB/s": round(cmp_gbs, 1),
                        "frac": round(cmp_gbs / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes": int(cmp_bytes)},
            "decode": {"bound": "hbm", "GB/s": round(dec_gbs, 1),
                       "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                       "algorithmic_bytes": int(dec_bytes)},
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(cfg, budgets, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
