"""Benchmark of the MoE layer step on one MI355X.

Prints ONE JSON line on stdout.  The headline is the largest configuration
the metric covers (384 rows: the wide verify step); every other workload is
measured in the same run and listed under `per_workload`:
  metric/value/unit  — effective weight GB/s (unique selected experts' weight
                       bytes / step time) of the headline workload, with
                       us/step beside it;
  per_workload       — for each of the six workloads: us/step (eager, one
                       step per graph, a graph of consecutive steps), effective
                       weight GB/s and its fraction of the 8 TB/s peak and of
                       the measured stream read, and the routed gate_up and
                       down kernels each timed on their own;
  roofline           — the headline's dominant kernel (routed gate_up) timed
                       on its own with HIP events on its stream: algorithmic
                       bytes per launch / mean duration, against 8 TB/s;
  mfma               — the same launch's useful FLOP rate against the dense
                       FP4 matrix peak (the 384-row regime);
  cpu_baseline       — the oracle (plain fp64 C) timed on the host cores on a
                       bounded sample of the headline's rows (a baseline only);
  stream_read_GBps   — a 4 GiB streaming read in the same run (the practical
                       HBM read rate);
  pages_context      — the pages' own figures nearest this path, with the
                       hardware they were measured on (none is for this layer
                       on its own, none is on AMD hardware).
Inputs are seeded synthetic data already resident in HBM.  Every step reads a
different copy of the weights, rotating over at least two copies and at least
2 GiB of them, so no weight byte is read again within 2 GiB of other traffic
(the 256 MB Infinity Cache cannot serve repeats).

Only --gpus 1 is supported: the layer runs on one GPU (one GPU's share of an
expert-parallel / tensor-parallel layer at its real shape).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP4_PEAK_TFLOPS = 10100.0   # dense MXFP4 matrix peak of the MI355X
HEADLINE = "wide-m384-h7168-e256-k8-mxfp4"
CHAIN_MIN = 8               # layer steps per graph in the chained graph timing (at least)
ROTATE_BYTES = 2 << 30      # weight bytes read between two reads of the same copy (at least)
CPU_SAMPLE_ROWS = 32        # rows of the headline step the oracle baseline runs
DOMINANT = "k_gate_up"
# sources that decide what the measured expert kernels read and write
KERNEL_SOURCES = ("block_scaled_fp4_sigmoid_amd/csrc/k_stream.hip", "block_scaled_fp4_sigmoid_amd/csrc/moe_device.h",
                  "block_scaled_fp4_sigmoid_amd/csrc/moe_internal.h", "block_scaled_fp4_sigmoid_amd/csrc/route_dev.h",
                  "block_scaled_fp4_sigmoid_amd/csrc/dense_bf16_dev.h")

# The pages' figures nearest this path, restated, with their hardware.  None
# of them measures this layer on its own or any AMD GPU: context, not targets.
PAGES_CONTEXT = [
    {"figure": "at M = 1 an FP8 GEMM (CUTLASS fp8_scaled_mm) runs 2-3x faster than a BF16 matmul, "
               "while torch._scaled_mm is no faster than BF16",
     "hardware": "GB10 (SM121)", "precision": "FP8 vs BF16", "workload": "dense GEMM, one row",
     "source": "SGLang Spark GB10 Optimizations, section 2 (FP8 Post-Quantization)"},
    {"figure": "the balanced row-block schedule makes the wide MoE kernel 7.4% (batch 32) and 5.3% "
               "(batch 64) faster per call, the step 3.06% and 2.35%",
     "hardware": "GB300 (SM103), TP8, CUDA graphs", "precision": "NVFP4",
     "workload": "Qwen3.5-397B-A17B verify, batch 19-73",
     "source": "sgl-nvidia-mega PR #33, appended table, row wide-bal"},
    {"figure": "router logits computed before the all-reduce save 146 us per step (4.9%); the batch-1 "
               "decode step goes from 3206 to 3016 us; logit RMS error against FP64 0.989x stock",
     "hardware": "GB300 (SM103), TP8", "precision": "model dtype",
     "workload": "Qwen3.5 static decode, batch 1",
     "source": "sgl-nvidia-mega PR #33, update table, row route_lin"},
    {"figure": "fusing the shared expert's SiLU-and-mul with the static FP8 quant of its down input "
               "cuts the per-round time by 0.65% (mean) at batch 64",
     "hardware": "GB300 (SM103), TEP8", "precision": "FP8 shared-expert down input",
     "workload": "Qwen3.5 static decode, acceptance length 4.8",
     "source": "sgl-nvidia-mega PR #33, appended table, row shared act quant"},
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(fmt, N, K):
    """Packed weights + scales (+ fp32 global for NVFP4) of one [N, K] matrix."""
    from block_scaled_fp4_sigmoid_amd import synth
    if fmt == synth.BF16:
        return 2 * N * K
    if fmt == synth.MXFP4:
        return N * K // 2 + N * K // 32
    if fmt == synth.FP8S:
        return N * K + 4
    return N * K // 2 + N * K // 16 + 4


def byte_model(s, U):
    """Algorithmic bytes of one layer step with U unique routed experts, and
    of one routed gate_up and one routed down launch."""
    from block_scaled_fp4_sigmoid_amd import synth
    per_expert = expert_bytes(s.wfmt, 2 * s.I, s.H) + expert_bytes(s.wfmt, s.H, s.I)
    shared = 0
    if s.sfmt != synth.NONE:
        shared = expert_bytes(s.sfmt, 2 * s.I_sh, s.H) + expert_bytes(s.sfmt, s.H, s.I_sh)
    router = 4 * s.E * s.H
    acts = 8 * s.M * s.H  # x, residual in; out, residual_out
    a4 = s.act_fmt == synth.ACT_NVFP4
    anum, aden = (9, 16) if a4 else (33, 32)  # activation bytes per value: NVFP4 or MXFP8
    P = s.M * s.k
    gate_up_launch = (U * expert_bytes(s.wfmt, 2 * s.I, s.H)
                      + s.M * s.H * anum // aden            # activations in (the token rows)
                      + P * s.I * anum // aden)             # h out
    down_launch = U * expert_bytes(s.wfmt, s.H, s.I) + P * s.I * anum // aden  # weights + h in
    return dict(per_expert=per_expert, routed=U * per_expert, shared=shared, router=router,
                acts=acts, total=U * per_expert + shared + router + acts,
                gate_up_launch=gate_up_launch, down_launch=down_launch,
                down_y_bytes=P * s.H * 4,                   # fp32 y written per pair (not algorithmic)
                gate_up_flop=2 * P * 2 * s.I * s.H, down_flop=2 * P * s.I * s.H,
                step_flop=6 * P * s.I * s.H + 6 * s.M * s.I_sh * s.H + 2 * s.M * s.E * s.H)


def kernel_sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_expert_gemms_{workload}.md")


def read_counter_csv(path, counter):
    """Per-dispatch values of one counter from a rocprofv3 counter_collection CSV:
    {kernel name: [(grid, value), ...]} (value in the counter's unit, KiB for
    FETCH_SIZE / WRITE_SIZE)."""
    import csv
    out = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def traffic_summary(fetch_dir, write_dir, workload, command):
    """HBM bytes per launch of the routed gate_up and down kernels from two
    counter runs (FETCH_SIZE, then WRITE_SIZE, both of `--profile-kernels`),
    each scaled by what the same counter reports for the weight-packing
    kernel, a plain permuting copy of known size (16 bytes read and 16 written
    per thread)."""
    from block_scaled_fp4_sigmoid_amd import synth
    f = read_counter_csv(os.path.join(fetch_dir, "run_counter_collection.csv"), "FETCH_SIZE")
    w = read_counter_csv(os.path.join(write_dir, "run_counter_collection.csv"), "WRITE_SIZE")

    def pick(d, pred):
        return [v for name, vals in d.items() if pred(name) for v in vals]

    def copy_factor(d):
        vals = pick(d, lambda n: "k_pack_w" in n)
        known = sum(16 * g for g, _ in vals)
        counted = sum(1024 * v for _, v in vals)
        return known / counted, len(vals)

    ff, nf = copy_factor(f)
    fw, nw = copy_factor(w)
    s = synth.WORKLOADS[workload]
    U = stored_unique(workload)
    bm = byte_model(s, U) if U else None
    lines = [
        f"# HBM traffic of the routed expert GEMMs, {workload}",
        "",
        "Commands (from the repository root, on one MI355X):",
        "",
        "```",
        command,
        "```",
        "",
        f"- copy kernel (k_pack_w, 16 B read + 16 B written per thread): FETCH_SIZE x {ff:.4f}, "
        f"WRITE_SIZE x {fw:.4f} ({nf} and {nw} dispatches)",
        "- each kernel launched on its own, rotating over the bench's weight copies",
        "",
        "| kernel | dispatches | read MB / launch | written MB / launch | algorithmic MB / launch | read / algorithmic |",
        "|---|---:|---:|---:|---:|---:|",
    ]
    keys = {}
    for label, pred, alg in (("routed gate_up (k_gate_up)", lambda n: "k_gate_up" in n,
                              bm and bm["gate_up_launch"]),
                             ("routed down (k_down, k_down_rows)", lambda n: "k_down" in n,
                              bm and bm["down_launch"])):
        gf = [v for _, v in pick(f, pred)]
        gw = [v for _, v in pick(w, pred)]
        if not gf or not gw:
            continue
        fetch = 1024 * ff * float(np.mean(gf))
        write = 1024 * fw * float(np.mean(gw))
        ratio = f"{fetch / alg:.3f}" if alg else "n/a"
        lines.append(f"| {label} | {len(gf)} / {len(gw)} | {fetch / 1e6:.3f} | {write / 1e6:.3f} | "
                     f"{alg / 1e6 if alg else float('nan'):.3f} | {ratio} |")
        keys["gate_up" if "gate_up" in label else "down"] = int(round(fetch + write))
    lines += ["", "The down kernel also writes fp32 y per (row, slot) pair (an implementation buffer, "
              "not counted as algorithmic)." , ""]
    for k_, v_ in keys.items():
        lines.append(f"traffic_bytes_per_launch_{k_}: {v_}")
    lines += [f"unique_experts: {U}", f"kernel_sources_sha256_16: {kernel_sources_sha()}", ""]
    return "\n".join(lines)


def mfma_summary(pmc_dir, workload, command):
    """MFMA activity of the routed gate_up and down (each launched on its own
    by --profile-kernels) from one counter run of SQ_INSTS_MFMA,
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CU_CYCLES and GRBM_GUI_ACTIVE.  Every
    MFMA of the MXFP4 expert kernels is the scaled 16x16x128 FP4 x FP8 one
    (65536 FLOP); GRBM_GUI_ACTIVE is summed over the 8 XCDs."""
    import csv
    from block_scaled_fp4_sigmoid_amd import synth
    s = synth.WORKLOADS[workload]
    U = stored_unique(workload)
    bm = byte_model(s, U) if U else None
    vals = {}
    with open(os.path.join(pmc_dir, "run_counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            n = r["Kernel_Name"]
            key = "gate_up" if "k_gate_up" in n else "down" if "k_down" in n else None
            if key:
                vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = [f"# MFMA activity of the routed expert GEMMs, {workload}", "",
             "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
             "Each kernel launched on its own (`--profile-kernels`), rotating over the bench's weight copies. "
             "Useful FLOP = 2 x pairs x N x K over the real rows; the rest of the issued FLOP pads each "
             "expert's rows to 16-row MFMA tiles.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x "
             "GRBM_GUI_ACTIVE / 8).", "",
             "| kernel | dispatches | MFMA instr. | issued FLOP | useful FLOP | useful / issued | MFMA busy |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for key, useful in (("gate_up", bm and bm["gate_up_flop"]), ("down", bm and bm["down_flop"])):
        c = vals.get(key)
        if not c:
            continue
        mean = {k: float(np.mean(v)) for k, v in c.items()}
        n = len(c.get("SQ_INSTS_MFMA", []))
        issued = mean.get("SQ_INSTS_MFMA", 0.0) * 65536
        busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * mean.get("GRBM_GUI_ACTIVE", 1.0) / 8)
        lines.append(f"| routed {key} | {n} | {mean.get('SQ_INSTS_MFMA', 0):.4g} | {issued:.4g} | "
                     f"{useful if useful else float('nan'):.4g} | {useful / issued if useful and issued else float('nan'):.0%} | "
                     f"{busy:.1%} |")
    lines += ["", f"unique_experts: {U}", f"kernel_sources_sha256_16: {kernel_sources_sha()}", ""]
    return "\n".join(lines)


def _read_keys(path):
    vals = {}
    if not os.path.exists(path):
        return vals
    with open(path) as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith(("-", "#", " ", "|", "`")):
                k_, v_ = ln.split(":", 1)
                vals[k_.strip()] = v_.strip()
    return vals


def unique_path(workload):
    """Where a counter run leaves the unique-expert count of its input for the
    summary step that follows it (the in-tree build folder)."""
    return os.path.join(ROOT, "_build", f"unique_{workload}.txt")


def stored_unique(workload):
    """Unique experts of the workload's default input (written by --profile-kernels)."""
    v = _read_keys(unique_path(workload)).get("unique_experts")
    return int(v) if v else None


def stored_traffic(workload, kernel="gate_up"):
    """HBM bytes per launch from the committed summary, or None when there is
    none or the kernel's sources changed since the counters were taken."""
    vals = _read_keys(traffic_path(workload))
    if vals.get("kernel_sources_sha256_16") != kernel_sources_sha():
        return None
    try:
        return int(vals[f"traffic_bytes_per_launch_{kernel}"])
    except (KeyError, ValueError):
        return None


def kernel_name(n):
    """A kernel's name without its parameter list or namespace noise."""
    import re
    n = n.replace("(anonymous namespace)::", "")
    n = re.sub(r"^void ", "", n)
    depth, out = 0, ""
    for ch in n:
        if ch == "(" and depth == 0:
            break
        depth += (ch == "<") - (ch == ">")
        out += ch
    return out.replace("unsigned char", "u8")[:60]


def kernel_summary(db, title, command):
    """Markdown table of a rocprofv3 kernel trace (its rocpd SQLite output):
    per kernel name and grid size, calls and durations."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, grid_x / workgroup_x, count(*), avg(duration), min(duration), "
                       "max(duration), sum(duration) from kernels group by name, grid_x "
                       "order by sum(duration) desc").fetchall()
    tot = sum(r[6] for r in rows)
    out = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", f"    {command}", "",
           "Summary of the kernel trace (rocprofv3 --kernel-trace --stats), all kernels of the run",
           "including setup and warmup; durations in microseconds.", "",
           "| kernel | workgroups | calls | avg us | min us | max us | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for n, wg, c, a, mn, mx, s in rows:
        out.append(f"| {kernel_name(n)} | {wg} | {c} | {a / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | "
                   f"{100 * s / tot:.1f} |")
    return "\n".join(out) + "\n"


def timed_units(units, stream, windows=5):
    """Times a sequence of launches given as (callable, steps it covers), with
    HIP events on `stream`: one event before the first unit and one after each
    of `windows` groups of consecutive units.  Returns (ms per step over all of
    them, [ms per step of each window])."""
    import torch
    nw = max(1, min(windows, len(units)))
    cut = [len(units) * w // nw for w in range(nw + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in cut]
    torch.cuda.synchronize()
    ev[0].record(stream)
    w = 1
    for u, (fn, _) in enumerate(units):
        fn()
        if u + 1 == cut[w]:
            ev[w].record(stream)
            w += 1
    torch.cuda.synchronize()
    steps = [sum(n for _, n in units[cut[j]:cut[j + 1]]) for j in range(nw)]
    per = [ev[j].elapsed_time(ev[j + 1]) / steps[j] for j in range(nw)]
    return ev[0].elapsed_time(ev[-1]) / sum(steps), per


def timed(fn, steps, warmup, stream, windows=5):
    """fn(i) for i < warmup untimed, then exactly `steps` calls timed in
    `windows` windows; returns (ms per step, [ms per step of each window])."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    return timed_units([((lambda i=i: fn(i)), 1) for i in range(steps)], stream, windows)


def window_stats(per):
    """median, p10 and p90 (us per step) over the windows."""
    a = np.asarray(per) * 1e3
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "windows": len(a)}


class ExpertAlone:
    """The routed gate_up and down as launches of their own on one routing of
    the step's input: gate_up(w13) and down(w2) launch one kernel each on the
    given weight copy (bucket-ordered MXFP8 activations, or NVFP4 for W4A4)."""

    def __init__(self, moe, s, d, dev):
        import torch
        from block_scaled_fp4_sigmoid_amd import synth
        self.moe, self.s = moe, s
        rt = moe.Routing(s.M, s.E, s.k, dev)
        lg = torch.empty((s.M, s.E), dtype=torch.float32, device=dev)
        moe.route_topk(rt, x=d.x, w_router=d.Wr, bias=d.bias, routed_scale=s.routed_scale, logits_out=lg)
        P = s.M * s.k
        self.rt, self.d = rt, d
        self.a4 = s.act_fmt == synth.ACT_NVFP4
        self.y = torch.empty((P, s.H), dtype=torch.float32, device=dev)
        if self.a4:
            self.xq = torch.empty((P, s.H // 2), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((P, s.H // 16), dtype=torch.uint8, device=dev)
            moe.quant_act_nvfp4(d.x, d.x_global, self.xq, self.xs, routing=rt)
            self.hq = torch.empty((P, s.I // 2), dtype=torch.uint8, device=dev)
            self.hs = torch.empty((P, s.I // 16), dtype=torch.uint8, device=dev)
            self.ws = None
        else:
            self.xq = torch.empty((P, s.H), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((P, s.H // 32), dtype=torch.uint8, device=dev)
            moe.quant_act_mxfp8(d.x, self.xq, self.xs, routing=rt)
            self.hq = torch.empty((P, s.I), dtype=torch.uint8, device=dev)
            self.hs = torch.empty((P, s.I // 32), dtype=torch.uint8, device=dev)
            nb = moe.lib().moe_gate_up_workspace_bytes(d.w13.fmt, s.M, s.H, s.I, s.E, s.k, 0)
            self.ws = moe.workspace(max(256, nb), dev)
        torch.cuda.synchronize()
        self.U = int(torch.unique(rt.topk_ids).numel())

    def gate_up(self, w13):
        s, moe = self.s, self.moe
        if self.a4:
            moe.expert_gate_up_nvfp4a(w13, s.M, s.H, s.I, s.E, s.k, self.xq, self.xs, self.d.x_global,
                                      self.d.h_globals, self.hq, self.hs, routing=self.rt)
        else:
            moe.expert_gate_up(w13, s.M, s.H, s.I, s.E, s.k, routing=self.rt, a_q=self.xq, a_s=self.xs,
                               h_q=self.hq, h_s=self.hs, ws=self.ws)

    def down(self, w2):
        s, moe = self.s, self.moe
        if self.a4:
            moe.expert_down_nvfp4a(w2, s.M, s.H, s.I, s.E, s.k, self.hq, self.hs, self.d.h_globals, self.y,
                                   routing=self.rt)
        else:
            moe.expert_down(w2, s.M, s.H, s.I, s.E, s.k, self.y, routing=self.rt, h_q=self.hq, h_s=self.hs)


def stage_workload(name, seed, copies_arg):
    """Inputs drawn and staged, the weight copies rotated over, and the layer
    objects (one per copy)."""
    import torch
    from block_scaled_fp4_sigmoid_amd import moe, staging, synth
    dev = "cuda"
    s = synth.WORKLOADS[name]
    t0 = time.time()
    inp = synth.make_inputs(name, seed=seed)
    d = staging.to_device(inp, dev)
    layer0 = d.layer()
    out = torch.empty((s.M, s.H), dtype=torch.int16, device=dev)
    res = torch.empty_like(out)
    logits = torch.empty((s.M, s.E), dtype=torch.float32, device=dev)
    ids = torch.empty((s.M, s.k), dtype=torch.int32, device=dev)
    layer0(d.x, d.x, out, res, logits, ids)
    torch.cuda.synchronize()
    U = int(np.unique(ids.cpu().numpy()).size)
    bm = byte_model(s, U)
    copies = copies_arg or max(2, math.ceil(ROTATE_BYTES / bm["total"]))
    copies_w = [(d.w13, d.w2, d.sh13, d.sh2, d.Wr)]
    layers = [layer0]
    for c in range(1, copies):
        cw = (staging.clone_weights(d.w13), staging.clone_weights(d.w2), staging.clone_weights(d.sh13),
              staging.clone_weights(d.sh2), d.Wr.clone())
        copies_w.append(cw)
        layers.append(moe.Layer(s.M, s.H, s.E, s.k, s.I, s.I_sh, s.routed_scale, s.eps, cw[4], d.bias,
                                cw[0], cw[1], cw[2], cw[3], d.gamma, s.swiglu_limit, s.act_fmt, d.x_global,
                                d.h_globals, d.sh_h_global if s.sfmt == synth.NVFP4 else None, d.sh_in_scale,
                                d.sh_h_scale))
    torch.cuda.synchronize()
    log(f"[bench] {name}: U={U} unique experts, routed bytes {bm['routed'] / 1e6:.1f} MB, total "
        f"{bm['total'] / 1e6:.1f} MB, {copies} weight copies; staged in {time.time() - t0:.1f}s")
    return dict(name=name, s=s, inp=inp, d=d, layers=layers, copies_w=copies_w, copies=copies, U=U, bm=bm,
                out=out, res=res, logits=logits)


def measure(st, steps, warmup, read_gbps, graphs=True):
    """One workload: the layer step (eager, one step per graph, a chained
    graph) and its routed gate_up and down on their own."""
    import torch
    from block_scaled_fp4_sigmoid_amd import moe, synth
    s, d, layers, copies, bm = st["s"], st["d"], st["layers"], st["copies"], st["bm"]
    out, res = st["out"], st["res"]
    stream = torch.cuda.current_stream()

    def step_eager(i):
        layers[i % copies](d.x, d.x, out, res)

    ms_eager, win_eager = timed(step_eager, steps, warmup, stream)
    ms_graph = ms_chain = chain = None
    win_chain = None
    if graphs:
        gs = torch.cuda.Stream()
        one = []
        with torch.cuda.stream(gs):
            for c in range(copies):
                layers[c](d.x, d.x, out, res, stream=gs)
            gs.synchronize()
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=gs):
                    layers[c](d.x, d.x, out, res, stream=gs)
                one.append(g)
        torch.cuda.synchronize()
        ms_graph, _ = timed(lambda i: one[i % copies].replay(), steps, warmup, stream)
        # A decode step's graph holds every layer back to back: a chain of G
        # consecutive layer steps (rotating the weight copies, G a multiple of
        # the copy count) in one graph.  K steps = K // G chain replays plus
        # K % G one-step replays.
        chain = copies * math.ceil(CHAIN_MIN / copies)
        gchain = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(gchain, stream=gs):
                for j in range(chain):
                    layers[j % copies](d.x, d.x, out, res, stream=gs)
        torch.cuda.synchronize()
        full, rem = divmod(steps, chain)
        units = [(gchain.replay, chain)] * full + [(one[j % copies].replay, 1) for j in range(rem)]
        gchain.replay()  # warm
        torch.cuda.synchronize()
        ms_chain, win_chain = timed_units(units, stream)
        del one, gchain
    ms, timing, win = ms_eager, "eager launches", win_eager
    if ms_chain is not None and ms_chain < ms_eager:
        ms, timing, win = ms_chain, "graph of %d consecutive layer steps, replayed" % chain, win_chain

    alone = ExpertAlone(moe, s, d, "cuda")
    w13s = [c[0] for c in st["copies_w"]]
    w2s = [c[1] for c in st["copies_w"]]
    ms_gu, win_gu = timed(lambda i: alone.gate_up(w13s[i % copies]), steps, warmup, stream)
    ms_dn, win_dn = timed(lambda i: alone.down(w2s[i % copies]), steps, warmup, stream)
    gu_gbps = bm["gate_up_launch"] / (ms_gu * 1e-3) / 1e9
    dn_gbps = bm["down_launch"] / (ms_dn * 1e-3) / 1e9
    value = bm["routed"] / (ms * 1e-3) / 1e9
    log(f"[bench] {s.name}: {ms * 1e3:.2f} us/step ({timing}); eager {ms_eager * 1e3:.2f}"
        + (f", graph {ms_graph * 1e3:.2f}, chain {ms_chain * 1e3:.2f}" if graphs else "")
        + f"; gate_up alone {ms_gu * 1e3:.2f} us ({gu_gbps:.0f} GB/s), down alone {ms_dn * 1e3:.2f} us "
        f"({dn_gbps:.0f} GB/s)")
    e = {
        "workload": s.name, "rows": s.M, "hidden": s.H, "experts": s.E, "top_k": s.k, "intermediate": s.I,
        "weights": synth.FMT_NAMES[s.wfmt],
        "activations": "nvfp4" if s.act_fmt == synth.ACT_NVFP4 else "mxfp8",
        "shared": synth.FMT_NAMES[s.sfmt], "unique_experts": st["U"], "weight_copies": copies,
        "us_per_step": round(ms * 1e3, 2), "timing": timing,
        "us_per_step_eager": round(ms_eager * 1e3, 2),
        "us_per_step_graph": None if ms_graph is None else round(ms_graph * 1e3, 2),
        "us_per_step_graph_chain": None if ms_chain is None else round(ms_chain * 1e3, 2),
        "us_per_step_windows": window_stats(win),
        "weight_GBps": round(value, 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "frac_of_stream_read": round(value / read_gbps, 4),
        "total_alg_GBps": round(bm["total"] / (ms * 1e-3) / 1e9, 1),
        "alg_bytes_per_step": bm["total"],
        "floor_us_at_8TBps": round(bm["total"] / HBM_PEAK_GBPS / 1e3, 2),
        "gate_up_alone": {"us_per_launch": round(ms_gu * 1e3, 2), "GBps": round(gu_gbps, 1),
                          "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
                          "frac_of_stream_read": round(gu_gbps / read_gbps, 4),
                          "alg_bytes_per_launch": bm["gate_up_launch"],
                          "us_per_launch_windows": window_stats(win_gu),
                          "traffic": stored_traffic(s.name, "gate_up")},
        "down_alone": {"us_per_launch": round(ms_dn * 1e3, 2), "GBps": round(dn_gbps, 1),
                       "frac": round(dn_gbps / HBM_PEAK_GBPS, 4),
                       "frac_of_stream_read": round(dn_gbps / read_gbps, 4),
                       "alg_bytes_per_launch": bm["down_launch"],
                       "us_per_launch_windows": window_stats(win_dn),
                       "traffic": stored_traffic(s.name, "down")},
    }
    if s.M >= 256:  # the MFMA-bound regime the metric names: FLOP rate against the FP4 matrix peak
        gu_tf = bm["gate_up_flop"] / (ms_gu * 1e-3) / 1e12
        e["mfma"] = {"kernel": "k_gate_up (routed, alone)", "useful_TFLOPs": round(gu_tf, 1),
                     "peak_TFLOPs": FP4_PEAK_TFLOPS, "frac_of_fp4_peak": round(gu_tf / FP4_PEAK_TFLOPS, 4),
                     "step_useful_TFLOPs": round(bm["step_flop"] / (ms * 1e-3) / 1e12, 1),
                     "step_frac_of_fp4_peak": round(bm["step_flop"] / (ms * 1e-3) / 1e12 / FP4_PEAK_TFLOPS, 4),
                     "flop_per_weight_byte": round(bm["step_flop"] / bm["total"], 1),
                     "ridge_flop_per_byte": round(FP4_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9))}
    del alone
    return e, ms, ms_gu


def cpu_baseline(inp, logits, U, bm):
    """The oracle on a bounded sample of the step's rows (all k routed experts
    of each sampled row and the shared expert), one warm run then the median
    of 3, scaled to the whole step by rows."""
    from oracle import oracle as orc
    s = inp.shape
    rows = np.arange(s.M) if s.M <= CPU_SAMPLE_ROWS else np.linspace(0, s.M - 1, CPU_SAMPLE_ROWS).astype(np.int32)
    need = set()
    for r in rows:
        ids, _, _ = orc.topk_row(logits[r], inp.bias, s.k, s.routed_scale)
        need.update(int(e) for e in ids)
    L = orc.Layer(inp, experts=need)
    items = len(rows) * (s.k + (1 if s.sfmt else 0))
    threads = min(orc.num_cores(), items)
    L.rows(rows, logits=logits, nthreads=threads)  # warm
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        L.rows(rows, logits=logits, nthreads=threads)
        times.append(time.perf_counter() - t0)
    t_step = float(np.median(times)) * s.M / len(rows)
    return {"value": round(bm["routed"] / t_step / 1e9, 4), "unit": "GB/s", "us_per_step": round(t_step * 1e6, 1),
            "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of the {s.M} rows of the {s.name} step (each row's {s.k} routed experts"
                      + (" and the shared expert" if s.sfmt else "") + "), 1 warm run then the median of 3, "
                      f"scaled to the whole step by rows ({s.M}/{len(rows)}); weight GB/s = the step's "
                      f"{U} unique experts' bytes / that time"}


def calibrate(stream):
    """A streaming read of 4 GiB in the GEMMs' row pattern (the practical HBM
    read rate) and a plain 1 GiB device copy (context)."""
    import torch
    from block_scaled_fp4_sigmoid_amd import probe
    dev = "cuda"
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(1, dtype=torch.int32, device=dev)
    read_gbps, read_row = 0.0, 0
    for row_bytes in (1152, 3584):  # the GEMMs' row pattern at two row lengths; the faster counts
        nb = buf.numel() // row_bytes * row_bytes
        ms_read, _ = timed(lambda i: probe.stream_read(buf, row_bytes, sink), 10, 2, stream)
        if nb / (ms_read * 1e-3) / 1e9 > read_gbps:
            read_gbps, read_row = nb / (ms_read * 1e-3) / 1e9, row_bytes
    del buf
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    buf2 = torch.empty_like(buf)
    ms_copy, _ = timed(lambda i: buf2.copy_(buf), 20, 3, stream)
    copy_gbps = 2 * buf.numel() / (ms_copy * 1e-3) / 1e9
    del buf, buf2
    torch.cuda.empty_cache()
    log(f"[bench] stream read 4 GiB: {read_gbps:.0f} GB/s (rows of {read_row} B); "
        f"device copy 1 GiB: {copy_gbps:.0f} GB/s")
    return read_gbps, copy_gbps


def profile_kernels(name, seed, n, copies_arg):
    """Counter runs: the routed gate_up, then the routed down, each launched
    n times on its own (rotating the weight copies); nothing else launches
    these kernels in the run."""
    import torch
    from block_scaled_fp4_sigmoid_amd import moe, staging, synth
    s = synth.WORKLOADS[name]
    inp = synth.make_inputs(name, seed=seed)
    d = staging.to_device(inp, "cuda")
    alone = ExpertAlone(moe, s, d, "cuda")
    bm = byte_model(s, alone.U)
    copies = copies_arg or max(2, math.ceil(ROTATE_BYTES / bm["total"]))
    cw = [(d.w13, d.w2)] + [(staging.clone_weights(d.w13), staging.clone_weights(d.w2)) for _ in range(1, copies)]
    for i in range(n):
        alone.gate_up(cw[i % copies][0])
    for i in range(n):
        alone.down(cw[i % copies][1])
    torch.cuda.synchronize()
    os.makedirs(os.path.dirname(unique_path(name)), exist_ok=True)
    with open(unique_path(name), "w") as fh:
        fh.write(f"unique_experts: {alone.U}\n")
    log(f"[bench] {name}: routed gate_up and down launched {n} times each ({copies} weight copies, U={alone.U})")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, help="the headline workload")
    ap.add_argument("--only", action="store_true", help="measure the headline workload only")
    ap.add_argument("--seed", type=int, default=None, help="seed of the headline workload")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-kernels", type=int, default=0,
                    help="only launch the routed gate_up and down N times each (for counter runs)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary of two rocprofv3 counter runs to stdout")
    ap.add_argument("--kernel-summary", nargs=2, metavar=("ROCPD_DB", "TITLE"),
                    help="write the summary of a rocprofv3 kernel trace to stdout")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="write the MFMA counter summary of a --profile-kernels counter run to stdout")
    ap.add_argument("--summary-command", default="", help="the commands to record in a summary")
    args = ap.parse_args()
    if args.traffic_summary:
        print(traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.workload,
                              args.summary_command))
        return
    if args.mfma_summary:
        print(mfma_summary(args.mfma_summary, args.workload, args.summary_command))
        return
    if args.kernel_summary:
        print(kernel_summary(args.kernel_summary[0], args.kernel_summary[1], args.summary_command), end="")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the layer is one "
              "GPU's share of an expert-parallel / tensor-parallel MoE layer and the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_scaled_fp4_sigmoid_amd import synth

    head = args.workload
    seed = args.seed if args.seed is not None else synth.seed_of(head)
    if args.profile_kernels:
        profile_kernels(head, seed, args.profile_kernels, args.copies)
        return

    stream = torch.cuda.current_stream()
    read_gbps, copy_gbps = calibrate(stream)
    names = [head] + ([] if args.only else [n for n in synth.WORKLOAD_ORDER + list(synth.EXTRA_WORKLOADS)
                                            if n != head])
    per = []
    hctx = None
    for name in names:
        st = stage_workload(name, seed if name == head else synth.seed_of(name), args.copies)
        e, ms, ms_gu = measure(st, args.steps, args.warmup, read_gbps, graphs=not args.no_graph)
        per.append(e)
        if name == head:
            hctx = dict(inp=st["inp"], logits=st["logits"].cpu().numpy(), U=st["U"], bm=st["bm"], ms=ms,
                        ms_gu=ms_gu, s=st["s"], copies=st["copies"])
        del st
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    s, bm, ms, ms_gu = hctx["s"], hctx["bm"], hctx["ms"], hctx["ms_gu"]
    he = per[0]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(hctx["inp"], hctx["logits"], hctx["U"], bm)
        log(f"[bench] oracle on host: {cpu['us_per_step'] / 1e3:.1f} ms/step with {cpu['cores']} threads "
            f"({cpu['sample']})")

    gu_gbps = bm["gate_up_launch"] / (ms_gu * 1e-3) / 1e9
    value = bm["routed"] / (ms * 1e-3) / 1e9
    line = {
        "metric": "MoE layer us/step and effective weight GB/s at 1-384 rows (% of HBM peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "us_per_step_eager": he["us_per_step_eager"],
        "us_per_step_graph": he["us_per_step_graph"],
        "us_per_step_graph_chain": he["us_per_step_graph_chain"],
        "timing": he["timing"],
        "us_per_step_windows": he["us_per_step_windows"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4xfp4->fp32" if s.act_fmt == synth.ACT_NVFP4 else "fp4xfp8->fp32",
        "data": "synthetic (seeded; weights drawn N(0,0.02) and encoded offline)",
        "config": {"workload": s.name, "rows": s.M, "hidden": s.H, "experts": s.E, "top_k": s.k,
                   "intermediate": s.I, "weights": he["weights"], "activations": he["activations"],
                   "shared": he["shared"], "unique_experts": hctx["U"], "weight_copies": hctx["copies"],
                   "parallelism": "single GPU"},
        "frac_of_hbm_peak": he["frac_of_hbm_peak"],
        "stream_read_GBps": round(read_gbps, 1),
        "frac_of_stream_read": he["frac_of_stream_read"],
        "total_alg_GBps": he["total_alg_GBps"],
        "copy_GBps": round(copy_gbps, 1),
        "roofline": {"kernel": "k_gate_up (routed, alone)", "bound": "hbm",
                     "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gu_gbps / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(s.name, "gate_up"),
                     "us_per_launch": round(ms_gu * 1e3, 2),
                     "us_per_launch_windows": he["gate_up_alone"]["us_per_launch_windows"],
                     "frac_of_stream_read": round(gu_gbps / read_gbps, 4),
                     "alg_bytes_per_launch": bm["gate_up_launch"]},
        "mfma": he.get("mfma"),
        "cpu_baseline": cpu,
        "per_workload": per,
        "pages_context": PAGES_CONTEXT,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
