"""Benchmark of the MoE layer step on one MI355X.

Prints ONE JSON line on stdout:
  metric/value/unit  — effective weight GB/s (unique selected experts' weight
                       bytes / step time) at the measured workload, with
                       ms_per_step beside it;
  roofline           — the dominant kernel (routed gate_up) timed on its own
                       with HIP events: algorithmic bytes per launch / mean
                       duration, against the 8 TB/s HBM peak;
  cpu_baseline       — the oracle (plain fp64 C) timed on the host cores on
                       the same inputs (a baseline only);
  stream_read_GBps   — a 4 GiB streaming read in the same run (the practical
                       HBM read rate); fractions are given against it and
                       against the 8 TB/s peak;
  *_windows          — the K timed steps split in 5 windows: median, p10, p90.
Inputs are seeded synthetic data already resident in HBM; each step reads a
different copy of the weights (rotation over enough copies that no step
finds the previous step's weights in the 256 MB Infinity Cache).

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
DEFAULT_WORKLOAD = "verify-m8-h7168-e256-k8-nvfp4"
CHAIN_MIN = 8  # layer steps per graph in the chained graph timing (at least)
DOMINANT = "k_gate_up"
# sources that decide what the dominant kernel reads and writes
KERNEL_SOURCES = ("block_scaled_fp4_sigmoid_amd/csrc/k_stream.hip", "block_scaled_fp4_sigmoid_amd/csrc/moe_device.h",
                  "block_scaled_fp4_sigmoid_amd/csrc/moe_internal.h", "block_scaled_fp4_sigmoid_amd/csrc/route_dev.h",
                  "block_scaled_fp4_sigmoid_amd/csrc/dense_bf16_dev.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(s, fmt, N, K):
    """Packed weights + scales (+ fp32 global for NVFP4) of one [N, K] matrix."""
    from block_scaled_fp4_sigmoid_amd import synth
    if fmt == synth.BF16:
        return 2 * N * K
    if fmt == synth.MXFP4:
        return N * K // 2 + N * K // 32
    return N * K // 2 + N * K // 16 + 4


def byte_model(s, U):
    from block_scaled_fp4_sigmoid_amd import synth
    per_expert = expert_bytes(s, s.wfmt, 2 * s.I, s.H) + expert_bytes(s, s.wfmt, s.H, s.I)
    shared = 0
    if s.sfmt != synth.NONE:
        shared = expert_bytes(s, s.sfmt, 2 * s.I_sh, s.H) + expert_bytes(s, s.sfmt, s.H, s.I_sh)
    router = 4 * s.E * s.H
    acts = 8 * s.M * s.H  # x, residual in; out, residual_out
    a4 = s.act_fmt == synth.ACT_NVFP4
    anum, aden = (9, 16) if a4 else (33, 32)  # activation bytes per value: NVFP4 or MXFP8
    gate_up_launch = (U * expert_bytes(s, s.wfmt, 2 * s.I, s.H)
                      + s.M * s.H * anum // aden            # activations in
                      + s.M * s.k * s.I * anum // aden)     # h out
    return dict(per_expert=per_expert, routed=U * per_expert, shared=shared, router=router,
                acts=acts, total=U * per_expert + shared + router + acts,
                gate_up_launch=gate_up_launch)


def kernel_sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{DOMINANT}_{workload}.md")


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
    """HBM bytes per launch of the routed gate_up from two counter runs
    (FETCH_SIZE, WRITE_SIZE), each scaled by what the same counter reports for
    the weight-packing kernel, a plain permuting copy of known size (16 bytes
    read and 16 written per thread)."""
    f = read_counter_csv(os.path.join(fetch_dir, "run_counter_collection.csv"), "FETCH_SIZE")
    w = read_counter_csv(os.path.join(write_dir, "run_counter_collection.csv"), "WRITE_SIZE")

    def pick(d, key):
        return [v for name, vals in d.items() if key in name for v in vals]

    def copy_factor(d):
        vals = pick(d, "k_pack_w")
        known = sum(16 * g for g, _ in vals)
        counted = sum(1024 * v for _, v in vals)
        return known / counted, len(vals)

    ff, nf = copy_factor(f)
    fw, nw = copy_factor(w)
    gf = [v for _, v in pick(f, DOMINANT)]
    gw = [v for _, v in pick(w, DOMINANT)]
    fetch = 1024 * ff * float(np.mean(gf))
    write = 1024 * fw * float(np.mean(gw))
    lines = [
        f"# HBM traffic of the routed gate_up, {workload}",
        "",
        "Commands (from the repository root, on one MI355X):",
        "",
        "```",
        command,
        "```",
        "",
        f"- copy kernel (k_pack_w, 16 B read + 16 B written per thread): FETCH_SIZE x {ff:.4f}, "
        f"WRITE_SIZE x {fw:.4f} ({nf} and {nw} dispatches)",
        f"- gate_up dispatches: {len(gf)} (FETCH_SIZE), {len(gw)} (WRITE_SIZE)",
        f"- FETCH_SIZE mean {np.mean(gf):.1f} KiB -> {fetch / 1e6:.3f} MB read per launch",
        f"- WRITE_SIZE mean {np.mean(gw):.1f} KiB -> {write / 1e6:.3f} MB written per launch",
        "",
        f"traffic_bytes_per_launch: {int(round(fetch + write))}",
        f"kernel_sources_sha256_16: {kernel_sources_sha()}",
        "",
    ]
    return "\n".join(lines)


def stored_traffic(workload):
    """Traffic per launch from the committed summary, or None when there is
    none or the kernel's sources changed since the counters were taken."""
    p = traffic_path(workload)
    if not os.path.exists(p):
        return None
    vals = {}
    with open(p) as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith(("-", "#", " ")):
                k_, v_ = ln.split(":", 1)
                vals[k_.strip()] = v_.strip()
    if vals.get("kernel_sources_sha256_16") != kernel_sources_sha():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed_units(units, stream, windows=5):
    """Times a sequence of launches given as (callable, steps it covers), with
    HIP events on `stream`: one event before the first unit and one after each
    of `windows` groups of consecutive units.  Returns (ms per step over all of
    them, [ms per step of each window])."""
    import torch
    nw = max(1, min(windows, len(units)))
    cut = [len(units) * w // nw for w in range(nw + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in cut]
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


def gate_up_alone(moe, s, d, logits, dev):
    """The routed gate_up as one launch on bucket-ordered activations (MXFP8,
    or NVFP4 for W4A4 workloads): returns a function of the W13 copy."""
    import torch
    from block_scaled_fp4_sigmoid_amd import synth
    rt = moe.Routing(s.M, s.E, s.k, dev)
    moe.route_topk(rt, x=d.x, w_router=d.Wr, bias=d.bias, routed_scale=s.routed_scale, logits_out=logits)
    P = s.M * s.k
    if s.act_fmt == synth.ACT_NVFP4:
        xq = torch.empty((P, s.H // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty((P, s.H // 16), dtype=torch.uint8, device=dev)
        moe.quant_act_nvfp4(d.x, d.x_global, xq, xs, routing=rt)
        hq = torch.empty((P, s.I // 2), dtype=torch.uint8, device=dev)
        hs = torch.empty((P, s.I // 16), dtype=torch.uint8, device=dev)
        return lambda w13: moe.expert_gate_up_nvfp4a(w13, s.M, s.H, s.I, s.E, s.k, xq, xs, d.x_global,
                                                     d.h_globals, hq, hs, routing=rt)
    xq = torch.empty((P, s.H), dtype=torch.uint8, device=dev)
    xs = torch.empty((P, s.H // 32), dtype=torch.uint8, device=dev)
    moe.quant_act_mxfp8(d.x, xq, xs, routing=rt)
    hq = torch.empty((P, s.I), dtype=torch.uint8, device=dev)
    hs = torch.empty((P, s.I // 32), dtype=torch.uint8, device=dev)
    ws = moe.workspace(max(256, moe.lib().moe_gate_up_workspace_bytes(d.w13.fmt, s.M, s.H, s.I, s.E, s.k, 0)),
                       dev)
    return lambda w13: moe.expert_gate_up(w13, s.M, s.H, s.I, s.E, s.k, routing=rt, a_q=xq, a_s=xs, h_q=hq,
                                          h_s=hs, ws=ws)


def cpu_baseline(inp, logits):
    from oracle import oracle as orc
    s = inp.shape
    rows = np.arange(s.M)
    need = set()
    for r in rows:
        ids, _, _ = orc.topk_row(logits[r], inp.bias, s.k, s.routed_scale)
        need.update(int(e) for e in ids)
    L = orc.Layer(inp, experts=need)
    items = s.M * (s.k + (1 if s.sfmt else 0))
    threads = min(orc.num_cores(), items)
    L.rows(rows, logits=logits, nthreads=threads)  # warm
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        L.rows(rows, logits=logits, nthreads=threads)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), threads


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-gate-up", type=int, default=0,
                    help="only launch the routed gate_up kernel N times (for counter runs)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary of two rocprofv3 counter runs to stdout")
    ap.add_argument("--traffic-command", default="", help="the commands to record in the summary")
    args = ap.parse_args()
    if args.traffic_summary:
        print(traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.workload,
                              args.traffic_command))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the layer is one "
              "GPU's share of an expert/tensor-parallel MoE layer and the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_scaled_fp4_sigmoid_amd import moe, probe, staging, synth

    dev = "cuda"
    name = args.workload
    s = synth.WORKLOADS[name]
    seed = args.seed if args.seed is not None else synth.seed_of(name)
    t0 = time.time()
    inp = synth.make_inputs(name, seed=seed)
    d = staging.to_device(inp, dev)
    log(f"[bench] {name}: inputs drawn and staged in {time.time() - t0:.1f}s")

    # routing of this input (deterministic), for U and the byte model
    layer0 = d.layer()
    out = torch.empty((s.M, s.H), dtype=torch.int16, device=dev)
    res = torch.empty_like(out)
    logits = torch.empty((s.M, s.E), dtype=torch.float32, device=dev)
    ids = torch.empty((s.M, s.k), dtype=torch.int32, device=dev)
    layer0(d.x, d.x, out, res, logits, ids)
    torch.cuda.synchronize()
    U = int(np.unique(ids.cpu().numpy()).size)
    bm = byte_model(s, U)
    copies = args.copies or max(1, math.ceil((1 << 30) / bm["total"]))
    log(f"[bench] U={U} unique experts, routed bytes {bm['routed'] / 1e6:.1f} MB, "
        f"total {bm['total'] / 1e6:.1f} MB, rotating {copies} weight copies")

    layers = [layer0]
    keep = []
    for c in range(1, copies):
        w13, w2 = staging.clone_weights(d.w13), staging.clone_weights(d.w2)
        sh13, sh2 = staging.clone_weights(d.sh13), staging.clone_weights(d.sh2)
        Wr = d.Wr.clone()
        keep.append((w13, w2, sh13, sh2, Wr))
        layers.append(moe.Layer(s.M, s.H, s.E, s.k, s.I, s.I_sh, s.routed_scale, s.eps, Wr, d.bias,
                                w13, w2, sh13, sh2, d.gamma, s.swiglu_limit, s.act_fmt, d.x_global,
                                d.h_globals, d.sh_h_global if s.sfmt == synth.NVFP4 else None))
    stream = torch.cuda.current_stream()

    if args.profile_gate_up:
        gate_up_w = gate_up_alone(moe, s, d, logits, dev)
        for i in range(args.profile_gate_up):
            gate_up_w(d.w13 if i % copies == 0 else keep[i % copies - 1][0])
        torch.cuda.synchronize()
        log(f"[bench] launched routed gate_up {args.profile_gate_up} times")
        return

    def step_eager(i):
        layers[i % copies](d.x, d.x, out, res)

    ms_eager, win_eager = timed(step_eager, args.steps, args.warmup, stream)
    log(f"[bench] eager: {ms_eager * 1e3:.2f} us/step")

    ms_graph = ms_chain = chain = None
    if not args.no_graph:
        graphs = []
        gs = torch.cuda.Stream()
        with torch.cuda.stream(gs):
            for c in range(copies):
                layers[c](d.x, d.x, out, res, stream=gs)
            gs.synchronize()
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=gs):
                    layers[c](d.x, d.x, out, res, stream=gs)
                graphs.append(g)
        torch.cuda.synchronize()
        ms_graph, _ = timed(lambda i: graphs[i % copies].replay(), args.steps, args.warmup, stream)
        log(f"[bench] graph replay, one layer step per graph: {ms_graph * 1e3:.2f} us/step")
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

        full, rem = divmod(args.steps, chain)
        units = [(gchain.replay, chain)] * full + [(graphs[j % copies].replay, 1) for j in range(rem)]
        gchain.replay()  # warm
        torch.cuda.synchronize()
        ms_chain, win_chain = timed_units(units, stream)
        log(f"[bench] graph replay, {chain} layer steps per graph: {ms_chain * 1e3:.2f} us/step")
    # the layer step as it runs fastest: eager launches or the chained graph
    ms, timing, win = ms_eager, "eager launches", win_eager
    if ms_chain is not None and ms_chain < ms_eager:
        ms, timing, win = ms_chain, "graph of %d consecutive layer steps, replayed" % chain, win_chain

    # dominant kernel alone: routed gate_up, timed with HIP events on its stream
    w13s = [d.w13] + [k_[0] for k_ in keep]
    gate_up_w = gate_up_alone(moe, s, d, logits, dev)

    def gate_up(i):
        gate_up_w(w13s[i % copies])

    ms_gu, win_gu = timed(gate_up, args.steps, args.warmup, stream)
    gu_gbps = bm["gate_up_launch"] / (ms_gu * 1e-3) / 1e9
    log(f"[bench] routed gate_up alone: {ms_gu * 1e3:.2f} us, {gu_gbps:.0f} GB/s")

    # calibration: a streaming read of 4 GiB (the practical HBM read rate) and
    # a plain 1 GiB device copy (context)
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
    log(f"[bench] stream read 4 GiB: {read_gbps:.0f} GB/s (rows of {read_row} B); "
        f"device copy 1 GiB: {copy_gbps:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        lg = logits.cpu().numpy()
        t_cpu, threads = cpu_baseline(inp, lg)
        cpu = {"value": round(bm["routed"] / t_cpu / 1e9, 4), "unit": "GB/s",
               "us_per_step": round(t_cpu * 1e6, 1), "cores": threads, "kind": "oracle",
               "sample": f"the whole {s.M}-row step (all rows, all {U} routed experts + shared), "
                         "1 warm run then the median of 3"}
        log(f"[bench] oracle on host: {t_cpu * 1e3:.1f} ms/step with {threads} threads")

    value = bm["routed"] / (ms * 1e-3) / 1e9
    line = {
        "metric": "MoE layer effective weight GB/s (unique selected experts' weight bytes / step time) "
                  "at 1-384 rows, with us/step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "us_per_step_eager": round(ms_eager * 1e3, 2),
        "us_per_step_graph": None if ms_graph is None else round(ms_graph * 1e3, 2),
        "us_per_step_graph_chain": None if ms_chain is None else round(ms_chain * 1e3, 2),
        "timing": timing,
        "us_per_step_windows": window_stats(win),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4xfp4->fp32" if s.act_fmt == synth.ACT_NVFP4 else "fp4xfp8->fp32",
        "data": "synthetic (seeded; weights drawn N(0,0.02) and encoded offline)",
        "config": {"workload": name, "rows": s.M, "hidden": s.H, "experts": s.E, "top_k": s.k,
                   "intermediate": s.I, "weights": synth.FMT_NAMES[s.wfmt],
                   "activations": "nvfp4" if s.act_fmt == synth.ACT_NVFP4 else "mxfp8",
                   "shared": synth.FMT_NAMES[s.sfmt], "unique_experts": U,
                   "weight_copies": copies, "parallelism": "single GPU"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "stream_read_GBps": round(read_gbps, 1),
        "frac_of_stream_read": round(value / read_gbps, 4),
        "total_alg_GBps": round(bm["total"] / (ms * 1e-3) / 1e9, 2),
        "copy_GBps": round(copy_gbps, 1),
        "roofline": {"kernel": "k_gate_up_fp4 (routed)", "bound": "hbm",
                     "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gu_gbps / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(name),
                     "us_per_launch": round(ms_gu * 1e3, 2),
                     "us_per_launch_windows": window_stats(win_gu),
                     "frac_of_stream_read": round(gu_gbps / read_gbps, 4),
                     "alg_bytes_per_launch": bm["gate_up_launch"]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
