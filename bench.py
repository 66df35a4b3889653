"""Throughput of the gated delta rule forward + backward on one MI355X.

One step = gdn_fwd then gdn_bwd (reusing the forward's snapshots) over the whole workload,
inputs already resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--input-dtype f32|f16|bf16]
                  [--no-cpu-baseline]

Metric: tokens x value-heads per second, fwd+bwd, and the fraction of the FP32 vector peak
(157.3 TFLOP/s) that the credited work reaches.  Credited work per token x head is
28 S^2 flops: forward 7 S^2, segment replay 5 S^2, reverse walk 16 S^2.

The same line, with the roofline of each op's own bound, for the other entry points:
  --op ssm_conv   the short convolution fwd+bwd on the layer shape's packed rows (HBM)
  --op l2norm     the q/k row normalisation fwd+bwd on the same rows (HBM)
  --op ssm_scan   the selective scan fwd+bwd, --workload ssm2_layer_h80_p64_n128 (default) or
                  ssm1_layer_d5120_n16 (FP32 VALU)
Helpers for the counter summaries in profiles/: --copy-calibration MIB, --pmc-summary DIR.
"""
from __future__ import annotations

import argparse
import json

import numpy as np
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_VALU = 157.3e12      # 256 CU x 2.4 GHz x 256 flop/clk (packed FMA)
METRIC = "GATED_DELTA_NET fwd+bwd tokens·heads/s at S_v=128; % FP32 VALU peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--input-dtype", choices=("f32", "f16", "bf16"), default="f32",
                    help="element type of q, k, v, g, beta, gy (state and gradients stay fp32)")
    ap.add_argument("--op", choices=("gdn", "ssm_conv", "l2norm", "ssm_scan"), default="gdn",
                    help="gdn: the recurrence fwd+bwd (default); ssm_conv: the short "
                         "convolution fwd+bwd on the layer shape's packed rows; l2norm: the "
                         "q/k row normalisation fwd+bwd on the same rows; ssm_scan: the "
                         "selective scan fwd+bwd (--workload ssm2_layer_h80_p64_n128 or "
                         "ssm1_layer_d5120_n16)")
    ap.add_argument("--cpu-sample-heads", type=int, default=0,
                    help="key heads of sequence 0 in the oracle sample (0: auto)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--pmc-summary", default=None, metavar="DIR",
                    help="summarise rocprofv3 counter runs under DIR (fetch/, write/, cfetch/, "
                         "cwrite/ with run_counter_collection.csv) of --op / --workload into "
                         "its traffic file under profiles/ and exit")
    return ap.parse_args()


# Traffic measurements: per (op, workload), the kernels of the timed call whose HBM bytes make
# the roofline's `traffic`, the file holding the counter summary, and the sources whose hash
# stamps it (a summary is reported only while those sources are unchanged).
_C = "gated_delta_rule_bwd_amd/csrc/"
TRAFFIC = {
    ("gdn", "layer_kda_s128"): {
        "file": "traffic_layer_kda_s128.json",
        "sources": [_C + "gdn_mf.hip", _C + "gdn_kernels.hip", _C + "gdn_api.hip", _C + "gdn_internal.h"],
        "kernels": ("chain_kernel<0, 8>", "colsum_kernel<0>")},
    ("ssm_conv", "conv_layer_d10240_k4"): {
        "file": "traffic_conv_layer_d10240_k4.json",
        "sources": [_C + "ssm_conv.hip", _C + "gdn_internal.h"],
        "kernels": ("conv_kernel<4, 4, true>",)},
    ("l2norm", "l2norm_layer_qk_rows"): {
        "file": "traffic_l2norm_layer_qk_rows.json",
        "sources": [_C + "l2norm.hip", _C + "gdn_internal.h"],
        "kernels": ("l2norm_kernel<4, 16, true>",)},
    ("ssm_scan", "ssm2_layer_h80_p64_n128"): {
        "file": "traffic_ssm2_layer_h80_p64_n128.json",
        "sources": [_C + "ssm_chunk.hip", _C + "ssm_scan.hip", _C + "ssm_common.h", _C + "gdn_api.hip",
                    _C + "gdn_internal.h"],
        "kernels": ("ssm_dsq_kernel<64, 128>", "ssm_chunk_kernel<64, 128>", "ssm_chunk_combine_kernel")},
    ("ssm_scan", "ssm1_layer_d5120_n16"): {
        "file": "traffic_ssm1_layer_d5120_n16.json",
        "sources": [_C + "ssm_scan.hip", _C + "ssm_common.h", _C + "gdn_api.hip", _C + "gdn_internal.h"],
        "kernels": ("ssm_gsw_kernel<true>", "ssm_win16_kernel<true>", "ssm_combine_kernel")},
}


def sources_hash(sources):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_key(name):
    """A kernel's name with its template arguments, without namespaces and parameters."""
    import re
    m = re.search(r"(\w+_kernel(?:<[^()]*>)?)\(", name)
    return m.group(1) if m else name[:64]


def pmc_summary(d, op, workload):
    """Per-dispatch HBM bytes of every kernel from FETCH_SIZE / WRITE_SIZE runs (d/fetch,
    d/write), each scaled by what the same counter reads for the plain copy of
    --copy-calibration (d/cfetch, d/cwrite)."""
    import csv

    def load(sub):
        out, disp = {}, {}
        with open(os.path.join(d, sub, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                k = kernel_key(r["Kernel_Name"])
                out[(k, r["Counter_Name"])] = out.get((k, r["Counter_Name"]), 0.0) + float(r["Counter_Value"])
                disp.setdefault(k, set()).add(r["Dispatch_Id"])
        return out, {k: len(v) for k, v in disp.items()}

    fe, nfe = load("fetch")
    wr, nwr = load("write")
    cf, ncf = load("cfetch")
    cw, ncw = load("cwrite")
    copy = [k for k in ncf if "copyBuffer" in k]
    with open(os.path.join(d, "cfetch.log")) as f:
        cal = json.loads([l for l in f if "copy_calibration_bytes" in l][-1])
    n_copy = sum(ncf[k] for k in copy)
    fetch_scale = n_copy * cal["copy_calibration_bytes"] / (1024 * sum(cf[(k, "FETCH_SIZE")] for k in copy))
    write_scale = n_copy * cal["copy_calibration_bytes"] / (1024 * sum(cw[(k, "WRITE_SIZE")] for k in copy))
    # the counter runs time PMC_CALLS calls of the op (one warm-up step, one timed step); a call
    # may launch a kernel several times (the pieces of a pipelined pass)
    kernels = {}
    for k in nfe:
        if k not in nwr:
            continue
        kernels[k] = {"fetch_bytes": fe[(k, "FETCH_SIZE")] * 1024 * fetch_scale / nfe[k],
                      "write_bytes": wr[(k, "WRITE_SIZE")] * 1024 * write_scale / nwr[k],
                      "dispatches_per_call": nfe[k] / PMC_CALLS}
    spec = TRAFFIC[(op, workload)]
    return {"op": op, "workload": workload, "source_sha256": sources_hash(spec["sources"]),
            "counter_scale": {"fetch": fetch_scale, "write": write_scale},
            "kernels": kernels}


PMC_CALLS = 2   # calls of the op in a counter run (--steps 1 --warmup 1)


def traffic_bytes(op, workload):
    """HBM bytes of one timed call (every launch of the roofline kernels in it) from the
    committed counter summary, or None when there is none or the kernels changed since it was
    taken."""
    spec = TRAFFIC.get((op, workload))
    if spec is None:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", spec["file"])) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("source_sha256") != sources_hash(spec["sources"]):
        return None
    ks = t["kernels"]
    if not all(k in ks for k in spec["kernels"]):
        return None
    return sum((ks[k]["fetch_bytes"] + ks[k]["write_bytes"]) * ks[k].get("dispatches_per_call", 1)
               for k in spec["kernels"])


def copy_calibration(mib):
    """A plain copy of known size: reads and writes mib MiB once per launch (3 launches)."""
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)


def cpu_baseline(w, n_key_heads, n_seqs=2):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload: the first
    n_seqs sequences, the first n_key_heads key heads with all their value heads, full length,
    fwd+bwd."""
    import oracle
    from gated_delta_rule_bwd_amd import inputs as I
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    kh = list(range(n_key_heads))
    seqs = list(range(min(n_seqs, w.n_seqs)))
    arrays, vh = I.make_all(w, seqs=seqs, key_heads=kh)
    sub = I.sub_workload(w, seqs, kh)
    orc = oracle.Oracle(threads=cores)
    shape = sub.shape_dict()
    args = [arrays[n] for n in ("q", "k", "v", "g", "beta", "state0")]
    t0 = time.perf_counter()
    orc.fwd(shape, *args)
    orc.bwd(shape, *args, arrays["gy"], arrays["dstate_out"])
    dt = time.perf_counter() - t0
    th = sub.tokens_heads
    used = min(cores, len(kh) * len(seqs))  # the oracle threads over (sequence, key head) pairs
    return {"value": th / dt, "unit": "tokens·heads/s", "cores": used, "kind": "oracle",
            "sample": f"sequences 0..{len(seqs) - 1}, key heads 0..{len(kh) - 1} with their "
                      f"{len(vh)} value heads, {w.T} tokens each ({th} tokens·heads), fp64 "
                      f"fwd+bwd, {dt:.1f} s"}


PEAK_HBM = 8.0e12              # MI355X HBM3E, bytes/s


def bench_conv(args):
    """The convolution forward + backward (gdn_ssm_conv_fwd then gdn_ssm_conv_bwd) on the
    layer shape's packed rows.  Algorithmic bytes per launch: forward reads sx and c and
    writes y; backward reads dy and c and writes d_sx, each once."""
    import torch
    from gated_delta_rule_bwd_amd import binding as B
    from gated_delta_rule_bwd_amd import inputs as I
    cfg = I.CONV_LAYER
    n, T, D, K = cfg["n_seqs"], cfg["T"], cfg["d_inner"], cfg["d_conv"]
    sx, c, dy = I.make_conv(cfg)
    dev = "cuda:0"
    gsx, gc, gdy = (torch.from_numpy(a).to(dev) for a in (sx, c, dy))
    del sx, dy
    y = torch.empty((n, T, D), device=dev)
    dsx = torch.empty((n, T + K - 1, D), device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        B.ssm_conv_fwd(gsx, gc, y, stream)
        B.ssm_conv_bwd(gdy, gc, dsx, stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for e0, e1, e2 in ev:
        e0.record(stream)
        B.ssm_conv_fwd(gsx, gc, y, stream)
        e1.record(stream)
        B.ssm_conv_bwd(gdy, gc, dsx, stream)
        e2.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    bwd_ms = sum(b.elapsed_time(e) for _, b, e in ev) / args.steps
    rows_in = n * (T + K - 1) * D * 4
    rows_out = n * T * D * 4
    taps = D * K * 4
    launch_bytes = rows_in + rows_out + taps          # the same for both directions
    tc = n * T * D
    out = {
        "metric": "SSM_CONV fwd+bwd tokens·channels/s; % HBM peak",
        "value": tc / (ms / 1e3), "unit": "tokens·channels/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "n_seqs": n, "T": T, "d_inner": D, "d_conv": K},
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "roofline": {"bound": "hbm", "kernel": "conv_kernel (backward launch)",
                     "achieved": launch_bytes / (bwd_ms / 1e3) / 1e9, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": launch_bytes / (bwd_ms / 1e3) / PEAK_HBM,
                     "traffic": traffic_bytes("ssm_conv", cfg["name"])},
        "fwd_GBps": launch_bytes / (fwd_ms / 1e3) / 1e9,
    }
    if not args.no_cpu_baseline:
        import oracle.ssm_conv as OC
        s_sx, s_c, s_dy = I.make_conv(cfg, seqs=[0])
        t0 = time.perf_counter()
        reps = 0
        while True:
            OC.conv_fwd(s_sx, s_c)
            OC.conv_bwd(s_dy, s_c)
            reps += 1
            dt = time.perf_counter() - t0
            if dt > 10.0:
                break
        out["cpu_baseline"] = {"value": reps * T * D / dt, "unit": "tokens·channels/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"sequence 0 ({T} tokens x {D} channels), fp64 fwd+bwd, "
                                         f"{reps} repetitions in {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def bench_l2norm(args):
    """The q/k row normalisation forward + backward (gdn_l2norm_fwd then gdn_l2norm_bwd) on
    the layer shape: 4 x 4096 tokens, the 32 q and k heads of 128 at the start of each packed
    [10240]-float token row; the cotangent and the outputs are contiguous.  Algorithmic bytes:
    the forward reads x and writes y, the backward reads x and dy and writes dx, once each."""
    import torch
    from gated_delta_rule_bwd_amd import binding as B
    n, T, H, W, eps = 4, 4096, 32, 128, 1e-6
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(1200)
    buf = torch.randn((n, T, 10240), device=dev, generator=g)
    x = buf[:, :, :H * W].unflatten(2, (H, W))
    dy = torch.randn((n, T, H, W), device=dev, generator=g)
    y = torch.empty_like(dy)
    dx = torch.empty_like(dy)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        B.l2norm_fwd(x, y, eps, stream)
        B.l2norm_bwd(x, dy, dx, eps, stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for e0, e1, e2 in ev:
        e0.record(stream)
        B.l2norm_fwd(x, y, eps, stream)
        e1.record(stream)
        B.l2norm_bwd(x, dy, dx, eps, stream)
        e2.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    bwd_ms = sum(b.elapsed_time(e) for _, b, e in ev) / args.steps
    tensor = n * T * H * W * 4
    rows = n * T * H
    out = {
        "metric": "L2-norm (q/k rows) fwd+bwd rows/s; % HBM peak",
        "value": rows / (ms / 1e3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "l2norm_layer_qk_rows", "n_seqs": n, "T": T, "H": H, "W": W},
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "roofline": {"bound": "hbm", "kernel": "l2norm_kernel (backward launch)",
                     "achieved": 3 * tensor / (bwd_ms / 1e3) / 1e9, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": 3 * tensor / (bwd_ms / 1e3) / PEAK_HBM,
                     "traffic": traffic_bytes("l2norm", "l2norm_layer_qk_rows")},
        "fwd_GBps": 2 * tensor / (fwd_ms / 1e3) / 1e9,
    }
    if not args.no_cpu_baseline:
        import oracle.l2norm as OL
        xs = x[0].cpu().numpy()          # sample: sequence 0, all its rows
        dys = dy[0].cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while True:
            OL.l2norm_fwd(xs, eps)
            OL.l2norm_bwd(xs, dys, eps)
            reps += 1
            dt = time.perf_counter() - t0
            if dt > 10.0:
                break
        out["cpu_baseline"] = {"value": reps * T * H / dt, "unit": "rows/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"sequence 0 ({T} tokens x {H} heads of {W}), fp64 "
                                         f"fwd+bwd, {reps} repetitions in {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def bench_ssm(args):
    """The selective scan forward + backward (gdn_ssm_fwd, then gdn_ssm_bwd reusing its window
    states) on a layer-sized workload.  Credited work per token x state element: forward 5
    flops (decay, input, readout), backward 12 (window replay 3, reverse walk 9) -- the
    per-token recurrence's count, also for the Mamba-2 shape, whose backward runs in 32-token
    chunks on the fp32 matrix cores (the same 157.3 TFLOP/s peak as the vector ALUs)."""
    import torch
    from gated_delta_rule_bwd_amd import binding as B
    from gated_delta_rule_bwd_amd import inputs as I
    name = args.workload or "ssm2_layer_h80_p64_n128"
    cfg = I.SSM_WORKLOADS[name]
    arr = I.make_ssm(cfg)
    dev = "cuda:0"
    g = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in arr.items()}
    del arr
    p = B.ssm_problem_from(g["x"], g["B"], g["A"], True)
    ws = torch.empty(max(B.ssm_workspace_size(p), 16) // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(g["x"])
    s_out = torch.empty_like(g["s0"])
    total, _ = B.ssm_grad_layout(p)
    gp = torch.empty(total, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        B.ssm_fwd(p, g["s0"], g["x"], g["dt"], g["A"], g["B"], g["C"], y, s_out, ws, stream)

    def bwd():
        B.ssm_bwd(p, g["s0"], g["x"], g["dt"], g["A"], g["B"], g["C"], g["gy"], g["gs"], gp, ws,
                  flags=B.BWD_REUSE_SNAPSHOTS, stream=stream)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for e0, e1, e2 in ev:
        e0.record(stream)
        fwd()
        e1.record(stream)
        bwd()
        e2.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    bwd_ms = sum(b.elapsed_time(e) for _, b, e in ev) / args.steps
    n, T, H, P, N = (cfg[k] for k in ("n_seqs", "T", "H", "P", "N"))
    elems = n * T * H * P * N                     # token x state-element steps
    bwd_flops = 12 * elems
    chunked = not cfg["a_per_state"] and P == 64 and N == 128
    out = {
        "metric": "SSM_SCAN fwd+bwd token·state-element steps/s; % FP32 VALU peak",
        "value": elems / (ms / 1e3), "unit": "token·state-elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, **{k: cfg[k] for k in ("n_seqs", "T", "H", "P", "N", "G",
                                                             "a_per_state")}},
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "pct_fp32_valu_peak": 100.0 * 17 * elems / (ms / 1e3) / PEAK_FP32_VALU,
        "roofline": {"bound": "mfma" if chunked else "alu",
                     "kernel": "gdn_ssm_bwd (" + " + ".join(TRAFFIC[("ssm_scan", name)]["kernels"]) + ")",
                     "achieved": bwd_flops / (bwd_ms / 1e3) / 1e12, "peak": PEAK_FP32_VALU / 1e12,
                     "unit": "TFLOP/s", "frac": bwd_flops / (bwd_ms / 1e3) / PEAK_FP32_VALU,
                     "traffic": traffic_bytes("ssm_scan", name)},
    }
    if not args.no_cpu_baseline:
        import oracle.ssm_scan as OS
        a = I.make_ssm(cfg)
        hs = 1 if cfg["P"] > 1 else 64           # sample: sequence 0, the first hs heads
        sub = {"s0": a["s0"][:1, :hs], "x": a["x"][:1, :, :hs], "dt": a["dt"][:1, :, :hs],
               "A": a["A"][:hs], "B": a["B"][:1], "C": a["C"][:1], "gy": a["gy"][:1, :, :hs],
               "gs": a["gs"][:1, :hs]}
        t0 = time.perf_counter()
        reps = 0
        while True:
            OS.ssm_fwd(sub["s0"], sub["x"], sub["dt"], sub["A"], sub["B"], sub["C"])
            OS.ssm_bwd(sub["s0"], sub["x"], sub["dt"], sub["A"], sub["B"], sub["C"], sub["gy"], sub["gs"])
            reps += 1
            dt_s = time.perf_counter() - t0
            if dt_s > 10.0:
                break
        se = T * hs * P * N
        out["cpu_baseline"] = {"value": reps * se / dt_s, "unit": "token·state-elements/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"sequence 0, heads 0..{hs - 1} ({T} tokens, {se} "
                                         f"token·state-elements), fp64 fwd+bwd, {reps} "
                                         f"repetitions in {dt_s:.1f} s"}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.op != "gdn" and not (args.pmc_summary or args.copy_calibration):
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        {"ssm_conv": bench_conv, "l2norm": bench_l2norm, "ssm_scan": bench_ssm}[args.op](args)
        return
    if args.pmc_summary:
        from gated_delta_rule_bwd_amd import inputs as I
        wl = args.workload or {"gdn": I.HEADLINE, "ssm_conv": I.CONV_LAYER["name"],
                               "l2norm": "l2norm_layer_qk_rows",
                               "ssm_scan": "ssm2_layer_h80_p64_n128"}[args.op]
        summ = pmc_summary(args.pmc_summary, args.op, wl)
        with open(os.path.join(ROOT, "profiles", TRAFFIC[(args.op, wl)]["file"]), "w") as f:
            json.dump(summ, f, indent=1)
        print(json.dumps(summ, indent=1))
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); every (sequence, "
              "head) unit is independent, so more GPUs would shard units without exchange "
              "beyond the grouped-head dq/dk sum.", file=sys.stderr)
        sys.exit(2)
    import torch
    from gated_delta_rule_bwd_amd import inputs as I
    from gated_delta_rule_bwd_amd.device import DeviceCase

    name = args.workload or I.HEADLINE
    w = I.WORKLOADS[name] if name in I.WORKLOADS else I.EXTRA_WORKLOADS[name]
    arrays, _ = I.make_all(w)
    in_dtype = torch.float32
    if args.input_dtype != "f32":
        arrays = I.round_inputs(arrays, args.input_dtype)
        in_dtype = torch.float16 if args.input_dtype == "f16" else torch.bfloat16
    dc = DeviceCase(w, arrays, device="cuda:0", in_dtype=in_dtype)
    del arrays
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        dc.fwd(stream)
        dc.bwd(reuse=True, stream=stream)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for e0, e1, e2 in ev:
        e0.record(stream)
        dc.fwd(stream)
        e1.record(stream)
        dc.bwd(reuse=True, stream=stream)
        e2.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    bwd_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps
    ms = total_ms / args.steps
    step_ms = sorted(a.elapsed_time(c) for a, _, c in ev)   # each step's fwd + bwd alone
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])

    S = w.S
    S2 = w.S_k * w.S_v                 # state elements (S^2 for square heads)
    th = w.tokens_heads
    value = th / (ms / 1e3)
    credited = 28 * S2 * th
    bwd_flops = 21 * S2 * th           # segment replay 5 S^2 + reverse walk 16 S^2
    achieved = bwd_flops / (bwd_ms / 1e3)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "input_dtype": args.input_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n_seqs": w.n_seqs, "T": w.T, "H_k": w.H_k,
                   "H_v": w.H_v, "S_k": w.S_k, "S_v": w.S_v, "gate": "kda" if w.kda else "scalar",
                   "C": w.C, "layout": "q/k/v row views of a packed buffer" if w.packed
                   else "contiguous", "tokens_heads": th},
        "pct_fp32_valu_peak": 100.0 * credited / (ms / 1e3) / PEAK_FP32_VALU,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "median_step_ms": median_ms,        # the median over the timed steps (value uses the mean)
        # head size 128 runs on the fp32 matrix cores (dense fp32 MFMA peak, the same figure as
        # the fp32 vector peak); the small heads on the vector ALUs
        "roofline": {"bound": "mfma" if S2 == 128 * 128 else "alu",
                     "kernel": "gdn_bwd (chain_kernel + colsum_kernel)" if S2 == 128 * 128 else
                     "gdn_bwd (bwd_kernel" + (" + combine_kernel)" if w.H_v != w.H_k else ")"),
                     "achieved": achieved / 1e12, "peak": PEAK_FP32_VALU / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU,
                     "traffic": traffic_bytes("gdn", w.name)},
    }
    if not args.no_cpu_baseline:
        cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8
        nkh = args.cpu_sample_heads or max(1, min(w.H_k, cores))
        out["cpu_baseline"] = cpu_baseline(w, nkh)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
