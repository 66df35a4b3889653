"""Throughput of the gated delta rule forward + backward on one MI355X.

One step = gdn_fwd then gdn_bwd (reusing the forward's snapshots) over the whole workload,
inputs already resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Metric: tokens x value-heads per second, fwd+bwd, and the fraction of the FP32 vector peak
(157.3 TFLOP/s) that the credited work reaches.  Credited work per token x head is
28 S^2 flops: forward 7 S^2, segment replay 5 S^2, reverse walk 16 S^2.
"""
from __future__ import annotations

import argparse
import json
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
    ap.add_argument("--cpu-sample-heads", type=int, default=0,
                    help="key heads of sequence 0 in the oracle sample (0: auto)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


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


def cpu_baseline(w, n_key_heads):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload: sequence 0,
    the first n_key_heads key heads with all their value heads, full length, fwd+bwd."""
    import oracle
    from gated_delta_rule_bwd_amd import inputs as I
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    kh = list(range(n_key_heads))
    arrays, vh = I.make_all(w, seqs=[0], key_heads=kh)
    sub = I.sub_workload(w, [0], kh)
    orc = oracle.Oracle(threads=cores)
    shape = sub.shape_dict()
    args = [arrays[n] for n in ("q", "k", "v", "g", "beta", "state0")]
    t0 = time.perf_counter()
    orc.fwd(shape, *args)
    orc.bwd(shape, *args, arrays["gy"], arrays["dstate_out"])
    dt = time.perf_counter() - t0
    th = sub.tokens_heads
    used = min(cores, len(kh))  # the oracle threads over (sequence, key head) pairs
    return {"value": th / dt, "unit": "tokens·heads/s", "cores": used, "kind": "oracle",
            "sample": f"sequence 0, key heads 0..{len(kh) - 1} with their {len(vh)} value heads, "
                      f"{w.T} tokens each ({th} tokens·heads), fp64 fwd+bwd, {dt:.1f} s"}


def main():
    args = parse()
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

    w = I.WORKLOADS[args.workload or I.HEADLINE]
    arrays, _ = I.make_all(w)
    dc = DeviceCase(w, arrays, device="cuda:0")
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

    S = w.S
    th = w.tokens_heads
    value = th / (ms / 1e3)
    credited = 28 * S * S * th
    bwd_flops = 21 * S * S * th        # segment replay 5 S^2 + reverse walk 16 S^2
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
        "data": "synthetic",
        "config": {"workload": w.name, "n_seqs": w.n_seqs, "T": w.T, "H_k": w.H_k,
                   "H_v": w.H_v, "S_k": S, "S_v": S, "gate": "kda" if w.kda else "scalar",
                   "C": w.C, "layout": "q/k/v row views of a packed buffer" if w.packed
                   else "contiguous", "tokens_heads": th},
        "pct_fp32_valu_peak": 100.0 * credited / (ms / 1e3) / PEAK_FP32_VALU,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "roofline": {"bound": "alu", "kernel": "gdn_bwd (bwd_kernel + grouped-head combine)",
                     "achieved": achieved / 1e12, "peak": PEAK_FP32_VALU / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU, "traffic": None},
    }
    if not args.no_cpu_baseline:
        cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8
        nkh = args.cpu_sample_heads or max(1, min(w.H_k, cores))
        out["cpu_baseline"] = cpu_baseline(w, nkh)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
