"""Shared pieces of the GPU tests: running the HIP path and the oracle on one workload."""
from __future__ import annotations

import os
import sys
import threading

import numpy as np

from gated_delta_rule_bwd_amd import inputs as I

REGIONS_FWD = ("y", "state_out")
REGIONS_BWD = ("dq", "dk", "dv", "dg", "dbeta", "dstate")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def oracle_results(w: I.Workload, arrays: dict, threads=None):
    import oracle
    orc = oracle.Oracle(threads=threads or min(16, os.cpu_count() or 1))
    shape = w.shape_dict()
    args = [arrays[n] for n in ("q", "k", "v", "g", "beta", "state0")]
    y, so = orc.fwd(shape, *args)
    d = orc.bwd(shape, *args, arrays["gy"], arrays.get("dstate_out"))
    out = {"y": y, "state_out": so}
    out.update(d)
    return out


def oracle_sampled(w: I.Workload, seqs, key_heads, threads=None):
    """Oracle on the sub-problem made of some sequences and key heads (all value heads of
    those key heads).  Each value head is run as a problem of its own, in parallel, and
    dq/dk are summed over the value heads of a key head in increasing order."""
    import oracle
    key_heads = sorted(key_heads)
    arrays, vh = I.make_all(w, seqs=seqs, key_heads=key_heads)
    sub = I.sub_workload(w, seqs, key_heads)
    r = w.H_v // w.H_k
    nk = len(key_heads)
    jobs = []
    for j in range(len(vh)):
        kh = j % nk
        one = {n: arrays[n] for n in arrays}
        for n in ("v", "g", "beta", "gy"):
            one[n] = arrays[n][:, :, j:j + 1]
        for n in ("state0", "dstate_out"):
            one[n] = arrays[n][:, j:j + 1]
        for n in ("q", "k"):
            one[n] = arrays[n][:, :, kh:kh + 1]
        jobs.append(one)
    shape1 = sub.shape_dict(H_k=1, H_v=1)
    res = [None] * len(jobs)

    def run(j):
        orc = oracle.Oracle(threads=1)
        a = jobs[j]
        args = [a[n] for n in ("q", "k", "v", "g", "beta", "state0")]
        y, so = orc.fwd(shape1, *args)
        d = orc.bwd(shape1, *args, a["gy"], a["dstate_out"])
        d.update(y=y, state_out=so)
        res[j] = d

    ths = [threading.Thread(target=run, args=(j,)) for j in range(len(jobs))]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    out = {}
    for n in ("y", "dv", "dg", "dbeta"):
        out[n] = np.concatenate([x[n] for x in res], axis=2)
    for n in ("state_out", "dstate"):
        out[n] = np.concatenate([x[n] for x in res], axis=1)
    for n in ("dq", "dk"):
        acc = np.zeros_like(res[0][n][:, :, 0:1]).repeat(nk, axis=2)
        for m in range(r):              # value heads of a key head, increasing h
            for kh in range(nk):
                acc[:, :, kh] += res[m * nk + kh][n][:, :, 0]
        out[n] = acc
    return out, vh


def gpu_subset(res: dict, w: I.Workload, seqs, key_heads, vh):
    seqs = list(seqs)
    out = {}
    for n in ("y", "dv", "dg", "dbeta"):
        out[n] = res[n][seqs][:, :, vh]
    for n in ("state_out", "dstate"):
        out[n] = res[n][seqs][:, vh]
    for n in ("dq", "dk"):
        out[n] = res[n][seqs][:, :, sorted(key_heads)]
    return out
