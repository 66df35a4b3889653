"""Seeded synthetic inputs for the gated delta rule workloads.

This module holds input recipes only (shapes, distributions, layouts, seeds) and none
of the method's arithmetic; both the HIP path's tests/benchmark and the fp64 oracle
draw their inputs from here.

Every array is produced per (tensor, sequence, head) slice from its own PCG64 stream,
seeded with ``SeedSequence([seed, tensor_id, s, head])``, so any slice can be
regenerated alone (sampled parity checks at full size) and the result does not depend
on how much of the problem is materialised.  Draws are float64, cast to float32.

Recipe (distributions follow the workload descriptions):
  q, k      N(0, 1), then L2-normalised per (token, head) in float64
  v         N(0, 1)
  g         log-gate, U(g_lo, g_hi) with g_hi = 0 (gates at most one) unless a workload
            says otherwise: one value per (token, head) for the scalar gate, S_k values for
            the per-key-channel gate
  beta      U(0, 1)
  state0    N(0, 0.1^2)
  gy        N(0, 1)           (output cotangent)
  dstate_out N(0, 1)          (final-state cotangent)
Tokens t >= len_s of a sequence are filled with ``pad_value`` (0 by default; NaN in the
tests that prove padded tokens are never read).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TENSORS = ("q", "k", "v", "g", "beta", "state0", "gy", "dstate_out")
_TID = {n: i for i, n in enumerate(TENSORS)}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one problem."""
    name: str
    n_seqs: int
    T: int
    H_k: int
    H_v: int
    S: int
    kda: bool
    C: int                      # checkpoint interval (0: ceil(sqrt(T)))
    g_lo: float                 # log-gate ~ U(g_lo, g_hi)
    seq_lens: tuple | None = None   # None: all T
    packed: bool = False        # q/k/v are row views of one [n_seqs, T, W] buffer
    seed: int = 1000
    g_hi: float = 0.0           # upper end of the log-gate range (above 0: some gates exceed one)
    Sv: int = 0                 # value head size when it differs from the key head size S

    @property
    def S_k(self):
        return self.S

    @property
    def S_v(self):
        return self.Sv or self.S

    @property
    def scale(self):
        return float(np.float32(1.0 / math.sqrt(self.S)))

    @property
    def G(self):
        return self.S if self.kda else 1

    @property
    def lens(self):
        return tuple(self.seq_lens) if self.seq_lens is not None else (self.T,) * self.n_seqs

    @property
    def tokens_heads(self):
        return sum(self.lens) * self.H_v

    @property
    def packed_width(self):
        return 2 * self.H_k * self.S + self.H_v * self.S_v

    def shape_dict(self, **over):
        d = dict(n_seqs=self.n_seqs, T=self.T, H_k=self.H_k, H_v=self.H_v, S_k=self.S,
                 S_v=self.S_v, kda=self.kda, C=self.C, scale=self.scale,
                 seq_lens=list(self.lens))
        d.update(over)
        return d

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


# The five workloads (sizes and distributions as the workload descriptions give them).
WORKLOADS = {
    # tiny scalar gate, 1 seq, 1 q/k head, 1 v head, S=32, T=16, C=4
    "tiny_scalar_s32": Workload("tiny_scalar_s32", 1, 16, 1, 1, 32, False, 4, -1.0, seed=1000),
    # per-key-channel gate, 2 seqs (64 and a ragged 61), 4/4 heads, S=64, C=8
    "kda_ragged_s64": Workload("kda_ragged_s64", 2, 64, 4, 4, 64, True, 8, -0.5,
                               seq_lens=(64, 61), seed=1001),
    # GQA v_repeat 2 with q/k/v as row views of a packed [T, 1024] buffer, S=32, T=256
    "gqa_strided_s32": Workload("gqa_strided_s32", 2, 256, 8, 16, 32, False, 0, -1.0,
                                packed=True, seed=1002),
    # hybrid delta-net layer shape: 4 seqs x 4096, 16 q/k heads, 48 v heads, S=128, C=64,
    # packed [T, 10240] qkv buffer, per-key-channel gate
    "layer_kda_s128": Workload("layer_kda_s128", 4, 4096, 16, 48, 128, True, 64, -0.3,
                               packed=True, seed=1003),
    # long context: 1 seq x 65536, 16/48 heads, S=128, C=256, scalar gate (slow decay)
    "long_scalar_s128": Workload("long_scalar_s128", 1, 65536, 16, 48, 128, False, 256, -0.05,
                                 seed=1004),
}
WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "layer_kda_s128"

# Beyond the five: head size 16 (the layer shape with 16-wide heads; packed [T, 1280] qkv).
EXTRA_WORKLOADS = {
    "layer_kda_s16": Workload("layer_kda_s16", 4, 4096, 16, 48, 16, True, 64, -0.3,
                              packed=True, seed=1005),
}


def _rng(seed, tensor, s, head):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TID[tensor], s, head])))


def _slice(w: Workload, tensor: str, s: int, head: int) -> np.ndarray:
    """One (sequence, head) slice of a tensor, float64, before padding."""
    r = _rng(w.seed, tensor, s, head)
    T, S = w.T, w.S
    if tensor in ("q", "k"):
        x = r.standard_normal((T, S))
        n = np.sqrt(np.sum(x * x, axis=1, keepdims=True))
        return x / n
    if tensor in ("v", "gy"):
        return r.standard_normal((T, w.S_v))
    if tensor == "g":
        return w.g_lo + (w.g_hi - w.g_lo) * r.random((T, w.G))
    if tensor == "beta":
        return r.random(T)
    if tensor == "state0":
        return 0.1 * r.standard_normal((w.S_v, S))
    if tensor == "dstate_out":
        return r.standard_normal((w.S_v, S))
    raise KeyError(tensor)


def _heads(w: Workload, tensor: str) -> int:
    return w.H_k if tensor in ("q", "k") else w.H_v


def make_tensor(w: Workload, tensor: str, seqs=None, heads=None, pad_value=0.0) -> np.ndarray:
    """float32 array in the logical layout, restricted to the given sequences / heads.

    Logical layouts: q, k [n][T][H_k][S_k]; v, gy [n][T][H_v][S_v]; g [n][T][H_v][G];
    beta [n][T][H_v]; state0, dstate_out [n][H_v][S_v][S_k].
    """
    seqs = list(range(w.n_seqs)) if seqs is None else list(seqs)
    heads = list(range(_heads(w, tensor))) if heads is None else list(heads)
    lens = w.lens
    if tensor in ("state0", "dstate_out"):
        out = np.empty((len(seqs), len(heads), w.S_v, w.S), np.float32)
        for a, s in enumerate(seqs):
            for b, h in enumerate(heads):
                out[a, b] = _slice(w, tensor, s, h)
        return out
    if tensor == "beta":
        out = np.empty((len(seqs), w.T, len(heads)), np.float32)
    elif tensor == "g":
        out = np.empty((len(seqs), w.T, len(heads), w.G), np.float32)
    else:
        width = w.S if tensor in ("q", "k") else w.S_v
        out = np.empty((len(seqs), w.T, len(heads), width), np.float32)
    for a, s in enumerate(seqs):
        for b, h in enumerate(heads):
            x = _slice(w, tensor, s, h).astype(np.float32)
            if tensor == "beta":
                out[a, :, b] = x
            else:
                out[a, :, b] = x.reshape(w.T, -1)
        if lens[s] < w.T:
            out[a, lens[s]:] = pad_value
    return out


def make_all(w: Workload, seqs=None, key_heads=None, pad_value=0.0, with_cotangents=True):
    """All inputs for the given sequences and key heads (value heads h with h mod H_k in
    key_heads, increasing).  Returns (dict of float32 arrays, value-head list)."""
    kh = list(range(w.H_k)) if key_heads is None else list(key_heads)
    vh = [h for h in range(w.H_v) if (h % w.H_k) in kh]
    names = TENSORS if with_cotangents else TENSORS[:6]
    out = {}
    for n in names:
        heads = kh if n in ("q", "k") else vh
        out[n] = make_tensor(w, n, seqs=seqs, heads=heads, pad_value=pad_value)
    return out, vh


def sub_workload(w: Workload, seqs, key_heads) -> Workload:
    """The workload restricted to some sequences and key heads, as a problem of its own:
    the kept value heads keep their key head under the modulo map (h -> h mod H_k)."""
    lens = [w.lens[s] for s in seqs]
    r = w.H_v // w.H_k
    return w.replace(name=w.name + "_sub", n_seqs=len(seqs), H_k=len(key_heads),
                     H_v=len(key_heads) * r, seq_lens=tuple(lens))


HALF_INPUTS = ("q", "k", "v", "g", "beta", "gy")


def round_inputs(arrays: dict, kind: str) -> dict:
    """The arrays with q, k, v, g, beta, gy rounded to the nearest "f16" or "bf16" value
    (ties to even), still stored as float32: the values a half-precision run receives, so the
    oracle and the device see the same numbers."""
    out = dict(arrays)
    for n in HALF_INPUTS:
        x = np.ascontiguousarray(arrays[n], dtype=np.float32)
        if kind == "f16":
            out[n] = x.astype(np.float16).astype(np.float32)
        elif kind == "bf16":
            u = x.view(np.uint32).astype(np.uint64)
            u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
            out[n] = u.astype(np.uint32).view(np.float32)
        else:
            raise ValueError(kind)
    return out


def pack_qkv(w: Workload, q, k, v) -> np.ndarray:
    """Place q, k, v as row views of one [n, T, W] buffer: q at columns [0, H_k S),
    k at [H_k S, 2 H_k S), v at [2 H_k S, W); head h at offset h S (h S_v for v) in its block."""
    n, T = q.shape[0], q.shape[1]
    HkS = w.H_k * w.S
    buf = np.zeros((n, T, w.packed_width), np.float32)
    buf[:, :, :HkS] = q.reshape(n, T, -1)
    buf[:, :, HkS:2 * HkS] = k.reshape(n, T, -1)
    buf[:, :, 2 * HkS:] = v.reshape(n, T, -1)
    return buf


# The short convolution feeding the layer shape's packed rows: 4 sequences x 4096 tokens,
# d_inner = 2 H_k S + H_v S = 10240 channels, 4 taps (3 carried state rows per sequence).
CONV_LAYER = {"name": "conv_layer_d10240_k4", "n_seqs": 4, "T": 4096, "d_inner": 10240,
              "d_conv": 4, "seed": 1100}


def make_conv(cfg: dict, seqs=None):
    """Seeded inputs of the convolution, float32: sx [n, d_conv - 1 + T, D] and dy [n, T, D]
    standard normal (one generator per sequence, so a sample of sequences is reproducible on
    its own), taps c [D, d_conv] normal with variance 1 / d_conv."""
    n, T, D, K, seed = cfg["n_seqs"], cfg["T"], cfg["d_inner"], cfg["d_conv"], cfg["seed"]
    seqs = list(range(n)) if seqs is None else list(seqs)
    sx = np.empty((len(seqs), T + K - 1, D), np.float32)
    dy = np.empty((len(seqs), T, D), np.float32)
    for i, s in enumerate(seqs):
        r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1, s])))
        sx[i] = r.standard_normal((T + K - 1, D), dtype=np.float32)
        dy[i] = r.standard_normal((T, D), dtype=np.float32)
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0])))
    c = (r.standard_normal((D, K)) / np.sqrt(K)).astype(np.float32)
    return sx, c, dy


# Selective-scan workloads, 4 sequences x 4096 tokens like the recurrence's layer shape:
# a Mamba-2 layer (80 heads of 64, 128 states, one group, one decay per head) and a Mamba-1
# layer (5120 channels, 16 states, one decay per state).
SSM_WORKLOADS = {
    "ssm2_layer_h80_p64_n128": {"n_seqs": 4, "T": 4096, "H": 80, "P": 64, "N": 128, "G": 1,
                                "a_per_state": False, "seed": 1400},
    "ssm1_layer_d5120_n16": {"n_seqs": 4, "T": 4096, "H": 5120, "P": 1, "N": 16, "G": 1,
                             "a_per_state": True, "seed": 1401},
}


def make_ssm(cfg: dict, seed=None):
    """Seeded float32 inputs and cotangents of one scan: x, B, C, gy, gs ~ N(0, 1),
    s0 ~ N(0, 0.1^2), raw steps dt ~ U(-6, -2) (softplus(dt) in about [0.0025, 0.13]),
    decays A = -exp(U(0, log 16)) per head, or A[h][n] = -(n + 1) per state (all negative)."""
    n, T, H, P, N, G = (cfg[k] for k in ("n_seqs", "T", "H", "P", "N", "G"))
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [cfg.get("seed", 0) if seed is None else seed, 7])))
    f32 = np.float32
    out = {
        "s0": (0.1 * r.standard_normal((n, H, P, N), dtype=f32)).astype(f32),
        "x": r.standard_normal((n, T, H, P), dtype=f32),
        "dt": r.uniform(-6.0, -2.0, (n, T, H)).astype(f32),
        "B": r.standard_normal((n, T, G, N), dtype=f32),
        "C": r.standard_normal((n, T, G, N), dtype=f32),
        "gy": r.standard_normal((n, T, H, P), dtype=f32),
        "gs": r.standard_normal((n, H, P, N), dtype=f32),
    }
    if cfg["a_per_state"]:
        out["A"] = np.ascontiguousarray(np.broadcast_to(-(np.arange(N, dtype=f32) + 1), (H, N)))
    else:
        out["A"] = (-np.exp(r.uniform(0.0, np.log(16.0), H))).astype(f32)
    return out
