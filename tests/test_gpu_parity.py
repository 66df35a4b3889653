"""HIP path (through the C ABI) against the fp64 oracle, on the GPU."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gated_delta_rule_bwd_amd import inputs as I  # noqa: E402
from compare import check  # noqa: E402
from gpu_cases import (REGIONS_BWD, REGIONS_FWD, gpu_subset, log, oracle_results,  # noqa: E402
                       oracle_sampled)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd.device import DeviceCase  # loads libgdn.so
    return DeviceCase


def run_case(DeviceCase, w, arrays, reuse=True, **kw):
    dc = DeviceCase(w, arrays, **kw)
    dc.fwd()
    dc.bwd(reuse=reuse)
    torch.cuda.synchronize()
    return dc, dc.results_numpy()


SMALL = ["tiny_scalar_s32", "kda_ragged_s64", "gqa_strided_s32"]


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("reuse", [True, False])
def test_parity_full(dev, name, reuse):
    w = I.WORKLOADS[name]
    log(f"[parity] {name} reuse={reuse} lens={w.lens}")
    arrays, _ = I.make_all(w)
    _, got = run_case(dev, w, arrays, reuse=reuse)
    ref = oracle_results(w, arrays)
    rep = check(got, ref, REGIONS_FWD + REGIONS_BWD)
    log(f"[parity] {name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


def test_parity_layer_shape_full(dev):
    """Full-size layer shape in the benchmark's launch configuration, every unit against the
    oracle: the oracle runs one sequence at a time (its 16 key heads with their 48 value heads,
    each value head a problem of its own on the host cores)."""
    w = I.WORKLOADS["layer_kda_s128"]
    log(f"[parity] {w.name} full size, every (sequence, key head) group")
    arrays, _ = I.make_all(w)
    _, got = run_case(dev, w, arrays, reuse=True)
    del arrays
    khs = list(range(w.H_k))
    for s in range(w.n_seqs):
        ref, vh = oracle_sampled(w, [s], khs)
        rep = check(gpu_subset(got, w, [s], khs, vh), ref, REGIONS_FWD + REGIONS_BWD)
        log(f"[parity] {w.name} seq {s}, all key heads: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


def test_parity_s128_many_units(dev):
    """512 units (four sequences of 128 value heads over 32 key heads, ragged, KDA), so 512
    workgroups run at once; every unit against the oracle."""
    w = I.Workload("s128_many_units", 4, 40, 32, 128, 128, True, 16, -0.3, seq_lens=(40, 33, 17, 40),
                   seed=521)
    log(f"[parity] {w.name} lens={w.lens}")
    arrays, _ = I.make_all(w)
    _, got = run_case(dev, w, arrays, reuse=True)
    rep = check(got, oracle_results(w, arrays), REGIONS_FWD + REGIONS_BWD)
    log(f"[parity] {w.name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


def test_layer_shape_bf16_inputs_bitwise(dev):
    """Full-size layer shape with bf16 inputs, as the benchmark's bf16 mode launches it: every
    output is bitwise equal to the fp32-input run on the same (rounded) values, which holds at
    any size because the kernels widen each input exactly at the load; the fp32 kernels' own
    parity at this shape is checked in full against the oracle above."""
    w = I.WORKLOADS["layer_kda_s128"]
    log(f"[parity] {w.name} full size, bf16 inputs against fp32 inputs holding the same values")
    arrays = I.round_inputs(I.make_all(w)[0], "bf16")
    outs = []
    for dt in (torch.bfloat16, torch.float32):
        dc = dev(w, arrays, in_dtype=dt)
        dc.fwd()
        dc.bwd(reuse=True)
        torch.cuda.synchronize()
        outs.append((dc.y.clone(), dc.state_out.clone(), dc.grad.clone()))
        del dc
    for name, a, b in zip(("y", "state_out", "grad"), *outs):
        assert torch.equal(a, b), name
    assert bool(torch.isfinite(outs[0][2]).all())


def test_parity_long_context_full(dev):
    """Full-size long-context workload (one 65536-token sequence, 48 value heads, interval
    256, scalar gate), every unit against the oracle, four key heads (twelve value heads) at a
    time."""
    w = I.WORKLOADS["long_scalar_s128"]
    log(f"[parity] {w.name} full size, every key head")
    arrays, _ = I.make_all(w)
    _, got = run_case(dev, w, arrays, reuse=True)
    del arrays
    for k0 in range(0, w.H_k, 4):
        khs = list(range(k0, min(w.H_k, k0 + 4)))
        ref, vh = oracle_sampled(w, [0], khs)
        rep = check(gpu_subset(got, w, [0], khs, vh), ref, REGIONS_FWD + REGIONS_BWD)
        log(f"[parity] {w.name} key heads {khs}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


# Head size 16: one wave per unit (16 rows, one column per lane).
S16_CASES = {
    "kda_ragged": I.Workload("s16_kda_ragged", 2, 64, 2, 4, 16, True, 8, -0.5,
                             seq_lens=(64, 37), seed=601),
    "scalar_gqa_packed": I.Workload("s16_scalar_gqa", 2, 100, 2, 6, 16, False, 0, -1.0,
                                    packed=True, seed=602),
}


@pytest.mark.parametrize("name", list(S16_CASES))
@pytest.mark.parametrize("reuse", [True, False])
def test_parity_s16(dev, name, reuse):
    w = S16_CASES[name]
    log(f"[parity] {w.name} reuse={reuse} lens={w.lens}")
    arrays, _ = I.make_all(w)
    _, got = run_case(dev, w, arrays, reuse=reuse)
    rep = check(got, oracle_results(w, arrays), REGIONS_FWD + REGIONS_BWD)
    log(f"[parity] {w.name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


def test_parity_s16_layer_sampled(dev):
    """The layer shape with head size 16 at full size; the oracle checks two groups."""
    w = I.EXTRA_WORKLOADS["layer_kda_s16"]
    arrays, _ = I.make_all(w)
    _, got = run_case(dev, w, arrays, reuse=True)
    del arrays
    for seqs, khs in (([1], [3]), ([2], [12])):
        ref, vh = oracle_sampled(w, seqs, khs)
        rep = check(gpu_subset(got, w, seqs, khs, vh), ref, REGIONS_FWD + REGIONS_BWD)
        log(f"[parity] {w.name} seq {seqs} key heads {khs}: " +
            ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


# Key and value head sizes that differ: the small-head kernels over S_v rows x S_k columns.
RECT_CASES = {
    "k64_v32_kda_ragged": I.Workload("r_k64_v32", 2, 64, 2, 4, 64, True, 8, -0.5,
                                     seq_lens=(64, 45), seed=801, Sv=32),
    "k32_v128_scalar_gqa_packed": I.Workload("r_k32_v128", 2, 80, 2, 6, 32, False, 0, -1.0,
                                             packed=True, seed=802, Sv=128),
    "k128_v64_kda": I.Workload("r_k128_v64", 1, 72, 1, 2, 128, True, 16, -0.3, seed=803, Sv=64),
    "k16_v64_scalar": I.Workload("r_k16_v64", 1, 50, 1, 1, 16, False, 0, -1.0, seed=804, Sv=64),
}


@pytest.mark.parametrize("name", list(RECT_CASES))
@pytest.mark.parametrize("reuse", [True, False])
def test_parity_rectangular_heads(dev, name, reuse):
    w = RECT_CASES[name]
    log(f"[parity] {w.name} S_k={w.S_k} S_v={w.S_v} reuse={reuse} lens={w.lens}")
    arrays, _ = I.make_all(w)
    _, got = run_case(dev, w, arrays, reuse=reuse)
    rep = check(got, oracle_results(w, arrays), REGIONS_FWD + REGIONS_BWD)
    log(f"[parity] {w.name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


# Half-precision inputs (q, k, v, g, beta, gy in fp16 or bf16; state and gradients fp32).
HALF_CASES = {
    "bf16_s128_kda": ("bf16", I.Workload("h_s128_kda", 2, 150, 2, 4, 128, True, 64, -0.3,
                                         seq_lens=(150, 77), packed=True, seed=701)),
    "f16_s128_scalar": ("f16", I.Workload("h_s128_scalar", 1, 140, 1, 3, 128, False, 0, -0.5,
                                          seed=702)),
    "bf16_s32_gqa": ("bf16", I.Workload("h_s32_gqa", 2, 100, 4, 8, 32, False, 0, -1.0,
                                        packed=True, seed=703)),
    "f16_s64_kda": ("f16", I.Workload("h_s64_kda", 2, 64, 2, 2, 64, True, 8, -0.5,
                                      seq_lens=(64, 41), seed=704)),
}
TORCH_HALF = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("name", list(HALF_CASES))
def test_parity_half_inputs(dev, name):
    """Against the oracle on the rounded values, and bitwise equal to the fp32 run on the
    same values (the widening is exact), with the snapshots reused and recomputed and with a
    strided gy."""
    kind, w = HALF_CASES[name]
    log(f"[parity] {w.name} {kind} lens={w.lens}")
    arrays = I.round_inputs(I.make_all(w)[0], kind)
    _, got = run_case(dev, w, arrays, reuse=True, in_dtype=TORCH_HALF[kind])
    rep = check(got, oracle_results(w, arrays), REGIONS_FWD + REGIONS_BWD)
    log(f"[parity] {w.name} {kind}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))
    _, f32 = run_case(dev, w, arrays, reuse=True)
    _, rec = run_case(dev, w, arrays, reuse=False, in_dtype=TORCH_HALF[kind], strided_gy=True)
    for n in got:
        assert np.array_equal(got[n], f32[n]), ("half vs fp32 inputs", n)
        assert np.array_equal(got[n], rec[n]), ("recomputed, strided gy", n)


def test_single_ragged_sequence(dev):
    """A standalone 61-token sequence with an 8-token interval: partial last segment."""
    w = I.WORKLOADS["kda_ragged_s64"].replace(name="kda_t61", n_seqs=1, T=61, seq_lens=None)
    arrays, _ = I.make_all(w)
    _, got = run_case(dev, w, arrays)
    check(got, oracle_results(w, arrays))


def test_one_token_and_empty_sequences(dev):
    w = I.Workload("edge", 3, 5, 2, 4, 64, True, 2, -0.5, seq_lens=(1, 0, 5), seed=77)
    arrays, _ = I.make_all(w)
    _, got = run_case(dev, w, arrays)
    ref = oracle_results(w, arrays)
    check(got, ref)
    # the empty sequence passes state and cotangent through bit for bit
    assert np.array_equal(got["state_out"][1], arrays["state0"][1])
    assert np.array_equal(got["dstate"][1], arrays["dstate_out"][1])


def test_t1_zero_state(dev):
    w = I.Workload("t1", 1, 1, 1, 1, 128, False, 0, -1.0, seed=78)
    arrays, _ = I.make_all(w)
    arrays["state0"][:] = 0
    _, got = run_case(dev, w, arrays)
    check(got, oracle_results(w, arrays))


def test_padded_tokens_are_never_read(dev):
    """NaN in every padded token of every per-token input changes no bit of any output."""
    w = I.WORKLOADS["kda_ragged_s64"]
    arrays, _ = I.make_all(w)
    nan_arrays, _ = I.make_all(w, pad_value=np.nan)
    _, a = run_case(dev, w, arrays)
    _, b = run_case(dev, w, nan_arrays)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
    for s, L in enumerate(w.lens):
        for n in ("y", "dq", "dk", "dv", "dg", "dbeta"):
            assert not np.any(b[n][s, L:]), n


def test_null_final_state_cotangent(dev):
    w = I.WORKLOADS["tiny_scalar_s32"]
    arrays, _ = I.make_all(w)
    arrays["dstate_out"] = None
    _, got = run_case(dev, w, arrays)
    ref_arrays = dict(arrays, dstate_out=np.zeros((1, 1, 32, 32), np.float32))
    check(got, oracle_results(w, ref_arrays))


def test_bitwise_run_to_run_and_interval(dev):
    """Run-to-run bitwise reproducibility; checkpoint interval C = T versus sqrt(T) and the
    recomputed versus the forward's snapshots change no bit."""
    w = I.WORKLOADS["gqa_strided_s32"]
    arrays, _ = I.make_all(w)
    _, a = run_case(dev, w, arrays, reuse=True)
    _, b = run_case(dev, w, arrays, reuse=True)
    _, c = run_case(dev, w, arrays, reuse=False, C=w.T)
    _, d = run_case(dev, w, arrays, reuse=False, C=5)
    for n in a:
        assert np.array_equal(a[n], b[n]), ("run-to-run", n)
        assert np.array_equal(a[n], c[n]), ("C=T", n)
        assert np.array_equal(a[n], d[n]), ("C=5", n)


def test_strided_views_equal_contiguous_bitwise(dev):
    w = I.WORKLOADS["gqa_strided_s32"]
    arrays, _ = I.make_all(w)
    _, a = run_case(dev, w, arrays, packed=True, strided_gy=True)
    _, b = run_case(dev, w, arrays, packed=False, strided_gy=False)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


# Head size 128: matrix-core kernels over 16-token blocks; the backward's column pass replays
# each checkpoint segment (C tokens, a multiple of 16) from its snapshot.
S128_CASES = {
    # three segments (64, 64, 22 tokens), ragged second sequence, grouped heads
    "kda_c64": I.Workload("s128_kda_c64", 2, 150, 2, 4, 128, True, 64, -0.3,
                          seq_lens=(150, 77), seed=501),
    # long segments (200 rounded up to 208 tokens: 13 blocks), a ragged last one
    "scalar_c200": I.Workload("s128_scalar_c200", 2, 300, 1, 3, 128, False, 200, -0.05,
                              seq_lens=(300, 133), seed=502),
    # default interval ceil(sqrt(T)) = 10, rounded up to 16: one block per segment
    "kda_default": I.Workload("s128_kda_default", 1, 100, 1, 2, 128, True, 0, -0.5, seed=503),
    # interval 1, rounded up to one block; a partial last block
    "kda_c1": I.Workload("s128_kda_c1", 1, 19, 1, 1, 128, True, 1, -0.5, seed=504),
    # one segment over the whole sequence, its last block a single token
    "scalar_cT": I.Workload("s128_scalar_cT", 1, 129, 1, 1, 128, False, 129, -1.0, seed=505),
    # gates above one whose block products stay in range: column scaling with c > 1
    "kda_gate_above_one": I.Workload("s128_kda_up", 1, 150, 1, 2, 128, True, 64, -0.5,
                                     seed=507, g_hi=0.5),
    "scalar_gate_above_one": I.Workload("s128_scalar_up", 1, 150, 1, 2, 128, False, 64, -1.0,
                                        seed=508, g_hi=1.0),
    # blocks processed token by token, mixed with column-scaled ones: block products below
    # 2^-60 ...
    "kda_tiny_products": I.Workload("s128_kda_tiny", 1, 150, 1, 2, 128, True, 64, -3.8, seed=507),
    "scalar_tiny_products": I.Workload("s128_scalar_tiny", 1, 150, 1, 2, 128, False, 200, -5.5,
                                       seed=508),
}
TOKENWISE = ("kda_tiny_products", "scalar_tiny_products")


def tokenwise_fraction(w, arrays):
    """Share of the 16-token blocks of each (sequence, value head) whose running gate product
    (float32, token order, as the kernels take it) leaves [2^-60, 2^60] in some channel: those
    blocks are processed token by token."""
    a = np.exp(arrays["g"].astype(np.float32)).reshape(w.n_seqs, w.T, w.H_v, w.G)
    hits = tot = 0
    with np.errstate(over="ignore"):
        for s, L in enumerate(w.lens):
            for t0 in range(0, L, 16):
                c = np.cumprod(a[s, t0:min(t0 + 16, L)], axis=0, dtype=np.float32)
                bad = ((c < np.float32(2.0 ** -60)) | (c > np.float32(2.0 ** 60))).any(axis=(0, 2))
                hits += int(bad.sum())
                tot += bad.size
    return hits / tot


@pytest.mark.parametrize("name", list(S128_CASES))
def test_parity_s128(dev, name):
    w = S128_CASES[name]
    log(f"[parity] {w.name} lens={w.lens} C={w.C}")
    arrays, _ = I.make_all(w)
    if name in TOKENWISE:   # the case must mix both kinds of block
        f = tokenwise_fraction(w, arrays)
        log(f"[parity] {w.name}: blocks processed token by token {f:.2f}")
        assert 0.1 < f < 0.9, f
    _, got = run_case(dev, w, arrays, reuse=True)
    rep = check(got, oracle_results(w, arrays))
    log(f"[parity] {w.name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


@pytest.mark.parametrize("kda", [True, False])
def test_parity_s128_products_above_range(dev, kda):
    """Blocks whose running gate product rises past 2^60 and falls back inside the block
    (eight tokens of log-gate +5.5, then eight of -5.5, in every channel of one head) are
    processed token by token, mixed with column-scaled blocks; the values stay finite."""
    w = I.Workload("s128_above_" + ("kda" if kda else "scalar"), 1, 96, 1, 2, 128, kda, 32,
                   -0.3, seed=511)
    arrays, _ = I.make_all(w)
    g = arrays["g"]
    for b in (1, 4):
        g[0, 16 * b:16 * b + 8, 0, :] = 5.5
        g[0, 16 * b + 8:16 * b + 16, 0, :] = -5.5
    f = tokenwise_fraction(w, arrays)
    log(f"[parity] {w.name}: blocks processed token by token {f:.2f}")
    assert 0.1 < f < 0.9, f
    _, got = run_case(dev, w, arrays, reuse=True)
    rep = check(got, oracle_results(w, arrays))
    log(f"[parity] {w.name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


def test_s128_bitwise_interval_reuse_and_strides(dev):
    """S = 128: snapshot reuse, strided views and run-to-run repetition change no bit; the
    checkpoint interval changes no bit outside dg (dg is summed within each checkpoint segment
    from its value at the segment's first token, so other intervals round differently)."""
    w = I.Workload("s128_bits", 2, 140, 2, 4, 128, True, 64, -0.3, seq_lens=(140, 70),
                   packed=True, seed=506)
    arrays, _ = I.make_all(w)
    _, a = run_case(dev, w, arrays, reuse=True)
    _, b = run_case(dev, w, arrays, reuse=True)
    _, c = run_case(dev, w, arrays, reuse=False, C=w.T)
    _, d = run_case(dev, w, arrays, reuse=False, C=16)
    _, e = run_case(dev, w, arrays, reuse=True, C=100, packed=False, strided_gy=True)
    # a gradient buffer 4 bytes off a 16-byte boundary takes the one-column partial sums
    _, f = run_case(dev, w, arrays, reuse=True, grad_offset=1)
    for n in a:
        assert np.array_equal(a[n], b[n]), ("run-to-run", n)
        assert np.array_equal(a[n], f[n]), ("unaligned gradient buffer", n)
        for other, what in ((c, "C=T"), (d, "C=16"), (e, "C=100, contiguous, strided gy")):
            if n == "dg":
                check({n: other[n]}, {n: a[n]}, tol=1e-5)
            else:
                assert np.array_equal(a[n], other[n]), (what, n)



@pytest.mark.parametrize("kind", ["f32", "bf16", "f16"])
def test_s128_rows_off_four_element_boundary(dev, kind):
    """S = 128 with q, k, v, g, beta and gy one element past an allocation's start, so no row
    starts on a four-element boundary: the kernels take their one-element loads (for 16-bit
    inputs: four loads packed before the widening) and every output is bitwise equal to the
    aligned run on the same values."""
    w = I.Workload("s128_offrows", 2, 90, 2, 4, 128, True, 64, -0.3, seq_lens=(90, 37), seed=509)
    arrays, _ = I.make_all(w)
    dt = torch.float32
    if kind != "f32":
        arrays = I.round_inputs(arrays, kind)
        dt = TORCH_HALF[kind]
    log(f"[parity] {w.name} {kind}: inputs one element off")
    _, a = run_case(dev, w, arrays, in_dtype=dt)
    dc = dev(w, arrays, in_dtype=dt)
    for name in ("q", "k", "v", "g", "beta", "gy"):
        t = getattr(dc, name)
        assert t.is_contiguous()
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        off = buf[1:].view(t.shape)
        off.copy_(t)
        assert off.data_ptr() % 8 != 0
        setattr(dc, name, off)
    dc.fwd()
    dc.bwd(reuse=True)
    torch.cuda.synchronize()
    b = dc.results_numpy()
    for n in a:
        assert np.array_equal(a[n], b[n]), n

PIECE_CASES = {
    # two pieces of 1152 tokens, the second sequence ending inside the first
    "two_pieces": I.Workload("s128_pieces", 2, 2200, 1, 2, 128, True, 64, -0.3,
                             seq_lens=(2200, 1000), seed=511),
    # five pieces of 1088 tokens: the chain's results go through the ring of four piece slots
    "ring": I.Workload("s128_ring", 2, 5200, 1, 2, 128, False, 64, -0.2,
                       seq_lens=(5200, 3000), seed=512),
}


@pytest.mark.parametrize("name", list(PIECE_CASES))
def test_s128_pipelined_pieces(dev, name):
    """S = 128 over several pieces of the token axis: gdn_fwd and gdn_bwd pipeline the pieces,
    the chain's on the caller's stream and their column sums on a second one; two row slabs
    per unit.  Against the oracle, and bitwise against the single-stream allocation-free
    backward (one piece when the chain's results fit a buffer for every token, else the same
    pieces in turn on one stream)."""
    from gated_delta_rule_bwd_amd import binding as B
    w = PIECE_CASES[name]
    log(f"[parity] {w.name} lens={w.lens}")
    arrays, _ = I.make_all(w)
    dc, got = run_case(dev, w, arrays, reuse=True)
    rep = check(got, oracle_results(w, arrays), REGIONS_FWD + REGIONS_BWD)
    log(f"[parity] {w.name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))
    assert B.workspace_size(dc.p) <= B.NOALLOC_SCRATCH_BYTES
    dc.grad.fill_(float("nan"))
    B.bwd_noalloc(dc.p, dc.q, dc.k, dc.v, dc.g, dc.beta, dc.state0, dc.gy, dc.dstate_out, dc.grad)
    torch.cuda.synchronize()
    one = {k: v.detach().cpu().numpy() for k, v in dc.grads().items()}
    for n in REGIONS_BWD:
        assert np.array_equal(one[n], got[n]), ("pieces vs one piece", n)
