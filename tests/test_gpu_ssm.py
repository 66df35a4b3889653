"""The selective-scan kernels (through the C ABI) against the fp64 oracle, on the GPU."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_cases import log  # noqa: E402
from compare import slice_rel  # noqa: E402

TOL = 2e-4   # max |gpu - oracle| / max |oracle| per output region (fp32 recurrences vs fp64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd import binding  # loads libgdn.so
    return binding


# the (sequence, head) axes of each region: x, y, dx, dt, ddt [n][T][H][..], B, C, dB, dC
# [n][T][G][N], states [n][H][P][N]
AXES = {"y": (0, 2), "dx": (0, 2), "ddt": (0, 2), "dB": (0, 2), "dC": (0, 2),
        "s_out": (0, 1), "ds": (0, 1)}


def _rel(x, r, name="y"):
    """Worst error over the (sequence, head) slices of a region."""
    return slice_rel(x, r, AXES[name])


def run(B, arr, softplus=True, with_gs=True, flags=1, recompute_too=False):
    """Forward and backward on the GPU; returns (y, s_out, grads dict[, grads recomputed])."""
    g = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in arr.items()}
    p = B.ssm_problem_from(g["x"], g["B"], g["A"], softplus)
    ws = torch.empty(max(B.ssm_workspace_size(p), 16) // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(g["x"])
    s_out = torch.empty_like(g["s0"])
    B.ssm_fwd(p, g["s0"], g["x"], g["dt"], g["A"], g["B"], g["C"], y, s_out, ws)
    total, lay = B.ssm_grad_layout(p)
    gp = torch.full((max(total, 1),), float("nan"), device="cuda")
    gs = g["gs"] if with_gs else None
    B.ssm_bwd(p, g["s0"], g["x"], g["dt"], g["A"], g["B"], g["C"], g["gy"], gs, gp, ws, flags=flags)
    torch.cuda.synchronize()
    grads = {k: gp[o:o + int(np.prod(shp))].view(shp).cpu().numpy() for k, (o, shp) in lay.items()}
    out = [y.cpu().numpy(), s_out.cpu().numpy(), grads]
    if recompute_too:
        gp2 = torch.full_like(gp, float("nan"))
        ws.fill_(float("nan"))   # nothing of the forward's workspace may be read
        B.ssm_bwd(p, g["s0"], g["x"], g["dt"], g["A"], g["B"], g["C"], g["gy"], gs, gp2, ws, flags=0)
        torch.cuda.synchronize()
        out.append({k: gp2[o:o + int(np.prod(shp))].view(shp).cpu().numpy() for k, (o, shp) in lay.items()})
    return out


def oracle(arr, softplus=True, with_gs=True):
    from oracle import ssm_scan as S
    a = arr
    y, sT = S.ssm_fwd(a["s0"], a["x"], a["dt"], a["A"], a["B"], a["C"], softplus)
    ds, dx, ddt, dB, dC = S.ssm_bwd(a["s0"], a["x"], a["dt"], a["A"], a["B"], a["C"], a["gy"],
                                    a["gs"] if with_gs else None, softplus)
    return y, sT, {"ds": ds, "dx": dx, "ddt": ddt, "dB": dB, "dC": dC}


CASES = [
    # n, T, H, P, N, G, a_per_state, softplus, with_gs
    (2, 37, 4, 16, 32, 2, False, True, True),     # Mamba-2 branch, two heads per group, ragged window
    (2, 45, 32, 1, 16, 2, True, True, True),      # Mamba-1 branch, 16 channels per group
    (1, 20, 2, 64, 128, 1, False, True, True),    # the widest state (the chunked backward)
    (1, 20, 2, 32, 128, 1, False, True, True),    # the widest state, head size 32: per token
    (1, 17, 2, 64, 128, 1, True, True, True),     # the widest state with per-state decay: per token
    (2, 24, 4, 8, 64, 1, False, False, False),    # raw steps, no final-state cotangent
    (1, 9, 16, 1, 64, 1, True, True, True),       # per-state decay over 64 states
    (2, 8, 4, 16, 32, 4, False, True, True),      # exactly one window; one head per group
    (1, 1, 2, 16, 16, 1, False, True, True),      # one token
    (2, 0, 4, 16, 32, 2, False, True, True),      # no tokens: d_s0 is the cotangent itself
    # head size 64 with 128 states and one decay per head: the backward in 32-token chunks
    (2, 100, 4, 64, 128, 2, False, True, True),   # two groups of two heads, ragged last chunk
    (1, 64, 3, 64, 128, 1, False, False, False),  # raw steps, no final-state cotangent, 2 chunks
    (1, 40, 40, 64, 128, 1, False, True, True),   # 16 head slices of 3 heads, two of them empty
    (1, 1, 2, 64, 128, 2, False, True, True),     # one token
    (2, 0, 2, 64, 128, 1, False, True, True),     # no tokens
    # 16 states with a multiple of 128 rows per group: the backward in two passes, two lanes per row
    (2, 45, 256, 1, 16, 1, True, True, True),     # Mamba-1 channels, ragged last window
    (1, 30, 256, 1, 16, 2, True, True, True),     # 128 channels per group, two groups
    (1, 20, 64, 8, 16, 2, True, False, False),    # head size 8 (ddt sums 8 rows), two groups
    (2, 8, 128, 4, 16, 1, False, True, True),     # one decay per head, two row blocks
    (1, 1, 256, 1, 16, 1, True, True, True),      # one token
    (1, 0, 256, 1, 16, 1, True, True, True),      # no tokens
]


def _arrays(n, T, H, P, N, G, aps, softplus, seed):
    from gated_delta_rule_bwd_amd import inputs as I
    arr = I.make_ssm(dict(n_seqs=n, T=T, H=H, P=P, N=N, G=G, a_per_state=aps), seed=seed)
    if not softplus:
        arr["dt"] = np.abs(arr["dt"]) * 0.02     # raw positive steps in [0.04, 0.12]
    return arr


@pytest.mark.parametrize("n,T,H,P,N,G,aps,softplus,with_gs", CASES)
def test_ssm_parity(dev, n, T, H, P, N, G, aps, softplus, with_gs):
    arr = _arrays(n, T, H, P, N, G, aps, softplus, 1500 + T + H + N)
    y, sT, grads, grads2 = run(dev, arr, softplus, with_gs, recompute_too=True)
    ry, rsT, rg = oracle(arr, softplus, with_gs)
    errs = {"y": _rel(y, ry, "y"), "s_out": _rel(sT, rsT, "s_out")}
    errs.update({k: _rel(grads[k], rg[k], k) for k in rg})
    log(f"[ssm] n={n} T={T} H={H} P={P} N={N} G={G} aps={aps} softplus={softplus}: "
        + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs
    for k in grads:      # recomputed window states give the forward's bits
        assert np.array_equal(grads[k], grads2[k]), k
    if T == 0:
        assert np.array_equal(grads["ds"], arr["gs"] if with_gs else np.zeros_like(arr["gs"]))


def test_ssm_chunked_unaligned_rows(dev):
    """x and gy one float past a 16-byte boundary (the API asks 4-byte alignment of them): the
    chunked backward reads their rows with scalar loads and gives the aligned run's bits."""
    arr = _arrays(1, 70, 2, 64, 128, 1, False, True, 1700)
    y, sT, ga = run(dev, arr)
    g = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in arr.items()}
    for k in ("x", "gy"):
        buf = torch.empty(g[k].numel() + 1, device="cuda")
        buf[1:] = g[k].reshape(-1)
        g[k] = buf[1:].view(g[k].shape)
        assert g[k].data_ptr() % 16 == 4
    p = dev.ssm_problem_from(g["x"], g["B"], g["A"], True)
    ws = torch.empty(max(dev.ssm_workspace_size(p), 16) // 4, dtype=torch.float32, device="cuda")
    y2, s2 = torch.empty(g["x"].shape, device="cuda"), torch.empty_like(g["s0"])
    dev.ssm_fwd(p, g["s0"], g["x"], g["dt"], g["A"], g["B"], g["C"], y2, s2, ws)
    total, lay = dev.ssm_grad_layout(p)
    gp = torch.full((total,), float("nan"), device="cuda")
    dev.ssm_bwd(p, g["s0"], g["x"], g["dt"], g["A"], g["B"], g["C"], g["gy"], g["gs"], gp, ws, flags=1)
    torch.cuda.synchronize()
    for k, (o, shp) in lay.items():
        assert np.array_equal(gp[o:o + int(np.prod(shp))].view(shp).cpu().numpy(), ga[k]), k


def test_ssm_deterministic(dev):
    arr = _arrays(2, 50, 8, 16, 64, 2, False, True, 1600)
    a = run(dev, arr)
    b = run(dev, arr)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for k in a[2]:
        assert np.array_equal(a[2][k], b[2][k]), k


@pytest.mark.parametrize("name", ["ssm2_layer_h80_p64_n128", "ssm1_layer_d5120_n16"])
def test_ssm_layer_sampled(dev, name):
    """Full layer size in the benchmark's launch configuration.  Two sampled heads of sequence
    0 are checked against the oracle run on those heads alone (y, s_out, d_s0, dx, ddt do not
    depend on the other heads); dB and dC, which fold every head of a group, are checked at
    every token through identities of the backward that hold at any size:
    sum_n dB[t, g, n] B[t, g, n] = sum over the group's heads and rows of x dx, and
    sum_n dC[t, g, n] C[t, g, n] = sum over them of gy y."""
    from gated_delta_rule_bwd_amd import inputs as I
    cfg = I.SSM_WORKLOADS[name]
    arr = I.make_ssm(cfg)
    y, sT, gr = run(dev, arr)
    H = cfg["H"]
    for h in (0, H - 1):
        sub = {"s0": arr["s0"][:1, h:h + 1], "x": arr["x"][:1, :, h:h + 1], "dt": arr["dt"][:1, :, h:h + 1],
               "A": arr["A"][h:h + 1], "B": arr["B"][:1], "C": arr["C"][:1],
               "gy": arr["gy"][:1, :, h:h + 1], "gs": arr["gs"][:1, h:h + 1]}
        ry, rsT, rg = oracle(sub)
        errs = {"y": _rel(y[:1, :, h:h + 1], ry, "y"), "s_out": _rel(sT[:1, h:h + 1], rsT, "s_out"),
                "ds": _rel(gr["ds"][:1, h:h + 1], rg["ds"], "ds"),
                "dx": _rel(gr["dx"][:1, :, h:h + 1], rg["dx"], "dx"),
                "ddt": _rel(gr["ddt"][:1, :, h:h + 1], rg["ddt"], "ddt")}
        log(f"[ssm] {name} head {h}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
        assert all(v <= TOL for v in errs.values()), errs
    f64 = np.float64
    lhs_b = np.einsum("ntgk,ntgk->ntg", gr["dB"].astype(f64), arr["B"].astype(f64))
    rhs_b = np.einsum("nthp,nthp->nt", arr["x"].astype(f64), gr["dx"].astype(f64))[..., None]
    lhs_c = np.einsum("ntgk,ntgk->ntg", gr["dC"].astype(f64), arr["C"].astype(f64))
    rhs_c = np.einsum("nthp,nthp->nt", arr["gy"].astype(f64), y.astype(f64))[..., None]
    eb, ec = slice_rel(lhs_b, rhs_b, (0, 2)), slice_rel(lhs_c, rhs_c, (0, 2))
    log(f"[ssm] {name} fold identities: dB.B {eb:.1e}, dC.C {ec:.1e}")
    assert eb <= TOL and ec <= TOL


@pytest.mark.parametrize("name", ["ssm2_layer_h80_p64_n128", "ssm1_layer_d5120_n16"])
def test_ssm_layer_tail_elementwise(dev, name):
    """Full layer size in the benchmark's launch configuration, every head: dB and dC (which fold
    every head of the group), dx and ddt of the last 512 tokens of sequence 0, elementwise per
    slice.  The oracle takes the state before those tokens from its own forward over the
    sequence, then runs forward and backward over the tail from it with the final-state
    cotangent: the tail's gradients depend on nothing else."""
    from gated_delta_rule_bwd_amd import inputs as I
    from oracle import ssm_scan as S
    cfg = I.SSM_WORKLOADS[name]
    arr = I.make_ssm(cfg)
    y, sT, gr = run(dev, arr)
    T, K = cfg["T"], 512
    t0 = T - K
    head = {k: arr[k][:1] for k in ("s0", "x", "dt", "B", "C")}
    _, s_mid = S.ssm_fwd(head["s0"], head["x"][:, :t0], head["dt"][:, :t0], arr["A"],
                         head["B"][:, :t0], head["C"][:, :t0])
    tail = lambda v: v[:1, t0:]
    _, dx, ddt, dB, dC = S.ssm_bwd(s_mid, tail(arr["x"]), tail(arr["dt"]), arr["A"], tail(arr["B"]),
                                   tail(arr["C"]), tail(arr["gy"]), arr["gs"][:1])
    errs = {"dx": _rel(gr["dx"][:1, t0:], dx, "dx"), "ddt": _rel(gr["ddt"][:1, t0:], ddt, "ddt"),
            "dB": _rel(gr["dB"][:1, t0:], dB, "dB"), "dC": _rel(gr["dC"][:1, t0:], dC, "dC")}
    log(f"[ssm] {name} last {K} tokens of sequence 0, every head: "
        + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs


@pytest.mark.parametrize("name", ["ssm2_layer_h80_p64_n128", "ssm1_layer_d5120_n16"])
def test_ssm_layer_heads_elementwise(dev, name):
    """The layer's head and state shape (all heads, so dB and dC fold every head of the group)
    over 256 tokens of one sequence: every output, dB and dC included, elementwise per
    (sequence, head) slice against the oracle."""
    from gated_delta_rule_bwd_amd import inputs as I
    cfg = dict(I.SSM_WORKLOADS[name])
    cfg["n_seqs"], cfg["T"] = 1, 256
    arr = I.make_ssm(cfg)
    y, sT, gr = run(dev, arr)
    ry, rsT, rg = oracle(arr)
    errs = {"y": _rel(y, ry, "y"), "s_out": _rel(sT, rsT, "s_out")}
    errs.update({k: _rel(gr[k], rg[k], k) for k in rg})
    log(f"[ssm] {name} heads x 256 tokens: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs
